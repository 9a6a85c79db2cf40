// bf16 MFMA GEMMs of the latent path: the joint KV down-projection (7168 -> 576) and the KV
// up-projection (512 -> 128 heads x 256), both "x times W^T" with W stored [out, in]
// ("DeepSeek-V3.2-Exp · Key-value down-projection": formula c = x W_DKV and the Linear excerpt;
// "DeepSeek-V3.2-Exp · Keys": MHA-prefill excerpt, wkv_b followed by the per-head view).
//
// Both operands are K-contiguous, so both feed the 32x32x16 MFMA directly from LDS rows.
// The kernel computes D^T = W . X^T per 32x32 block: lane l then owns token (l % 32) and four
// consecutive output features per group of four accumulators, which become one 8-byte store.
// fp32 accumulation, one rounding to bf16 in the epilogue.
//
// Tiling: a 256-thread workgroup (4 waves, WM x WN) owns BM tokens x BN features; K advances in
// steps of 64 through one LDS stage, the next stage prefetched into registers meanwhile.
#include "mla_device.hpp"
#include "mla_launch.hpp"

namespace mla {

enum { kModeDown = 0, kModeUp = 1 };

constexpr int kBK = 64;
constexpr int kLdsPad = 8;              // bf16 elements of padding per LDS row
constexpr int kLdsRow = kBK + kLdsPad;  // 72 elements = 144 bytes

template <int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__(256) void gemm_nt_kernel(const uint16_t* __restrict__ X,
                                                      const uint16_t* __restrict__ W, int M, int K,
                                                      int T, int mtiles, int ntiles,
                                                      uint16_t* __restrict__ out) {
    static_assert(WM * WN == 4, "four waves");
    constexpr int WTM = BM / WM, WTN = BN / WN;     // wave tile (tokens, features)
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int CH_X = BM * kBK / 8, CH_W = BN * kBK / 8;   // 16-byte chunks per stage
    static_assert(CH_X % 256 == 0 && CH_W % 256 == 0, "whole chunks per thread");
    constexpr int NX = CH_X / 256, NW = CH_W / 256;

    __shared__ __attribute__((aligned(16))) uint16_t Xs[BM * kLdsRow];
    __shared__ __attribute__((aligned(16))) uint16_t Ws[BN * kLdsRow];

    // Tile selection.
    int mt, nt;
    const int wg = blockIdx.x;
    if (MODE == kModeDown) {
        // The N tiles of one M tile land on the same XCD (workgroups are dealt to the 8 XCDs
        // round-robin), so the shared X tile is read once per XCD L2.
        const int xcd = wg & 7, j = wg >> 3;
        nt = j % ntiles;
        mt = xcd + 8 * (j / ntiles);
    } else {
        // Consecutive workgroups sweep the token tiles of one head; XCD x then sees token tiles
        // x, x+8, ... for every head, so its X tiles stay L2-resident across heads.
        nt = wg / mtiles;
        mt = wg % mtiles;
    }
    if (mt >= mtiles || nt >= ntiles) return;
    const int m0 = mt * BM, n0 = nt * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;

    // Global addresses of this thread's chunks (rows past M are clamped; their results are
    // never stored).
    const uint16_t* xsrc[NX];
    const uint16_t* wsrc[NW];
    int xdst[NX], wdst[NW];
#pragma unroll
    for (int i = 0; i < NX; ++i) {
        const int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
        const int m = min(m0 + row, M - 1);
        xsrc[i] = X + (size_t)m * K + col;
        xdst[i] = row * kLdsRow + col;
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
        wsrc[i] = W + (size_t)(n0 + row) * K + col;
        wdst[i] = row * kLdsRow + col;
    }

    u32x4 xr[NX], wr[NW];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < NX; ++i) xr[i] = load16(xsrc[i] + k0);
#pragma unroll
        for (int i = 0; i < NW; ++i) wr[i] = load16(wsrc[i] + k0);
    };
    auto lstore = [&]() {
#pragma unroll
        for (int i = 0; i < NX; ++i) *reinterpret_cast<u32x4*>(&Xs[xdst[i]]) = xr[i];
#pragma unroll
        for (int i = 0; i < NW; ++i) *reinterpret_cast<u32x4*>(&Ws[wdst[i]]) = wr[i];
    };

    f32x16 acc[FN][FM];
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
        for (int b = 0; b < FM; ++b) acc[a][b] = f32x16{};

    // LDS read offsets of the MFMA operands: row (l % 32) of each 32-row block, eight
    // reduction elements chosen by (l / 32).
    const int frag_row = lane & 31, frag_k = (lane >> 5) * 8;
    const int xoff = (wm * WTM + frag_row) * kLdsRow + frag_k;
    const int woff = (wn * WTN + frag_row) * kLdsRow + frag_k;

    const int nk = K / kBK;
    gload(0);
    lstore();
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) gload((kt + 1) * kBK);
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 16) {
            bf16x8 bx[FM], aw[FN];
#pragma unroll
            for (int b = 0; b < FM; ++b)
                bx[b] = as_bf16x8(*reinterpret_cast<const u32x4*>(&Xs[xoff + b * 32 * kLdsRow + kk]));
#pragma unroll
            for (int a = 0; a < FN; ++a)
                aw[a] = as_bf16x8(*reinterpret_cast<const u32x4*>(&Ws[woff + a * 32 * kLdsRow + kk]));
#pragma unroll
            for (int a = 0; a < FN; ++a)
#pragma unroll
                for (int b = 0; b < FM; ++b) acc[a][b] = mfma32x32x16(aw[a], bx[b], acc[a][b]);
        }
        __syncthreads();
        if (kt + 1 < nk) {
            lstore();
            __syncthreads();
        }
    }

    // Epilogue: lane owns token (l % 32) of each block and features 8*g + 4*(l/32) + 0..3.
#pragma unroll
    for (int b = 0; b < FM; ++b) {
        const int m = m0 + wm * WTM + b * 32 + (lane & 31);
        if (m >= M) continue;
        uint16_t* dst_row;
        if (MODE == kModeDown) {
            dst_row = out + (size_t)m * kKvAOut;
        } else {
            const int bb = m / T, t = m - bb * T;
            dst_row = out + (((size_t)bb * kHeads + nt) * T + t) * 256;   // BN == 256: one head
        }
#pragma unroll
        for (int a = 0; a < FN; ++a) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = (MODE == kModeDown ? n0 : 0) + wn * WTN + a * 32 + 8 * g + 4 * (lane >> 5);
                u32x2 v;
                v[0] = pack_bf16(acc[a][b][4 * g + 0], acc[a][b][4 * g + 1]);
                v[1] = pack_bf16(acc[a][b][4 * g + 2], acc[a][b][4 * g + 3]);
                store8(dst_row + n, v);
            }
        }
    }
}

hipError_t launch_gemm_kv_down(const uint16_t* x, const uint16_t* w_dkv, int M, uint16_t* kv_raw,
                               hipStream_t stream) {
    constexpr int BM = 128, BN = 192;
    const int mtiles = (M + BM - 1) / BM, ntiles = kKvAOut / BN;
    const int groups = (mtiles + 7) / 8;
    const dim3 grid(groups * 8 * ntiles);
    gemm_nt_kernel<BM, BN, 2, 2, kModeDown><<<grid, 256, 0, stream>>>(x, w_dkv, M, kHidden, 0, mtiles,
                                                                      ntiles, kv_raw);
    return hipGetLastError();
}

hipError_t launch_gemm_kv_up(const uint16_t* c_kv, const uint16_t* w_ukv, int B, int T, uint16_t* kv,
                             hipStream_t stream) {
    constexpr int BM = 128, BN = 256;
    const int M = B * T;
    const int mtiles = (M + BM - 1) / BM, ntiles = kHeads;
    const dim3 grid(mtiles * ntiles);
    gemm_nt_kernel<BM, BN, 2, 2, kModeUp><<<grid, 256, 0, stream>>>(c_kv, w_ukv, M, kLora, T, mtiles,
                                                                    ntiles, kv);
    return hipGetLastError();
}

}  // namespace mla
