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



// ------------------------------------------------------------------------------------------------
// Up-projection GEMM, second form: BM tokens x 256 features (one head) per workgroup of BM/32
// waves (BM/64 along tokens x 2 along features), each wave 64 x 128. K streams in chunks of 32
// through a three-stage LDS ring filled by direct global->LDS loads issued two chunks ahead: no
// staging registers. LDS rows are 64 bytes (32 bf16); 16-byte chunk c of row r is stored at
// c ^ ((r >> 2) & 3), which keeps the 16-lane operand reads conflict free. The epilogue stages
// each wave's bf16 blocks in LDS so every global store writes whole 256-byte half rows.
// BM = 128 (four waves, 72 KB: two workgroups share a CU) or 256 (eight waves, 96 KB: operands
// reused over twice the tokens).
// ------------------------------------------------------------------------------------------------
#ifndef UP_BM
#define UP_BM 256
#endif
namespace up2 {
#ifndef UP_STAGES
#define UP_STAGES 3
#endif
constexpr int BN = 256, BK = 32, STAGES = UP_STAGES;
constexpr int ROWB = BK * 2;                                 // 64 bytes per LDS row
constexpr int WB = BN * ROWB;                                // 16 KB of W rows per stage
}

__device__ __forceinline__ void dma16_g(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// Workgroup barrier without the release fence of __syncthreads(), whose wait would drain every
// outstanding global->LDS load and so the prefetch ring. This thread's LDS reads are completed
// first, so no later load into a stage can overtake a read of it; the global->LDS loads that
// must have landed are waited for explicitly with vmcnt before the barrier.
__device__ __forceinline__ void barrier_keep_loads() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int BM>
__global__ __launch_bounds__(BM * 2) void gemm_up_kernel(const uint16_t* __restrict__ X,
                                                         const uint16_t* __restrict__ W, int M, int T,
                                                         int mtiles, uint16_t* __restrict__ out) {
    using namespace up2;
    constexpr int NW = BM / 32;                  // waves
    constexpr int XB = BM * ROWB;                // X rows per stage
    constexpr int WLOADS = 16 / NW;              // 1 KB W loads per wave per chunk
    constexpr int LOADS = 2 + WLOADS;            // loads per wave per chunk (2 of X)
    __shared__ __attribute__((aligned(16))) uint8_t xs0[XB], xs1[XB], xs2[XB], xs3[STAGES > 3 ? XB : 16];
    __shared__ __attribute__((aligned(16))) uint8_t ws0[WB], ws1[WB], ws2[WB], ws3[STAGES > 3 ? WB : 16];
    uint8_t* const xs[4] = {xs0, xs1, xs2, xs3};
    uint8_t* const ws[4] = {ws0, ws1, ws2, ws3};

    // Consecutive workgroups sweep the token tiles of one head; XCD x (workgroups are dealt
    // round-robin) then holds token tiles x, x+8, ... for every head in its L2.
    const int h = blockIdx.x / mtiles, mt = blockIdx.x % mtiles;
    const int m0 = mt * BM;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % (BM / 64), wn = wave / (BM / 64);

    // DMA: a stage is BM/16 one-KB loads of X rows and 16 of W rows; wave w loads X rows
    // 32w..32w+31 and W rows (16 WLOADS) w.., so every wave has the same count in flight. A 1 KB
    // load covers 16 rows of 64 bytes; lane i writes row (i >> 2), physical chunk (i & 3), so it
    // fetches logical chunk (i & 3) ^ ((row >> 2) & 3).
    int x_src[2], w_src[WLOADS];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int xr = 32 * wave + 16 * j + (lane >> 2);
        x_src[j] = (min(m0 + xr, M - 1) - m0) * kLora + (((lane & 3) ^ ((xr >> 2) & 3)) * 8);
    }
#pragma unroll
    for (int j = 0; j < WLOADS; ++j) {
        const int wr = 16 * WLOADS * wave + 16 * j + (lane >> 2);
        w_src[j] = wr * kLora + (((lane & 3) ^ ((wr >> 2) & 3)) * 8);
    }
    const uint16_t* xbase = X + (size_t)m0 * kLora;
    const uint16_t* wbase = W + (size_t)h * BN * kLora;
    auto issue = [&](int kc, uint8_t* xdst, uint8_t* wdst) {
#pragma unroll
        for (int j = 0; j < 2; ++j) dma16_g(xbase + kc * BK + x_src[j], xdst + (32 * wave + 16 * j) * ROWB);
#pragma unroll
        for (int j = 0; j < WLOADS; ++j)
            dma16_g(wbase + kc * BK + w_src[j], wdst + (16 * WLOADS * wave + 16 * j) * ROWB);
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

    // MFMA operand reads: row (l % 32) of a 32-row block, 16-byte chunk (2s + l/32), swizzled.
    const int fr = lane & 31, fh = lane >> 5;
    int x_off[2][2], w_off[4][2];   // [block][k-step of 16]
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int row = wm * 64 + b * 32 + fr;
            x_off[b][s] = row * ROWB + (((2 * s + fh) ^ ((row >> 2) & 3)) << 4);
        }
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int row = wn * 128 + a * 32 + fr;
            w_off[a][s] = row * ROWB + (((2 * s + fh) ^ ((row >> 2) & 3)) << 4);
        }
    }

    // Chunks are issued STAGES-1 ahead; the end of chunk kc waits for chunk kc+1 and leaves
    // the newer ones in flight.
    constexpr int NK = kLora / BK;   // 16 chunks
#pragma unroll
    for (int c = 0; c < STAGES - 1; ++c) issue(c, xs[c], ws[c]);
    __builtin_amdgcn_s_waitcnt(0x3F70 | (LOADS * (STAGES - 2)));   // chunk 0 landed
    barrier_keep_loads();
#pragma unroll
    for (int kc = 0; kc < NK; ++kc) {
        const int st = kc % STAGES;
        if (kc + STAGES - 1 < NK) issue(kc + STAGES - 1, xs[(kc + STAGES - 1) % STAGES], ws[(kc + STAGES - 1) % STAGES]);
        __builtin_amdgcn_sched_barrier(0);       // keep the loads at the top of the chunk
        const uint8_t* xb = xs[st];
        const uint8_t* wb = ws[st];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bf16x8 bx[2], aw[4];
#pragma unroll
            for (int b = 0; b < 2; ++b) bx[b] = as_bf16x8(*reinterpret_cast<const u32x4*>(xb + x_off[b][s]));
#pragma unroll
            for (int a = 0; a < 4; ++a) aw[a] = as_bf16x8(*reinterpret_cast<const u32x4*>(wb + w_off[a][s]));
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) acc[a][b] = mfma32x32x16(aw[a], bx[b], acc[a][b]);
        }
        // chunk kc+1 must have landed; the chunks issued after it may stay in flight
        {
            const int newer = min(NK - 1, kc + STAGES - 1) - (kc + 1);
            if (newer >= 2)
                __builtin_amdgcn_s_waitcnt(0x3F70 | (LOADS * 2));
            else if (newer == 1)
                __builtin_amdgcn_s_waitcnt(0x3F70 | LOADS);
            else
                __builtin_amdgcn_s_waitcnt(0x3F70);
        }
        barrier_keep_loads();
    }

    // Epilogue: each wave stages one 32-token x 128-feature block at a time in its own 8 KB of
    // the (now idle) ring, rows of 256 bytes with 16-byte chunk c at c ^ (row & 15), then
    // writes it back as whole 256-byte half rows of kv (16 bytes per lane, 4 rows per store).
    // The barrier ending the K loop (after vmcnt(0)) guarantees that no wave still reads the
    // ring and no load into it is in flight.
    uint8_t* ot;
    if (BM == 128) {
        ot = (wave < 2 ? ws0 : ws1) + (wave & 1) * 8192;
    } else {
        const int sl = wave >> 1;                           // 16 KB arrays: two waves each
        ot = (sl == 0 ? xs0 : sl == 1 ? xs1 : sl == 2 ? xs2 : ws0) + (wave & 1) * 8192;
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 v;
                v[0] = pack_bf16(acc[a][b][4 * g + 0], acc[a][b][4 * g + 1]);
                v[1] = pack_bf16(acc[a][b][4 * g + 2], acc[a][b][4 * g + 3]);
                const int chunk = (4 * a + g) ^ (fr & 15);
                *reinterpret_cast<u32x2*>(ot + fr * 256 + chunk * 16 + fh * 8) = v;
            }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int row = 4 * j + (lane >> 4), c = lane & 15;
            const u32x4 v = *reinterpret_cast<const u32x4*>(ot + row * 256 + ((c ^ (row & 15)) << 4));
            const int m = m0 + wm * 64 + b * 32 + row;
            if (m < M) {
                const int bb = m / T, t = m - bb * T;
                store16(out + (((size_t)bb * kHeads + h) * T + t) * 256 + wn * 128 + c * 8, v);
            }
        }
    }
}

hipError_t launch_gemm_kv_up(const uint16_t* c_kv, const uint16_t* w_ukv, int B, int T, uint16_t* kv,
                             hipStream_t stream) {
    constexpr int BM = UP_BM;
    const int M = B * T;
    const int mtiles = (M + BM - 1) / BM;
    gemm_up_kernel<BM><<<mtiles * kHeads, BM * 2, 0, stream>>>(c_kv, w_ukv, M, T, mtiles, kv);
    return hipGetLastError();
}

}  // namespace mla
