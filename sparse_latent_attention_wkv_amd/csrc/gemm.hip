// bf16 MFMA GEMMs of the latent path: the joint KV down-projection (7168 -> 576) and the KV
// up-projection (512 -> 128 heads x 256), both "x times W^T" with W stored [out, in]
// ("DeepSeek-V3.2-Exp · Key-value down-projection": formula c = x W_DKV and the Linear excerpt;
// "DeepSeek-V3.2-Exp · Keys": MHA-prefill excerpt, wkv_b followed by the per-head view).
//
// Both operands are K-contiguous, so both feed the 32x32x16 MFMA directly from LDS rows.
// The kernels compute D^T = W . X^T per 32x32 block: lane l then owns token (l % 32) and four
// consecutive output features per group of four accumulators. fp32 accumulation, one rounding
// to bf16 in the epilogue. Both stream K through an LDS ring filled by direct global->LDS loads
// (no staging registers) and stage the bf16 tile in LDS so global stores write whole row
// segments.
#include "mla_device.hpp"
#include "mla_launch.hpp"

namespace mla {

// ------------------------------------------------------------------------------------------------
// Down-projection GEMM: 128 tokens x 192 features per workgroup of four waves (2 x 2, each wave
// 64 x 96: six 32x32 accumulator blocks). K = 7168 streams in chunks of BK through a STAGES-deep
// LDS ring filled by direct global->LDS loads. LDS rows are BK*2 bytes; 16-byte chunk c of row r
// sits at c ^ key(r), key(r) = (r / (256 / rowbytes)) % (rowbytes / 16), so the 16 lanes of an
// operand read (16 rows, one logical chunk) hit 16 distinct 16-byte bank groups. Within a chunk
// the operands of k-step s + 1 are read before the MFMAs of step s, and the next chunk's first
// operands before the last step's MFMAs, so LDS latency hides behind MFMAs. The one barrier per
// chunk sits before the last step: it makes the next chunk visible and frees the current stage,
// which is refilled with the chunk STAGES ahead. The epilogue stages the whole bf16 tile in the
// idle ring and stores 384-byte row segments. Chunks of 64 (128 contiguous bytes of each x row,
// rows 14 KB apart) rather than 32: with x arriving from HBM rather than the last-level cache,
// 64-byte pieces made the kernel about a third slower.
// ------------------------------------------------------------------------------------------------
#ifndef DOWN_BK
#define DOWN_BK 64
#endif
#ifndef DOWN_STAGES
#define DOWN_STAGES 3
#endif
namespace down {
constexpr int BM = 128, BN = 192, BK = DOWN_BK, STAGES = DOWN_STAGES;
constexpr int ROWB = BK * 2;                 // bytes per LDS row
constexpr int CPR = ROWB / 16;               // 16-byte chunks per row
constexpr int RPL = 64 / CPR;                // rows per 1 KB load
constexpr int RPG = 256 / ROWB;              // rows per 256-byte bank sweep
constexpr int XB = BM * ROWB;                // X rows per stage
constexpr int SB = XB + BN * ROWB;           // bytes per stage
constexpr int XL = 32 / RPL, WL = 48 / RPL;  // 1 KB loads per wave per chunk (X rows 32w.., W rows 48w..)
constexpr int LOADS = XL + WL;
constexpr int KS = BK / 16;                  // MFMA k-steps per chunk
constexpr int GM = 4;                        // M tiles per group in the grouped tile order
static_assert(STAGES >= 2 && KS >= 2, "ring shape");
static_assert(STAGES * SB <= 160 * 1024 && STAGES * SB >= BM * 384, "LDS budget");
__device__ __forceinline__ int key(int r) { return (r / RPG) % CPR; }
}

// KD = K (row length of X and W), ND = N (row length of the output, a multiple of 192).
template <int KD, int ND>
__global__ __launch_bounds__(256) void gemm_down_kernel(const uint16_t* __restrict__ X,
                                                        const uint16_t* __restrict__ W, int M,
                                                        int mtiles, uint16_t* __restrict__ out) {
    using namespace down;
    constexpr int NK = KD / BK;
    constexpr int NTILES = ND / BN;
    static_assert(KD % BK == 0 && ND % BN == 0 && NK > STAGES + 1, "GEMM shape");
    __shared__ __attribute__((aligned(16))) uint8_t ring[STAGES * SB];

    // Workgroups are dealt to the 8 XCDs round-robin; XCD x takes the M tiles mt = x (mod 8).
    // Few N tiles (the key-value projection's 3): all N tiles of one M tile run on the same XCD,
    // so the shared X rows are fetched once per XCD L2. Many N tiles: groups of GM M tiles, N
    // tile by N tile, so the ~32 workgroups resident on an XCD share GM X tiles and about 8 W
    // tiles in its L2 instead of streaming every W tile once per M tile.
    const int wg = blockIdx.x, xcd = wg & 7, j = wg >> 3;
    int nt, mt;
    if constexpr (NTILES <= 4) {
        nt = j % NTILES;
        mt = (j / NTILES) * 8 + xcd;
    } else {
        const int g = j / (GM * NTILES), idx = j - g * (GM * NTILES);
        nt = idx / GM;
        mt = (g * GM + idx % GM) * 8 + xcd;
    }
    if (mt >= mtiles) return;
    const int m0 = mt * BM, n0 = nt * BN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;

    // DMA: a 1 KB load covers RPL LDS rows; lane i writes row (i / CPR), physical chunk
    // (i % CPR), which holds logical chunk (i % CPR) ^ key(row). X rows past M are clamped to
    // M - 1 (never stored).
    const int pc = lane % CPR;
    uint32_t x_voff[XL], w_voff[WL];
#pragma unroll
    for (int jj = 0; jj < XL; ++jj) {
        const int r = 32 * wave + RPL * jj + lane / CPR;
        x_voff[jj] = (uint32_t)((min(m0 + r, M - 1) - m0) * (KD * 2) + ((pc ^ key(r)) << 4));
    }
#pragma unroll
    for (int jj = 0; jj < WL; ++jj) {
        const int r = 48 * wave + RPL * jj + lane / CPR;
        w_voff[jj] = (uint32_t)(r * (KD * 2) + ((pc ^ key(r)) << 4));
    }
    const uint16_t* xg = X + (size_t)m0 * KD;
    const uint16_t* wgp = W + (size_t)n0 * KD;
    auto issue = [&](int kc, uint8_t* st) {
#pragma unroll
        for (int jj = 0; jj < XL; ++jj) dma16(xg + kc * BK, x_voff[jj], st + (32 * wave + RPL * jj) * ROWB);
#pragma unroll
        for (int jj = 0; jj < WL; ++jj) dma16(wgp + kc * BK, w_voff[jj], st + XB + (48 * wave + RPL * jj) * ROWB);
    };

    // Operand reads: row (l % 32) of a 32-row block, logical chunk 2s + l/32; block row bases
    // are multiples of 32, so the swizzle key is that of (l % 32) alone.
    const int fr = lane & 31, fh = lane >> 5, fk = key(fr);
    const int xrow = (wm * 64 + fr) * ROWB, wrow = XB + (wn * 96 + fr) * ROWB;
    struct Ops { bf16x8 x[2], w[3]; };
    auto read_ops = [&](const uint8_t* st, int s, Ops& o) {
        const int c = ((2 * s + fh) ^ fk) << 4;
#pragma unroll
        for (int b = 0; b < 2; ++b) o.x[b] = as_bf16x8(*reinterpret_cast<const u32x4*>(st + xrow + c + b * 32 * ROWB));
#pragma unroll
        for (int a = 0; a < 3; ++a) o.w[a] = as_bf16x8(*reinterpret_cast<const u32x4*>(st + wrow + c + a * 32 * ROWB));
    };
    f32x16 acc[3][2];
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};
    auto mma = [&](const Ops& o) {
#pragma unroll
        for (int a = 0; a < 3; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) acc[a][b] = mfma32x32x16(o.w[a], o.x[b], acc[a][b]);
    };
    // vmcnt wait leaving `newer` chunks of this wave's loads in flight.
    auto wait_newer = [](int newer) {
        switch (newer) {
            case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
            case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS * 1)); break;
            case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS * 2)); break;
            case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS * 3)); break;
            default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS * 4)); break;
        }
    };
    static_assert(STAGES - 1 <= 5 && LOADS * (STAGES - 1) < 64, "vmcnt range");

    // Prologue: all stages in flight; chunk 0 landed.
#pragma unroll
    for (int c = 0; c < STAGES; ++c) issue(c, ring + c * SB);
    switch (STAGES - 1) {
        case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS * 1)); break;
        case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS * 2)); break;
        case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS * 3)); break;
        case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS * 4)); break;
        default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS * 5)); break;
    }
    barrier_keep_loads();
    Ops o[2];
    read_ops(ring, 0, o[0]);

    int rs = 0;   // stage of chunk kc
    // One chunk: `newer` = chunks issued after kc + 1 that may stay in flight at the barrier;
    // `refill` issues chunk kc + STAGES into the freed stage; `next` reads chunk kc + 1.
    auto chunk = [&](int kc, int newer, bool refill, bool next) {
        uint8_t* cur = ring + rs * SB;
        const int ns = rs == STAGES - 1 ? 0 : rs + 1;
#pragma unroll
        for (int s = 0; s + 1 < KS; ++s) {
            read_ops(cur, s + 1, o[(s + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);   // these reads go out before the MFMAs
            mma(o[s & 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_newer(newer);
        barrier_keep_loads();
        if (refill) issue(kc + STAGES, cur);
        if (next) read_ops(ring + ns * SB, 0, o[0]);
        __builtin_amdgcn_sched_barrier(0);
        mma(o[(KS - 1) & 1]);
        rs = ns;
    };
    static_assert(((KS - 1) & 1) == 1, "the next chunk's first operands go to o[0]");
    int kc = 0;
    for (; kc < NK - STAGES; ++kc) chunk(kc, STAGES - 2, true, true);
    // Tail: the last STAGES chunks, nothing left to issue.
#pragma unroll
    for (int t = 0; t < STAGES; ++t) chunk(kc + t, max(0, STAGES - 2 - t), false, t < STAGES - 1);

    // Epilogue. Every ring read was completed before the last barrier and no load is in flight,
    // so the ring is free. Tile row r (token) occupies 384 bytes; 16-byte chunk c (features
    // 8c..8c+7) sits at c ^ (r & 7). Lane owns token (l % 32) of each block and features
    // 8g + 4(l/32) + 0..3.
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int row = wm * 64 + b * 32 + fr;
#pragma unroll
        for (int a = 0; a < 3; ++a)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 v;
                v[0] = pack_bf16(acc[a][b][4 * g + 0], acc[a][b][4 * g + 1]);
                v[1] = pack_bf16(acc[a][b][4 * g + 2], acc[a][b][4 * g + 3]);
                const int c = 12 * wn + 4 * a + g;
                *reinterpret_cast<u32x2*>(ring + row * 384 + ((c ^ (row & 7)) << 4) + fh * 8) = v;
            }
    }
    __syncthreads();
    constexpr int NC = BM * 24 / 256;   // 16-byte pieces per thread
    u32x4 v[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int idx = i * 256 + tid, row = idx / 24, c = idx - row * 24;
        v[i] = *reinterpret_cast<const u32x4*>(ring + row * 384 + ((c ^ (row & 7)) << 4));
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int idx = i * 256 + tid, row = idx / 24, c = idx - row * 24;
        if (m0 + row < M) store16(out + (size_t)(m0 + row) * ND + n0 + c * 8, v[i]);
    }
}

namespace {
template <int KD, int ND>
hipError_t launch_gemm_down_form(const uint16_t* x, const uint16_t* w, int M, uint16_t* out,
                                 hipStream_t stream) {
    constexpr int NTILES = ND / down::BN;
    const int mtiles = (M + down::BM - 1) / down::BM;
    const int per_xcd = (mtiles + 7) / 8;               // M tiles of each XCD
    const int slots = NTILES <= 4 ? per_xcd : ((per_xcd + down::GM - 1) / down::GM) * down::GM;
    const dim3 grid(slots * 8 * NTILES);
    gemm_down_kernel<KD, ND><<<grid, 256, 0, stream>>>(x, w, M, mtiles, out);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_kv_down(const uint16_t* x, const uint16_t* w_dkv, int M, uint16_t* kv_raw,
                               hipStream_t stream) {
    return launch_gemm_down_form<kHidden, kKvAOut>(x, w_dkv, M, kv_raw, stream);
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
