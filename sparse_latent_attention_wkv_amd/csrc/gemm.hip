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
// Up-projection GEMM: one head's 256 features x 256 tokens per workgroup of eight waves (4 along
// tokens x 2 along features), each wave 64 x 128: eight 32x32 accumulators. K = 512 streams in
// 8 chunks of 64 through a two-stage LDS ring (256 X rows and 256 W rows of 128 bytes, 64 KB per
// stage) filled by direct global->LDS loads one chunk ahead; every row
// piece a load fetches is one whole 128-byte line (32-deep chunks fetched half lines, each line
// twice, and ran 4% slower). 16-byte chunk c of row r sits at c ^ ((r >> 1) & 7), so the 16 lanes
// of an operand read hit 16 distinct bank groups. The epilogue stages each wave's 32 x 128 bf16
// blocks in the 8 KB of stage 1 that its own loads fill, and writes whole 256-byte half rows of
// kv[b][h][t]. Persistent: one workgroup per compute unit steps through its tiles; chunk 0 of its
// next tile loads into stage 0 during the last chunk and the epilogue, and each wave loads its
// part of chunk 1 as soon as it has stored its own rows, so the tile change costs no load latency
// and the stores drain under the next tile's MFMAs.
// ------------------------------------------------------------------------------------------------
namespace up {
constexpr int BM = 256, BN = 256, BK = 64, ROWB = BK * 2;
constexpr int XB = BM * ROWB, SB = XB + BN * ROWB;   // 64 KB per stage
constexpr int NK = kLora / BK, LOADS = 8;            // chunks; 1 KB loads per wave per chunk
__device__ __forceinline__ int key(int r) { return (r >> 1) & 7; }
}

__global__ __launch_bounds__(512) void gemm_up_kernel(const uint16_t* __restrict__ X,
                                                      const uint16_t* __restrict__ W, int M, int T,
                                                      int mtiles, uint16_t* __restrict__ out) {
    using namespace up;
    __shared__ __attribute__((aligned(16))) uint8_t ring[2 * SB];
    const int ntot = mtiles * kHeads;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % 4, wn = wave / 4;

    // DMA: a 1 KB load covers 8 rows of 128 bytes; lane i writes row i / 8, physical chunk i % 8,
    // i.e. logical chunk (i % 8) ^ key(row). Wave w loads X rows 32w..32w+31 and W rows
    // 32w..32w+31 (four loads each). X rows past M repeat row M - 1 (never stored).
    const int pc = lane & 7;
    uint32_t w_voff[4], x_voff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 32 * wave + 8 * j + (lane >> 3);
        w_voff[j] = (uint32_t)(r * (kLora * 2) + ((pc ^ key(r)) << 4));
    }
    // Tile id: head id / mtiles, token tile id % mtiles. Workgroup w (on XCD w % 8; the grid G is
    // a multiple of 8) takes ids w, w + G, ...: with mtiles a multiple of 8, XCD x only ever sees
    // the token tiles mt = x (mod 8), which stay in its L2 while the heads go by.
    int h = 0, m0 = 0;
    const uint16_t* xg = X;
    const uint16_t* wg = W;
    auto set_tile = [&](int id) {
        h = id / mtiles;
        m0 = (id - h * mtiles) * BM;
        xg = X + (size_t)m0 * kLora;
        wg = W + (size_t)h * BN * kLora;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 32 * wave + 8 * j + (lane >> 3);
            x_voff[j] = (uint32_t)((min(m0 + r, M - 1) - m0) * (kLora * 2) + ((pc ^ key(r)) << 4));
        }
    };
    const uint32_t ring_l = lds_addr(ring);
    auto issue = [&](int kc, int stage) {
        const uint32_t st = ring_l + stage * SB;
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16_lds(xg + kc * BK, x_voff[j], st + (32 * wave + 8 * j) * ROWB);
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16_lds(wg + kc * BK, w_voff[j], st + XB + (32 * wave + 8 * j) * ROWB);
    };

    // MFMA operand reads: row (l % 32) of a 32-row block, logical chunk 2s + l/32 of k-step s;
    // block row bases are multiples of 32, so the swizzle key is that of l % 32 alone.
    const int fr = lane & 31, fh = lane >> 5, fk = key(fr);
    const int xrow = (wm * 64 + fr) * ROWB, wrow = XB + (wn * 128 + fr) * ROWB;
    // kv row of token m = b T + t is (b * 128 + h) * T + t: one sequence further is (128 T - T)
    // rows further than the next position
    const size_t seq_jump = (size_t)(kHeads - 1) * T * 256;

    int id = blockIdx.x;
    set_tile(id);
    issue(0, 0);
    issue(1, 1);
    for (;;) {
        const int cur_m0 = m0, cur_h = h;
        const int next = id + (int)gridDim.x;
        const bool more = next < ntot;
        f32x16 acc[4][2];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};
        // chunk 0 has landed: at most eight of this wave's memory operations remain in flight,
        // and as its loads complete in issue order and the eight of chunk 1 were issued after
        // those of chunk 0, none of chunk 0's can be among them
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS));
        barrier_keep_loads();
#pragma unroll
        for (int kc = 0; kc < NK; ++kc) {
            const uint8_t* st = ring + (kc & 1) * SB;
#pragma unroll
            for (int s = 0; s < BK / 16; ++s) {
                const int c = ((2 * s + fh) ^ fk) << 4;
                bf16x8 bx[2], aw[4];
#pragma unroll
                for (int b = 0; b < 2; ++b) bx[b] = as_bf16x8(*reinterpret_cast<const u32x4*>(st + xrow + c + b * 32 * ROWB));
#pragma unroll
                for (int a = 0; a < 4; ++a) aw[a] = as_bf16x8(*reinterpret_cast<const u32x4*>(st + wrow + c + a * 32 * ROWB));
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int b = 0; b < 2; ++b) acc[a][b] = mfma32x32x16(aw[a], bx[b], acc[a][b]);
            }
            if (kc + 1 < NK) {
                // chunk kc + 1 (the only one of this tile in flight) has landed and every wave is
                // done with this stage, which then takes chunk kc + 2, or after the next-to-last
                // chunk, chunk 0 of the workgroup's next tile
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                barrier_keep_loads();
                if (kc + 2 < NK) {
                    issue(kc + 2, kc & 1);
                } else if (more) {
                    set_tile(next);
                    issue(0, 0);
                }
            } else {
                barrier_keep_loads();   // every wave is done with stage 1
            }
        }
        // Epilogue: wave w stages one 32-token x 128-feature block at a time in the stage-1 bytes
        // its own loads fill (rows 0-15 at 4096 w, rows 16-31 at XB + 4096 w), rows of 256 bytes
        // with 16-byte chunk c at c ^ (row & 15), then
        // writes it as whole 256-byte half rows of kv (16 bytes per lane, 4 rows per store). The
        // block's first token is split into (sequence, position) once; each later row is 256
        // elements further, plus one sequence jump per sequence end inside the block.
        uint8_t* ot = ring + SB + wave * 4096;   // rows 0-15; rows 16-31 at XB further
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
                    *reinterpret_cast<u32x2*>(ot + (fr & 15) * 256 + (fr >> 4) * XB + chunk * 16 + fh * 8) = v;
                }
            const int mb = cur_m0 + wm * 64 + b * 32;      // the block's first token (wave-uniform)
            const int b0 = mb / T, t0 = mb - b0 * T;
            const int c = lane & 15;
            uint16_t* const dst0 = out + (((size_t)b0 * kHeads + cur_h) * T + t0) * 256 + wn * 128 + c * 8;
            u32x4 v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int row = 4 * j + (lane >> 4);
                v[j] = *reinterpret_cast<const u32x4*>(ot + (row & 15) * 256 + (row >> 4) * XB + ((c ^ (row & 15)) << 4));
            }
            if (mb + 32 <= M && t0 + 32 <= T) {   // every row of the block is stored, one sequence
#pragma unroll
                for (int j = 0; j < 8; ++j) store16(dst0 + (size_t)(4 * j + (lane >> 4)) * 256, v[j]);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int row = 4 * j + (lane >> 4);
                    if (mb + row < M)
                        store16(dst0 + (size_t)row * 256 + (size_t)((t0 + row) / T) * seq_jump, v[j]);
                }
            }
        }
        if (!more) break;
        // the wave's staged rows are exactly the stage-1 rows its own loads fill
        issue(1, 1);
        id = next;
    }
}

hipError_t launch_gemm_kv_up(const uint16_t* c_kv, const uint16_t* w_ukv, int B, int T, uint16_t* kv,
                             hipStream_t stream) {
    const int M = B * T;
    const int mtiles = (M + up::BM - 1) / up::BM;
    const int ntot = mtiles * kHeads;                   // a multiple of 8
    // one workgroup per compute unit (its LDS admits one), a multiple of 8
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n >= 8) cus = n;
    }
    const int G = min(ntot, cus / 8 * 8);
    gemm_up_kernel<<<G, 512, 0, stream>>>(c_kv, w_ukv, M, T, mtiles, kv);
    return hipGetLastError();
}

}  // namespace mla
