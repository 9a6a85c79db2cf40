// Large-tile bf16 GEMM for the query path, D[M][ND] = X[M][KD] . W[ND][KD]^T with fp32
// accumulation and one bf16 rounding ("DeepSeek-V3.2-Exp · Key-value down-projection": the MLA
// constructor excerpt's wq_a (7168 -> q_lora_rank) and wq_b (q_lora_rank -> 128 x 192), both
// Linear layers that hold their weight [out, in]).
//
// One workgroup of four waves computes 256 tokens x BN features (BN = 192 or 256); wave (wm, wn)
// owns 128 tokens x BN/2 features, 4 x BN/64 blocks of 32x32 accumulated by
// v_mfma_f32_32x32x16_bf16 in the D^T = W . X^T form (lane l owns token l % 32 of a block and
// four consecutive features per group of four accumulators; at one wave per SIMD the compiler
// keeps the 192 or 256 accumulator registers in the accumulation file). Per 16-deep k-step a
// wave reads 4 + BN/64 operand fragments for 4 * BN/64 MFMAs: about 40% fewer LDS bytes per MFMA
// than a 64 x 96 wave tile, which with the ring fills took more than the LDS port delivers.
//
// K streams in chunks of BK (64) through STAGES (2) LDS stages of 256 + BN rows filled by direct
// global->LDS loads; 16-byte chunk c of row r sits at c ^ ((r / RPG) % CPR) (RPG rows per 256-byte
// bank sweep, CPR chunks per row), so the 16 lanes of an operand read hit distinct bank groups. Within a chunk the operands of k-step s + 1 are read
// before the MFMAs of step s; the one barrier per chunk sits before the last step, after which
// the freed stage is refilled with the chunk STAGES ahead. The
// epilogue stages the bf16 tile in the idle ring and writes 16-byte pieces of whole rows; its
// barriers wait for LDS work only, so the stores drain under the next tile's first loads. ROPE:
// features 128..191 of each 192-wide query head are rotated there, after the bf16 rounding of the
// product, at position start_pos + (row % T) (the query path's rotary step); the tile's (cos, sin)
// table rows are loaded into the ring before any store is issued and the tile is staged in two
// halves, so no wait in the store loop covers the stores already issued.
//
// Tile order: tile slot w goes to XCD w mod 8 (workgroups are dealt to the 8 XCDs round-robin,
// and a persistent workgroup keeps its XCD, stepping through slots by the grid size, a multiple
// of 8); XCD x takes the M tiles mt = x (mod 8), in groups of four M tiles walked N tile by N
// tile, so the workgroups resident on one XCD share four X tiles and a few W tiles in its L2.
// With fewer than 8 M tiles that order would leave XCDs idle; the tiles then go in plain order.
// At most one workgroup per compute unit (256) is launched; each runs its tiles one after
// another (2% faster than one workgroup per tile at 8192 tokens: no relaunch between tiles).
#include "mla_device.hpp"
#include "mla_launch.hpp"

namespace mla {

namespace big {
constexpr int BM = 256;
constexpr int GM = 4;                        // M tiles per group
}  // namespace big

template <int KD, int ND, int BN, int BK, int STAGES, bool ROPE>
__global__ __launch_bounds__(256) void gemm_big_kernel(const uint16_t* __restrict__ X,
                                                       const uint16_t* __restrict__ W, int M,
                                                       int mtiles, uint16_t* __restrict__ out,
                                                       const float* __restrict__ rope_cs, int T,
                                                       int start_pos, int nslots) {
    using namespace big;
    constexpr int ROWB = BK * 2;                 // bytes per LDS row
    constexpr int CPR = ROWB / 16;               // 16-byte chunks per row
    constexpr int RPL = 64 / CPR;                // rows per 1 KB load
    constexpr int RPG = 256 / ROWB;              // rows per 256-byte bank sweep
    constexpr int KS = BK / 16;                  // MFMA k-steps per chunk
    auto key = [](int r) { return (r / RPG) % CPR; };
    constexpr int NA = BN / 64;                  // 32-feature blocks per wave
    constexpr int XB = BM * ROWB, SB = XB + BN * ROWB;
    constexpr int XL = (BM / 4) / RPL, WL = (BN / 4) / RPL;   // 1 KB loads per wave per chunk
    constexpr int LOADS = XL + WL;
    constexpr int NK = KD / BK, NTILES = ND / BN;
    constexpr int PR = BN / 8;                   // 16-byte pieces per output row
    static_assert(KD % BK == 0 && ND % BN == 0 && NK >= STAGES && KS % 2 == 0, "GEMM shape");
    static_assert(STAGES * SB <= 160 * 1024 && STAGES * SB >= BM * BN * 2, "LDS budget");
    static_assert(LOADS * (STAGES - 1) < 64 && (BN / 4) % RPL == 0, "load split");
    static_assert(!ROPE || BN % 8 == 0, "rotary pieces");
    __shared__ __attribute__((aligned(16))) uint8_t ring[STAGES * SB];

    for (int wg = blockIdx.x; wg < nslots; wg += gridDim.x) {
    int nt, mt;
    if (mtiles >= 8) {
        const int xcd = wg & 7, j = wg >> 3;
        const int g = j / (GM * NTILES), idx = j - g * (GM * NTILES);
        nt = idx / GM;
        mt = (g * GM + idx % GM) * 8 + xcd;
        if (mt >= mtiles) continue;
    } else {   // fewer M tiles than XCDs: plain order, so every XCD gets tiles
        mt = wg % mtiles;
        nt = wg / mtiles;
    }
    const int m0 = mt * BM, n0 = nt * BN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;

    // DMA: a 1 KB load covers RPL rows; lane i writes row i / CPR, physical chunk i % CPR, which
    // holds logical chunk (i % CPR) ^ key(row). X rows past M repeat row M - 1 (never stored).
    const int pc = lane % CPR;
    uint32_t x_voff[XL], w_voff[WL];
#pragma unroll
    for (int jj = 0; jj < XL; ++jj) {
        const int r = (BM / 4) * wave + RPL * jj + lane / CPR;
        x_voff[jj] = (uint32_t)((min(m0 + r, M - 1) - m0) * (KD * 2) + ((pc ^ key(r)) << 4));
    }
#pragma unroll
    for (int jj = 0; jj < WL; ++jj) {
        const int r = (BN / 4) * wave + RPL * jj + lane / CPR;
        w_voff[jj] = (uint32_t)(r * (KD * 2) + ((pc ^ key(r)) << 4));
    }
    const uint16_t* xg = X + (size_t)m0 * KD;
    const uint16_t* wgp = W + (size_t)n0 * KD;
    const uint32_t ring_lds = lds_addr(ring);   // 32-bit LDS address: no per-load conversion
    auto issue = [&](int kc, int stage) {
        const uint32_t st = ring_lds + stage * SB;
#pragma unroll
        for (int jj = 0; jj < XL; ++jj)
            dma16_lds(xg + kc * BK, x_voff[jj], st + ((BM / 4) * wave + RPL * jj) * ROWB);
#pragma unroll
        for (int jj = 0; jj < WL; ++jj)
            dma16_lds(wgp + kc * BK, w_voff[jj], st + XB + ((BN / 4) * wave + RPL * jj) * ROWB);
    };

    // Operand reads: row l % 32 of a 32-row block, logical chunk 2s + l / 32; block row bases
    // are multiples of 32, so the swizzle key is that of l % 32 alone.
    const int fr = lane & 31, fh = lane >> 5, fk = key(fr);
    const int xrow = (wm * 128 + fr) * ROWB, wrow = XB + (wn * (BN / 2) + fr) * ROWB;
    struct Ops { bf16x8 x[4], w[NA]; };
    auto read_ops = [&](const uint8_t* st, int s, Ops& o) {
        const int c = ((2 * s + fh) ^ fk) << 4;
#pragma unroll
        for (int b = 0; b < 4; ++b)
            o.x[b] = as_bf16x8(*reinterpret_cast<const u32x4*>(st + xrow + c + b * 32 * ROWB));
#pragma unroll
        for (int a = 0; a < NA; ++a)
            o.w[a] = as_bf16x8(*reinterpret_cast<const u32x4*>(st + wrow + c + a * 32 * ROWB));
    };
    f32x16 acc[NA][4];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};
    auto mma = [&](const Ops& o) {
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] = mfma32x32x16(o.w[a], o.x[b], acc[a][b]);
    };

    // vmcnt wait leaving `newer` chunks of this wave's loads in flight.
    auto wait_newer = [](int newer) {
        switch (newer) {
            case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
            case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS * 1)); break;
            case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS * 2)); break;
            default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS * 3)); break;
        }
    };
    static_assert(STAGES <= 4, "vmcnt cases");

    // Prologue: every stage in flight, chunk 0 landed.
#pragma unroll
    for (int c = 0; c < STAGES; ++c) issue(c, c);
    wait_newer(STAGES - 1);
    barrier_keep_loads();
    Ops o[2];
    read_ops(ring, 0, o[0]);

    int rs = 0;   // stage of chunk kc
    // One chunk; at its barrier chunk kc + 1 must have landed, `newer` later chunks may still be
    // in flight.
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
        if (refill) issue(kc + STAGES, rs);
        if (next) read_ops(ring + ns * SB, 0, o[0]);
        __builtin_amdgcn_sched_barrier(0);
        mma(o[(KS - 1) & 1]);
        rs = ns;
    };
    int kc = 0;
    for (; kc < NK - STAGES; ++kc) chunk(kc, STAGES - 2, true, true);
#pragma unroll
    for (int t = 0; t < STAGES; ++t) chunk(kc + t, max(0, STAGES - 2 - t), false, t < STAGES - 1);

    // Epilogue: every ring read completed before the last barrier and no load is in flight.
    // Tile row r (token) takes BN * 2 bytes; piece c (features 8c..8c+7) sits at c ^ (r & 7).
    auto stage_rows = [&](int rbase) {   // this wave's rows, at rows - rbase of the ring
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int row = wm * 128 + b * 32 + fr - rbase;
#pragma unroll
            for (int a = 0; a < NA; ++a)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    u32x2 v;
                    v[0] = pack_bf16(acc[a][b][4 * q + 0], acc[a][b][4 * q + 1]);
                    v[1] = pack_bf16(acc[a][b][4 * q + 2], acc[a][b][4 * q + 3]);
                    const int c = wn * (BN / 16) + 4 * a + q;
                    *reinterpret_cast<u32x2*>(ring + row * (BN * 2) + ((c ^ (row & 7)) << 4) + fh * 8) = v;
                }
        }
    };
    if constexpr (ROPE) {
        // The (cos, sin) rows of the tile's 256 positions go to the upper half of the ring before
        // any store is issued; the tile is then staged and stored in two halves of 128 rows, so the
        // store loop reads only LDS and waits for no memory operation (vector memory waits count
        // stores too). Thread t stores piece column c = t % PR of rows r0 + 8 i of each half.
        constexpr int HB = (BM / 2) * (BN * 2);
        static_assert(PR == 32 && HB + BM * 256 <= STAGES * SB, "half staging plus table rows");
        {
            const int step4 = 4 % T;
            int qr = (m0 + wave * 64 + (lane >> 4)) % T;
#pragma unroll
            for (int k = 0; k < 16; ++k) {   // 64 rows per wave, 4 rows of 256 bytes per load
                dma16_lds(rope_cs, (uint32_t)(start_pos + qr) * 256u + (uint32_t)(lane & 15) * 16u,
                          ring_lds + HB + (uint32_t)(wave * 64 + 4 * k) * 256u);
                qr += step4;
                if (qr >= T) qr -= T;
            }
        }
        const int c = tid % PR, r0 = tid / PR;
        const int f = (n0 + 8 * c) % kQkHead;          // feature of this column within its head
        const bool rot = f >= kNope;
        const int jb = rot ? (f - kNope) / 2 : 0;      // first rotary pair of the piece
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (wm == h) stage_rows(h * 128);
            if (h == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // the table rows (no store of this tile is in flight yet)
            barrier_keep_loads();
#pragma unroll 4
            for (int i = 0; i < 16; ++i) {
                const int lr = r0 + 8 * i, row = h * 128 + lr;
                u32x4 v = *reinterpret_cast<const u32x4*>(ring + lr * (BN * 2) + ((c ^ (lr & 7)) << 4));
                if (rot) {
                    const f32x4* cs = reinterpret_cast<const f32x4*>(ring + HB + row * 256 + jb * 8);
                    const f32x4 cs0 = cs[0], cs1 = cs[1];
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const float re = bf16lo(v[p]), im = bf16hi(v[p]);
                        const float cq = p < 2 ? cs0[2 * p] : cs1[2 * p - 4];
                        const float sq = p < 2 ? cs0[2 * p + 1] : cs1[2 * p - 3];
                        v[p] = pack_bf16(re * cq - im * sq, re * sq + im * cq);
                    }
                }
                if (m0 + row < M) store16(out + (size_t)(m0 + row) * ND + n0 + c * 8, v);
            }
            // the staged rows are read before the next half is staged or the next tile's loads
            // land; the stores drain meanwhile
            barrier_keep_loads();
        }
    } else {
        stage_rows(0);
        barrier_keep_loads();
        constexpr int NC = BM * PR / 256;   // pieces per thread
#pragma unroll 4
        for (int i = 0; i < NC; ++i) {
            const int id = i * 256 + tid, row = id / PR, c = id - row * PR;
            const u32x4 v = *reinterpret_cast<const u32x4*>(ring + row * (BN * 2) + ((c ^ (row & 7)) << 4));
            if (m0 + row < M) store16(out + (size_t)(m0 + row) * ND + n0 + c * 8, v);
        }
        // the staging reads are done before the next tile's loads land; the stores drain
        barrier_keep_loads();
    }
    }
}

// 64-deep chunks in two stages: measured against 32-deep chunks in four stages (three chunks of
// lookahead, twice the barriers), which were slower for both shapes (743 vs 797 us, 202 vs
// 210 us at 8192 tokens).
constexpr int GQ_BK = 64, GQ_ST = 2;

namespace {
template <int KD, int ND, int BN, int BK, int STAGES, bool ROPE>
hipError_t launch_big(const uint16_t* x, const uint16_t* w, int M, uint16_t* out,
                      const float* rope_cs, int T, int start_pos, hipStream_t stream) {
    constexpr int NTILES = ND / BN;
    const int mtiles = (M + big::BM - 1) / big::BM;
    const int per_xcd = (mtiles + 7) / 8;
    const int slots = ((per_xcd + big::GM - 1) / big::GM) * big::GM;
    const int blocks = mtiles >= 8 ? slots * 8 * NTILES : mtiles * NTILES;
    const int grid = blocks < 256 ? blocks : 256;   // a multiple of 8 when it is 256
    gemm_big_kernel<KD, ND, BN, BK, STAGES, ROPE><<<dim3(grid), 256, 0, stream>>>(
        x, w, M, mtiles, out, rope_cs, T, start_pos, blocks);
    return hipGetLastError();
}
}  // namespace

// wq_a: 7168 -> 1536 in 256 x 192 tiles (8 N tiles: 256 workgroups at 8192 tokens).
hipError_t launch_gemm_q_a(const uint16_t* x, const uint16_t* w_qa, int M, uint16_t* qa,
                           hipStream_t stream) {
    return launch_big<kHidden, kQRank, 192, GQ_BK, GQ_ST, false>(x, w_qa, M, qa, nullptr, 1, 0, stream);
}

// wq_b: 1536 -> 128 x 192 in 256 x 256 tiles, rotary part of every head rotated in the epilogue.
hipError_t launch_gemm_q_b_rope(const uint16_t* qr, const uint16_t* w_qb, int M, uint16_t* q,
                                const float* rope_cs, int T, int start_pos, hipStream_t stream) {
    return launch_big<kQRank, kHeads * kQkHead, 256, GQ_BK, GQ_ST, true>(qr, w_qb, M, q, rope_cs, T,
                                                                           start_pos, stream);
}

}  // namespace mla
