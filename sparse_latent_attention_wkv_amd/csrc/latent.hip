// Latent-space ("absorbed") sparse prefill attention for long sequences.
//
// "DeepSeek-V3.2-Exp · Keys", MHA-prefill code excerpt: every head's non-rotary key and value
// are linear images of the normalised latent row c_t (k_nope[h,t] = W_UK[h] c_t,
// v[h,t] = W_UV[h] c_t, the two halves of wkv_b per head), the rotary key is shared, scores are
// q.k times the softmax scale over the selection intersected with the causal mask, and the
// softmax weights mix the values. Regrouped around the latent (associativity of the products;
// the pages do not show this form):
//   q_nope[h] . (W_UK[h] c_t) = (W_UK[h]^T q_nope[h]) . c_t
//   sum_t p_t W_UV[h] c_t     = W_UV[h] (sum_t p_t c_t)
// so every head scores the same 576-wide rows [c_t | k_pe_t], and only the selected rows are
// gathered: no key outside the selection is scored, and no per-head keys or values are formed.
// It costs 2*576 + 2*512 FLOP per selected (query, head, key) instead of 2*192 + 2*128, which
// pays once the query tiles of the head-major path would score several times the selected
// keys (long sequences with a fixed top-k).
//
// Kernels (one call, in order):
//  * sel_list:   the selection intersected with the causal mask as a sorted list of distinct key
//                positions per query (built through a bitmap row in LDS, as the index mask has
//                set semantics), padded with key 0 to a multiple of 64, plus the count.
//  * wuk_t:      W_UK[h] transposed to [h][512][128] so the next GEMM reads both operands along K.
//  * gemm_heads: q_lat[m][h] = bf16(W_UK[h]^T q_nope[m][h])          (K = 128, N = 512 per head)
//  * attn_latent: per query all 128 heads over the gathered latent rows; o_lat[h][m] = bf16(O/l)
//  * gemm_heads: out[m][h] = bf16(W_UV[h] o_lat[h][m])                 (K = 512, N = 128 per head)
#include <math.h>

#include <type_traits>

#include "mla_device.hpp"
#include "mla_launch.hpp"

namespace mla {

typedef short s16x4_l __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 lds16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ s16x4_l lds_tr8(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_l*)(p));
}
__device__ __forceinline__ float lane_pair_max(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float lane_pair_sum(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ------------------------------------------------------------------------------------------------
// Selection lists.
// ------------------------------------------------------------------------------------------------
int latent_list_stride(int T, int K) { return (min(T, K) + 63) / 64 * 64; }

// QR = 4 query rows per workgroup (one per wave): the wave sets its rows' allowed keys as bits in LDS
// (the same set semantics as the dense mask), then turns each bitmap row into the ascending list
// 2048 keys at a time: lane l counts the keys of word l of the batch, a wave-wide prefix count
// places them in the wave's LDS buffer, and the batch leaves as consecutive 4-byte stores. Rows
// s_lo..T-1 of each sequence; row s of sequence b is output row b*(T - s_lo) + s - s_lo.
template <int QR>
__global__ __launch_bounds__(256) void sel_list_kernel(const int32_t* __restrict__ topk, int T, int K, int s_lo,
                                                       int Lp, bool vec4, int32_t* __restrict__ lists,
                                                       int32_t* __restrict__ counts) {
    static_assert(QR == 4, "one row per wave");
    extern __shared__ uint32_t bits_lds[];
    const int Wd = (T + 31) / 32, WP = Wd + 1;
    uint32_t* const stage_all = bits_lds + QR * WP;   // 4 waves x 2048 entries
    const int Tr = T - s_lo;
    const int s0 = s_lo + blockIdx.x * QR, b = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t* const stage = stage_all + wave * 2048;
    {
        const int qi = wave, s = s0 + qi;
        if (s >= T) return;
        uint32_t* row = bits_lds + qi * WP;
        const int nw = (s >> 5) + 1;             // words that can hold keys <= s
        for (int w = lane; w < nw; w += 64) row[w] = 0u;
        // the row's entries; only this wave touches the row, and LDS operations of a wave
        // complete in order, so the clears land before the first bit is set
        __builtin_amdgcn_wave_barrier();
        const int32_t* src = topk + ((size_t)b * T + s) * K;
        if (vec4) {
            for (int i = lane; i < K / 4; i += 64) {
                const int4 v = reinterpret_cast<const int4*>(src)[i];
                if ((unsigned)v.x <= (unsigned)s) atomicOr(row + (v.x >> 5), 1u << (v.x & 31));
                if ((unsigned)v.y <= (unsigned)s) atomicOr(row + (v.y >> 5), 1u << (v.y & 31));
                if ((unsigned)v.z <= (unsigned)s) atomicOr(row + (v.z >> 5), 1u << (v.z & 31));
                if ((unsigned)v.w <= (unsigned)s) atomicOr(row + (v.w >> 5), 1u << (v.w & 31));
            }
        } else {
            for (int i = lane; i < K; i += 64) {
                const int t = src[i];
                if ((unsigned)t <= (unsigned)s) atomicOr(row + (t >> 5), 1u << (t & 31));
            }
        }
        __builtin_amdgcn_wave_barrier();
        const size_t orow = (size_t)b * Tr + (s - s_lo);
        int32_t* dst = lists + orow * Lp;
        int total = 0;
        for (int c = 0; c < nw; c += 64) {
            const int w = c + lane;
            uint32_t word = w < nw ? row[w] : 0u;
            const int pc = __popc(word);
            int incl = pc;                       // inclusive prefix over the wave
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int t = __shfl_up(incl, off, 64);
                if (lane >= off) incl += t;
            }
            int pos = incl - pc;
            while (word) {
                stage[pos++] = (uint32_t)((w << 5) + (__ffs(word) - 1));
                word &= word - 1;
            }
            const int n = __shfl(incl, 63, 64);
            __builtin_amdgcn_wave_barrier();
            for (int p = lane; p < n; p += 64) dst[total + p] = (int32_t)stage[p];
            __builtin_amdgcn_wave_barrier();
            total += n;
        }
        const int padded = (total + 63) & ~63;
        for (int p = total + lane; p < padded; p += 64) dst[p] = 0;
        if (lane == 0) counts[orow] = total;
    }
}

static hipError_t launch_sel_list_range(const int32_t* topk, int B, int T, int K, int s_lo, int32_t* lists,
                                        int32_t* counts, hipStream_t stream) {
    constexpr int QR = 4;
    const dim3 grid((T - s_lo + QR - 1) / QR, B);
    const size_t lds = ((size_t)QR * ((T + 31) / 32 + 1) + 4 * 2048) * sizeof(uint32_t);
    const bool vec4 = (K & 3) == 0 && ((uintptr_t)topk & 15) == 0;
    sel_list_kernel<QR><<<grid, 256, lds, stream>>>(topk, T, K, s_lo, latent_list_stride(T, K), vec4, lists, counts);
    return hipGetLastError();
}

hipError_t launch_sel_list(const int32_t* topk, int B, int T, int K, int32_t* lists, int32_t* counts,
                           hipStream_t stream) {
    return launch_sel_list_range(topk, B, T, K, 0, lists, counts, stream);
}

// ------------------------------------------------------------------------------------------------
// W_UK[h] (rows h*256 + j, j < 128, of the up-projection weight, 512 wide) -> wukT[h][n][j].
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void wuk_t_kernel(const uint16_t* __restrict__ w_ukv, uint16_t* __restrict__ wukT) {
    __shared__ uint16_t tile[64][66];
    const int n0 = blockIdx.x * 64, j0 = blockIdx.y * 64, h = blockIdx.z;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < 64; r += 4) tile[r][tx] = w_ukv[((size_t)h * 256 + j0 + r) * kLora + n0 + tx];
    __syncthreads();
    for (int r = ty; r < 64; r += 4) wukT[((size_t)h * kLora + n0 + r) * kNope + j0 + tx] = tile[tx][r];
}

// ------------------------------------------------------------------------------------------------
// Per-head GEMM  out[m][h][n0 + n] = bf16( sum_k X[m][h][k] W[h][n0 + n][k] ), K = KD.
//   X element (m, k) at X + m*ldx + h*xh + k; W row (n) at W + h*wh + n*KD; out (m, n) at
//   out + m*ldo + h*oh + n. Both operands are K-contiguous (the D^T = W . X^T form of the
//   up-projection kernel: lane l owns token l % 32 and four consecutive features per group).
// BM tokens x BN features per workgroup of (BM/64)*(BN/128) waves, each 64 x 128; K streams in
// chunks of 32 through a three-stage LDS ring filled two chunks ahead by direct global->LDS
// loads; rows of 64 bytes with 16-byte chunk c of row r at c ^ ((r >> 2) & 3). The epilogue
// stages each wave's 32 x 128 blocks in the idle ring and writes 256-byte row segments.
// ------------------------------------------------------------------------------------------------
namespace gh {
constexpr int BK = 32, STAGES = 3, ROWB = 64;
}

template <int BM, int BN, int KD>
__global__ __launch_bounds__(BM * BN / 128) void gemm_heads_kernel(
    const uint16_t* __restrict__ X, size_t ldx, size_t xh, const uint16_t* __restrict__ W, size_t wh,
    int M, int mtiles, int ntiles, uint16_t* __restrict__ out, size_t ldo, size_t oh) {
    using namespace gh;
    constexpr int WM = BM / 64, WN = BN / 128, NW = WM * WN;
    constexpr int XB = BM * ROWB, WB = BN * ROWB, SB = XB + WB;
    constexpr int XL = BM / 16 / NW, WL = BN / 16 / NW;   // 1 KB loads per wave per chunk
    constexpr int LOADS = XL + WL;
    constexpr int NK = KD / BK;
    static_assert(XL * NW * 16 == BM && WL * NW * 16 == BN, "load split");
    static_assert(STAGES * SB >= NW * 8192, "epilogue staging fits the ring");
    static_assert(NK >= STAGES, "ring depth");
    __shared__ __attribute__((aligned(16))) uint8_t ring[STAGES * SB];

    const int bid = blockIdx.x;
    const int mt = bid % mtiles, rest = bid / mtiles;
    const int nt = rest % ntiles, h = rest / ntiles;
    const int m0 = mt * BM, n0 = nt * BN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, wn = wave / WM;

    // DMA: a 1 KB load covers 16 rows of 64 bytes; lane i writes row (i >> 2), physical chunk
    // (i & 3), which holds logical chunk (i & 3) ^ ((row >> 2) & 3). X rows past M repeat row M-1.
    uint32_t x_src[XL], w_src[WL];
#pragma unroll
    for (int j = 0; j < XL; ++j) {
        const int r = 16 * (XL * wave + j) + (lane >> 2);
        x_src[j] = (uint32_t)(((size_t)(min(m0 + r, M - 1) - m0) * ldx + (((lane & 3) ^ ((r >> 2) & 3)) * 8)) * 2);
    }
#pragma unroll
    for (int j = 0; j < WL; ++j) {
        const int r = 16 * (WL * wave + j) + (lane >> 2);
        w_src[j] = (uint32_t)((r * KD + (((lane & 3) ^ ((r >> 2) & 3)) * 8)) * 2);
    }
    const uint16_t* xbase = X + (size_t)m0 * ldx + (size_t)h * xh;
    const uint16_t* wbase = W + (size_t)h * wh + (size_t)n0 * KD;
    auto issue = [&](int kc, uint8_t* st) {
#pragma unroll
        for (int j = 0; j < XL; ++j) dma16(xbase + kc * BK, x_src[j], st + 16 * (XL * wave + j) * ROWB);
#pragma unroll
        for (int j = 0; j < WL; ++j) dma16(wbase + kc * BK, w_src[j], st + XB + 16 * (WL * wave + j) * ROWB);
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

    const int fr = lane & 31, fh = lane >> 5;
    int x_off[2][2], w_off[4][2];
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
            w_off[a][s] = XB + row * ROWB + (((2 * s + fh) ^ ((row >> 2) & 3)) << 4);
        }
    }

#pragma unroll
    for (int c = 0; c < STAGES - 1; ++c) issue(c, ring + c * SB);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS * (STAGES - 2)));   // chunk 0 landed
    barrier_keep_loads();
#pragma unroll
    for (int kc = 0; kc < NK; ++kc) {
        const uint8_t* st = ring + (kc % STAGES) * SB;
        if (kc + STAGES - 1 < NK) issue(kc + STAGES - 1, ring + ((kc + STAGES - 1) % STAGES) * SB);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bf16x8 bx[2], aw[4];
#pragma unroll
            for (int b = 0; b < 2; ++b) bx[b] = as_bf16x8(lds16(st + x_off[b][s]));
#pragma unroll
            for (int a = 0; a < 4; ++a) aw[a] = as_bf16x8(lds16(st + w_off[a][s]));
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) acc[a][b] = mfma32x32x16(aw[a], bx[b], acc[a][b]);
        }
        const int newer = min(NK - 1, kc + STAGES - 1) - (kc + 1);
        if (newer >= 1)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        barrier_keep_loads();
    }

    // Epilogue: wave w stages 32 x 128 blocks in bytes [8192 w, 8192 w + 8192) of the ring, rows
    // of 256 bytes with chunk c at c ^ (row & 15), then writes 256-byte row segments.
    uint8_t* ot = ring + wave * 8192;
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
            const u32x4 v = lds16(ot + row * 256 + ((c ^ (row & 15)) << 4));
            const int m = m0 + wm * 64 + b * 32 + row;
            if (m < M) store16(out + (size_t)m * ldo + (size_t)h * oh + n0 + wn * 128 + c * 8, v);
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Attention over gathered latent rows. One workgroup per query (b, s), four waves, wave w owns
// heads 32w..32w+31 (one wave per SIMD, up to 512 registers: the 32 x 512 fp32 output block sits
// in accumulation registers, 25 of the 36 sixteen-feature steps of the query fragment in vector
// registers and the other 11 in LDS).
//
// S^T = Kg . Q_lat^T per 32-key tile (lane: head l % 32, 16 of the keys), so the row max and sum
// are in-lane plus one exchange with lane l ^ 32, and the probabilities are the B operand of
// O^T = Cg^T . P^T, where Cg (the first 512 features of the gathered rows) is read through the
// transposing LDS read in the key order of the S^T accumulator.
//
// Tiles of 32 gathered keys rotate through three LDS stages (36 KB each) and are gathered two
// tiles ahead by direct global->LDS loads, one 1024-byte latent row per wave instruction. The
// latent rows keep 16-byte chunk c of row r at c ^ sigma(r), sigma(r) = 4 (r & 3) + ((r >> 2) & 3),
// which keeps both the 16-lane row reads of the score MFMAs and the 4-row x 64-byte transposing
// reads of the value MFMAs conflict free; the 128-byte rotary rows keep chunk c at
// c ^ ((r >> 1) & 7). Softmax: fp32, base-2, running max moved lazily (only when a tile's max
// exceeds it by 2^8), as in the head-major kernel.
// ------------------------------------------------------------------------------------------------
namespace lat {
constexpr int KT = 32, STAGES = 3;
constexpr int KC_ROW = 1024, KP_ROW = 128;
constexpr int KC_BYTES = KT * KC_ROW, KP_BYTES = KT * KP_ROW, STAGE_BYTES = KC_BYTES + KP_BYTES;
constexpr int QREG = 25;                      // query steps in registers; steps QREG..35 in LDS
constexpr int QLDS = 36 - QREG;
constexpr int QROW = QLDS * 32 + 16;          // bytes per head in LDS (16 of padding)
constexpr int DMAS = KT / 4 + 1;              // gather instructions per wave per tile
#ifndef LAT_RS
#define LAT_RS 3
#endif
#ifndef LAT_RP
#define LAT_RP 4
#endif
constexpr int RS = LAT_RS;                    // score steps of operands in flight
constexpr int RP = LAT_RP;                    // value MFMAs of operands in flight
}
// Score MFMAs with their accumulators in vector registers: every accumulation register of the
// kernel holds the output block, which the compiler's MFMA form places there, so the score chains
// are written as instructions with vector-register operands. The compiler does not model their
// latency: a chain is back to back on its own accumulator (the matrix unit interlocks that), and
// mfma_vgpr_drain puts 24 wait states (more than a 32x32x16 MFMA needs before a vector
// instruction may read its result) between the last MFMA and the first vector read.
__device__ __forceinline__ void mfma_vgpr_first(f32x16& c, const bf16x8& a, const bf16x8& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vgpr(f32x16& c, const bf16x8& a, const bf16x8& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vgpr_drain(f32x16& c0, f32x16& c1) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(c0), "+v"(c1));
}
__device__ __forceinline__ constexpr int lat_sigma(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

// Queries s_lo..T-1 of every sequence; query row r = b*(T - s_lo) + s - s_lo indexes the
// per-row buffers (M = B*(T - s_lo) rows).
struct LatArgs {
    const uint16_t* qlat;    // [M][128][512]
    const uint16_t* q;       // [B][T][128][192], rotary part used
    const uint16_t* ckv;     // [B][T][512]
    const uint16_t* kpe;     // [B][T][64]
    const int32_t* lists;    // [M][Lp]
    const int32_t* counts;   // [M]
    int T, M, Lp, s_lo;
    float c2;                // softmax scale * log2(e)
    uint16_t* olat;          // [128][M][512]
};

// One query m, all heads. EXACT = false: the reference is the first tile's max and the return
// value (uniform over the workgroup) says whether a later tile exceeded it by more than 64;
// EXACT = true: one pass over the keys for the exact max per head, then the output with it.
// stage j of `ring`: latent rows at j * STAGE_BYTES, rotary rows KC_BYTES further.
template <bool EXACT>
__device__ __forceinline__ bool attn_latent_query(const LatArgs& A, int m, uint8_t* ring, uint8_t* qs) {
    using namespace lat;
    const int T = A.T, M = A.M, Lp = A.Lp;
    const float c2 = A.c2;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, col = lane & 31;
    const int Tr = T - A.s_lo;
    const int b = m / Tr;
    const int tok = b * T + A.s_lo + (m - b * Tr);     // global token index of query row m
    const int n = A.counts[m];
    const int ntiles = (n + KT - 1) / KT;
    const int h = wave * 32 + col;

    const uint16_t* ckv_b = A.ckv + (size_t)b * T * kLora;
    const uint16_t* kpe_b = A.kpe + (size_t)b * T * kRope;
    const int32_t* lrow = A.lists + (size_t)m * Lp;

    // ---- gather of one tile: wave w fetches latent rows 8w..8w+7 (one instruction each: lane i
    // writes physical chunk i, i.e. logical chunk i ^ sigma(row)) and rotary rows 8w..8w+7 (one
    // instruction each, lanes 0..7). The eight key positions are one wave-uniform 32-byte load.
    typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
    i32x8 iv;
    auto load_idx = [&](int kt) __attribute__((always_inline)) {
        iv = *reinterpret_cast<const i32x8*>(lrow + kt * KT + 8 * wave);
    };
    // instruction j of a tile's gather (DMAS = 9): j < 8 latent row 8w + j, j = 8 the rotary rows
    // 8w..8w+7 (lane i -> row 8w + i/8, its key position fetched from lane i/8 of a register
    // holding the eight). LDS destinations are 32-bit LDS addresses (no generic-pointer casts).
    const uint32_t ring_lds = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)ring;
    auto issue_one = [&](uint32_t stage_lds, int j) __attribute__((always_inline)) {
        if (j < 8) {
            const uint32_t voff = (uint32_t)iv[j] * (uint32_t)KC_ROW + (uint32_t)((lane ^ lat_sigma(8 * wave + j)) << 4);
            dma16_lds(ckv_b, voff, stage_lds + (uint32_t)((8 * wave + j) * KC_ROW));
        } else {
            int vi = 0;
#pragma unroll
            for (int q = 0; q < 8; ++q) asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(vi) : "s"(iv[q]), "i"(q));
            const int ip = __builtin_amdgcn_ds_bpermute((lane >> 3) << 2, vi);
            const int r = 8 * wave + (lane >> 3);
            const uint32_t voff = (uint32_t)ip * (uint32_t)KP_ROW + (uint32_t)(((lane & 7) ^ ((r >> 1) & 7)) << 4);
            dma16_lds(kpe_b, voff, stage_lds + (uint32_t)(KC_BYTES + 8 * wave * KP_ROW));
        }
    };
    auto issue = [&](uint32_t stage_lds) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < DMAS; ++j) issue_one(stage_lds, j);
    };

    // ---- query fragment (B operand of S^T): lane holds head h, features 16 kc + 8 half .. +7 of
    // [q_lat | q_pe]; steps kc < QREG in registers, the rest in LDS (row h, 32 bytes per step).
    bf16x8 qf[QREG];
    {
        const uint16_t* ql = A.qlat + ((size_t)m * kHeads + h) * kLora + half * 8;
        const uint16_t* qp = A.q + ((size_t)tok * kHeads + h) * kQkHead + kNope + half * 8;
        auto qsrc = [&](int kc) __attribute__((always_inline)) { return kc < 32 ? ql + kc * 16 : qp + (kc - 32) * 16; };
#pragma unroll
        for (int kc = 0; kc < QREG; ++kc) qf[kc] = as_bf16x8(load16(qsrc(kc)));
#pragma unroll
        for (int kc = QREG; kc < 36; ++kc)
            *reinterpret_cast<u32x4*>(qs + h * QROW + (kc - QREG) * 32 + half * 16) = load16(qsrc(kc));
    }
    const uint8_t* qsl = qs + h * QROW + half * 16;

    // ---- per-lane LDS offsets (bytes).
    // Score operand: row col, logical chunk 2 kc + half; kc = 8 K' + kk lands at
    // 256 K' + 16 ((2 kk + half) ^ sigma(col)).
    int kc_off[8], kp_off[4], v_off[4][2];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) kc_off[kk] = col * KC_ROW + (((2 * kk + half) ^ lat_sigma(col)) << 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) kp_off[j] = col * KP_ROW + (((2 * j + half) ^ ((col >> 1) & 7)) << 4);
    // Value operand through the transposing read: 16-lane group G = lane / 16, i = lane % 16,
    // k = i / 4, q4 = i % 4. The lane addresses key row 16 c + 8 x + 4 (G / 2) + k and the four
    // features 32 dt + 16 (G % 2) + 4 q4 (logical chunk 4 dt + a, a = 2 (G % 2) + q4 / 2, byte
    // 8 (q4 % 2)); sigma of that row is 4 k + 2 x + G / 2, so the physical chunk is
    // 16 (dt / 4) + 4 ((dt % 4) ^ k) + (a ^ (2 x + G / 2)). v_off[dt % 4][x] holds everything but
    // 1024 * 16 c + 256 (dt / 4).
    {
        const int G = lane >> 4, i = lane & 15, k = i >> 2, q4 = i & 3;
        const int a = 2 * (G & 1) + (q4 >> 1);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int x = 0; x < 2; ++x)
                v_off[e][x] = (8 * x + 4 * (G >> 1) + k) * KC_ROW + 64 * (e ^ k) + 16 * (a ^ (2 * x + (G >> 1))) +
                              8 * (q4 & 1);
    }

    f32x16 o[16];
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) o[dt] = f32x16{};
    // Softmax reference per head (base 2, scaled): fixed for the whole query rather than moved
    // with the running max, so the output block is only ever touched by MFMAs. Without EXACT it
    // is the first tile's max; a later tile whose max exceeds it by more than 64 (weights up to
    // 2^64 are still exact in fp32 and bf16) marks the query for the EXACT form.
    float m_ref = -INFINITY, l_run = 0.f;
    bool bad = false;

    // S^T of one tile: two MFMA chains (steps 0..17 and 18..35), summed. With one wave per SIMD
    // nothing else hides LDS latency, so the operands of step kc + RS - 1 are read before the MFMAs
    // of step kc (scheduling barriers keep that order and bound the live operands to RS steps).
    // The gather of a later tile into stage ld_lds is spread over the first DMAS steps, one
    // instruction per step, so the loads queue behind the MFMAs instead of in one burst.
    // `piece(kc)` adds independent vector work to step kc (the previous tile's softmax).
    auto s_tile = [&](const uint8_t* kcs, const uint8_t* kps, uint32_t ld_lds, bool gather, auto&& piece)
        __attribute__((always_inline)) -> f32x16 {
        f32x16 c0, c1;
        auto a_op = [&](int kc) __attribute__((always_inline)) {
            return kc < 32 ? as_bf16x8(lds16(kcs + kc_off[kc & 7] + 256 * (kc >> 3)))
                           : as_bf16x8(lds16(kps + kp_off[kc - 32]));
        };
        auto b_op = [&](int kc) __attribute__((always_inline)) {
            return kc < QREG ? qf[kc < QREG ? kc : 0] : as_bf16x8(lds16(qsl + (kc - QREG) * 32));
        };
        bf16x8 a0[RS], a1[RS], b1[RS];
        auto fetch = [&](int kc) __attribute__((always_inline)) {
            a0[kc % RS] = a_op(kc);
            a1[kc % RS] = a_op(kc + 18);
            b1[kc % RS] = b_op(kc + 18);
        };
#pragma unroll
        for (int kc = 0; kc + 1 < RS; ++kc) fetch(kc);
#pragma unroll
        for (int kc = 0; kc < 18; ++kc) {
            if (kc + RS - 1 < 18) fetch(kc + RS - 1);
            if (gather && kc < DMAS) issue_one(ld_lds, kc);
            piece(kc);
            __builtin_amdgcn_sched_barrier(0);
            if (kc == 0) {
                mfma_vgpr_first(c0, a0[kc % RS], qf[kc]);
                mfma_vgpr_first(c1, a1[kc % RS], b1[kc % RS]);
            } else {
                mfma_vgpr(c0, a0[kc % RS], qf[kc]);
                mfma_vgpr(c1, a1[kc % RS], b1[kc % RS]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        mfma_vgpr_drain(c0, c1);
        return c0 + c1;
    };
    // Keys at list positions >= n (the padding of the last tile) get -inf.
    auto mask_tile = [&](f32x16& sc, int kbase) __attribute__((always_inline)) {
        // accumulator r holds key kbase + 8 (r / 4) + 4 half + r % 4
        const int lim = n - kbase - 4 * half;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (8 * (r >> 2) + (r & 3) >= lim) sc[r] = -INFINITY;
    };
    auto tile_max = [&](const f32x16& sc) __attribute__((always_inline)) {
        float mx = fmaxf(sc[0], sc[1]);
#pragma unroll
        for (int r = 2; r < 16; ++r) mx = fmaxf(mx, sc[r]);
        return lane_pair_max(mx) * c2;
    };
    // The softmax of one tile, split into 14 pieces of a few vector instructions, one per score
    // step of the next tile, so it runs while the matrix core works: pieces 0-3 the max over
    // the lane's 16 scores, 4 the exchange with lane l ^ 32 and the reference, 5-12 two
    // exponentials each, 13 the row sum. sv: the tile's masked scores; the probabilities land
    // in pf.
    f32x16 sv;
    bf16x8 pf[2];
    float smx = 0.f, snb = 0.f, sacc0 = 0.f, sacc1 = 0.f;
    u32x4 spk0, spk1;
    auto sm_piece = [&](int kc) __attribute__((always_inline)) {
        if (kc < 4) {
            const int r = 4 * kc;
            const float a = fmaxf(fmaxf(sv[r], sv[r + 1]), fmaxf(sv[r + 2], sv[r + 3]));
            smx = kc == 0 ? a : fmaxf(smx, a);
        } else if (kc == 4) {
            const float mt = lane_pair_max(smx) * c2;
            if (m_ref == -INFINITY) m_ref = mt;    // first tile: it holds a selected key
            bad = bad || mt > m_ref + 64.0f;
            snb = -m_ref;
            sacc0 = 0.f;
            sacc1 = 0.f;
        } else if (kc < 13) {
            const int i = kc - 5;
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[2 * i], c2, snb));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[2 * i + 1], c2, snb));
            if (i < 4) spk0[i] = pack_bf16(p0, p1); else spk1[i - 4] = pack_bf16(p0, p1);
            sacc0 += p0;
            sacc1 += p1;
        } else if (kc == 13) {
            l_run += sacc0 + sacc1;
            pf[0] = as_bf16x8(spk0);
            pf[1] = as_bf16x8(spk1);
        }
    };
    auto no_piece = [](int) {};

    // P.V of one tile: 32 MFMAs into 16 independent accumulators; the operands of MFMA i+1 are
    // read before MFMA i.
    auto pv_tile = [&](const uint8_t* kcs, const bf16x8 pf[2]) __attribute__((always_inline)) {
        auto v_op = [&](int i) __attribute__((always_inline)) {
            const int c = i >> 4, dt = i & 15;
            const uint8_t* vb = kcs + 16 * c * KC_ROW + 256 * (dt >> 2);
            const s16x4_l lo = lds_tr8(vb + v_off[dt & 3][0]);
            const s16x4_l hi = lds_tr8(vb + v_off[dt & 3][1]);
            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        // operands read RP MFMAs ahead
        bf16x8 av[RP];
#pragma unroll
        for (int i = 0; i + 1 < RP; ++i) av[i] = v_op(i);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            if (i + RP - 1 < 32) av[(i + RP - 1) % RP] = v_op(i + RP - 1);
            __builtin_amdgcn_sched_barrier(0);
            o[i & 15] = mfma32x32x16(av[i % RP], pf[i >> 4], o[i & 15]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // One sweep over the key tiles; OUT: softmax and P.V, else only the running max. The stage
    // of tile kt is kt % 3, a run-time value, so the per-lane LDS offsets exist once (added to
    // the stage base per tile) rather than once per stage. Tile kt+2 is gathered into the stage
    // freed by the barrier that ended tile kt-1, with the key positions loaded one tile earlier.
    auto sweep = [&](auto out_c) __attribute__((always_inline)) {
        constexpr bool OUT = decltype(out_c)::value;
        if (ntiles > 0) {
            load_idx(0);
            issue(ring_lds);
            if (ntiles > 1) {
                load_idx(1);
                issue(ring_lds + STAGE_BYTES);
            }
            if (ntiles > 2) load_idx(2);
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();   // the query steps in LDS and tiles 0 and 1 are in place
        if constexpr (OUT) {
            // Software pipeline: iteration t computes the scores of tile t+1 with the softmax of
            // tile t spread over its steps, then P.V of tile t. Tile t+2 is gathered during the
            // scores into the stage freed by the barrier that ended iteration t-1 and waited for at
            // the end of the iteration. The scores of "tile ntiles" in the last iteration are
            // computed on a stage holding valid rows (or, for a one-tile query, unused LDS) and
            // discarded; past the last tile the gathers repeat the last key positions loaded.
            if (ntiles > 0) {
                sv = s_tile(ring, ring + KC_BYTES, 0u, false, no_piece);
                if (ntiles == 1 && (n & (KT - 1)) != 0) mask_tile(sv, 0);
            }
            int cs = 0;    // stage of tile t
            for (int t = 0; t < ntiles; ++t) {
                const int ns = cs == 2 ? 0 : cs + 1;   // stage of tile t + 1
                const int ls = ns == 2 ? 0 : ns + 1;   // stage of tile t + 2
                const uint8_t* kcs = ring + cs * STAGE_BYTES;
                const uint8_t* kcn = ring + ns * STAGE_BYTES;
                f32x16 snext = s_tile(kcn, kcn + KC_BYTES, ring_lds + ls * STAGE_BYTES, true, sm_piece);
                if (t + 2 == ntiles && (n & (KT - 1)) != 0) mask_tile(snext, (t + 1) * KT);
                if (t + 3 < ntiles) load_idx(t + 3);
                pv_tile(kcs, pf);
                sv = snext;
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // tile t+2 gathered
                barrier_keep_loads();
                cs = ns;
            }
        } else {
            int cs = 0;    // stage of tile kt
            for (int kt = 0; kt < ntiles; ++kt) {
                const int ls = cs == 0 ? 2 : cs - 1;   // stage of tile kt + 2
                const uint8_t* kcs = ring + cs * STAGE_BYTES;
                f32x16 sc = s_tile(kcs, kcs + KC_BYTES, ring_lds + ls * STAGE_BYTES, true, no_piece);
                if (kt + 3 < ntiles) load_idx(kt + 3);
                if (kt == ntiles - 1 && (n & (KT - 1)) != 0) mask_tile(sc, kt * KT);
                m_ref = fmaxf(m_ref, tile_max(sc));
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(DMAS));   // tile kt+1 landed
                barrier_keep_loads();
                cs = cs == 2 ? 0 : cs + 1;
            }
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // no gather left in flight
    };
    if constexpr (EXACT) sweep(std::false_type{});
    sweep(std::true_type{});

    // ---- epilogue: o_lat[h][m] = O / l, rounded to bf16 (zeros for a query with no allowed key,
    // whose l and O are both 0).
    const float l_tot = lane_pair_sum(l_run);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    uint16_t* dst = A.olat + ((size_t)h * M + m) * kLora + 4 * half;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 v;
            v[0] = pack_bf16(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv);
            v[1] = pack_bf16(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv);
            store8(dst + dt * 32 + 8 * g, v);
        }
    return EXACT ? false : __syncthreads_or(bad) != 0;
}

// One workgroup per query, queries with more keys first; flags[m] says whether query m needs the
// exact-max form.
#define LAT_KERNEL_ARGS                                                                           \
    const uint16_t *__restrict__ qlat, const uint16_t *__restrict__ q, const uint16_t *__restrict__ ckv, \
        const uint16_t *__restrict__ kpe, const int32_t *__restrict__ lists,                            \
        const int32_t *__restrict__ counts, int T, int M, int Lp, int s_lo, float c2,                   \
        uint16_t *__restrict__ olat
#define LAT_ARGS_STRUCT LatArgs A{qlat, q, ckv, kpe, lists, counts, T, M, Lp, s_lo, c2, olat}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_latent_kernel(LAT_KERNEL_ARGS, int32_t* __restrict__ flags) {
    LAT_ARGS_STRUCT;
    __shared__ __attribute__((aligned(16))) uint8_t ring[lat::STAGES * lat::STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t qs[kHeads * lat::QROW];
    const int Tr = A.T - A.s_lo;
    const int b = blockIdx.x / Tr, i = blockIdx.x - b * Tr;
    const int m = b * Tr + (Tr - 1 - i);       // later queries (more keys) first
    const bool bad = attn_latent_query<false>(A, m, ring, qs);
    if (threadIdx.x == 0) flags[m] = bad ? 1 : 0;
}

// The marked queries again, with the exact max: workgroup w scans flags in blocks of 64.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_latent_exact_kernel(LAT_KERNEL_ARGS, const int32_t* __restrict__ flags) {
    LAT_ARGS_STRUCT;
    __shared__ __attribute__((aligned(16))) uint8_t ring[lat::STAGES * lat::STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t qs[kHeads * lat::QROW];
    const int lane = threadIdx.x & 63;
    for (int base = blockIdx.x * 64; base < A.M; base += gridDim.x * 64) {
        const int f = base + lane < A.M ? flags[base + lane] : 0;
        uint64_t marked = __ballot(f != 0);   // the same in every wave
        while (marked) {
            const int i = __ffsll((unsigned long long)marked) - 1;
            marked &= marked - 1;
            attn_latent_query<true>(A, base + i, ring, qs);
            __syncthreads();
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Launch sequence and workspace.
// ------------------------------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

LatentWorkspace latent_workspace(int B, int T, int K, int s_lo) {
    LatentWorkspace w;
    const size_t M = (size_t)B * (T - s_lo);
    const int Lp = latent_list_stride(T, K);
    size_t off = 0;
    w.wukT = off;   off += align256((size_t)kHeads * kLora * kNope * 2);
    w.counts = off; off += align256(M * 4);
    w.flags = off;  off += align256(M * 4);
    w.lists = off;  off += align256(M * Lp * 4);
    w.qlat = off;   off += align256(M * kHeads * kLora * 2);
    w.olat = off;   off += align256(M * kHeads * kLora * 2);
    w.bytes = off;
    return w;
}

hipError_t launch_sparse_attn_latent(const uint16_t* q, const uint16_t* c_kv, const uint16_t* k_pe,
                                     const uint16_t* w_ukv, const int32_t* topk, int B, int T, int K, int s_lo,
                                     float scale, uint16_t* out, void* workspace, hipStream_t stream) {
    const LatentWorkspace w = latent_workspace(B, T, K, s_lo);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint16_t* wukT = reinterpret_cast<uint16_t*>(ws + w.wukT);
    int32_t* counts = reinterpret_cast<int32_t*>(ws + w.counts);
    int32_t* flags = reinterpret_cast<int32_t*>(ws + w.flags);
    int32_t* lists = reinterpret_cast<int32_t*>(ws + w.lists);
    uint16_t* qlat = reinterpret_cast<uint16_t*>(ws + w.qlat);
    uint16_t* olat = reinterpret_cast<uint16_t*>(ws + w.olat);
    const int Tr = T - s_lo;
    const int M = B * Tr;
    const int Lp = latent_list_stride(T, K);

    hipError_t e = launch_sel_list_range(topk, B, T, K, s_lo, lists, counts, stream);
    if (e != hipSuccess) return e;
    wuk_t_kernel<<<dim3(kLora / 64, kNope / 64, kHeads), 256, 0, stream>>>(w_ukv, wukT);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    // q_lat[r][h][n] = sum_j q[b][s][h][j] W_UK[h][j][n], one launch per sequence (rows s_lo..T-1)
    for (int b = 0; b < B; ++b) {
        constexpr int BM = 128, BN = 256;
        const int mtiles = (Tr + BM - 1) / BM, ntiles = kLora / BN;
        gemm_heads_kernel<BM, BN, kNope><<<mtiles * ntiles * kHeads, BM * BN / 128, 0, stream>>>(
            q + ((size_t)b * T + s_lo) * kHeads * kQkHead, (size_t)kHeads * kQkHead, kQkHead, wukT,
            (size_t)kLora * kNope, Tr, mtiles, ntiles, qlat + (size_t)b * Tr * kHeads * kLora,
            (size_t)kHeads * kLora, kLora);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }

    const float c2 = (float)((double)scale * 1.4426950408889634);
    attn_latent_kernel<<<M, 256, 0, stream>>>(qlat, q, c_kv, k_pe, lists, counts, T, M, Lp, s_lo, c2, olat, flags);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) == hipSuccess) {
            int nc = 0;
            if (hipDeviceGetAttribute(&nc, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && nc > 0) cus = nc;
        }
        const int blocks = min(cus, (M + 63) / 64);
        attn_latent_exact_kernel<<<blocks, 256, 0, stream>>>(qlat, q, c_kv, k_pe, lists, counts, T, M, Lp, s_lo, c2,
                                                             olat, flags);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }

    // out[b][s][h][d] = sum_n o_lat[h][r][n] W_UV[h][d][n], W_UV[h] = rows h*256 + 128 + d
    for (int b = 0; b < B; ++b) {
        constexpr int BM = 256, BN = 128;
        const int mtiles = (Tr + BM - 1) / BM;
        gemm_heads_kernel<BM, BN, kLora><<<mtiles * kHeads, BM * BN / 128, 0, stream>>>(
            olat + (size_t)b * Tr * kLora, kLora, (size_t)M * kLora, w_ukv + (size_t)kNope * kLora,
            (size_t)256 * kLora, Tr, mtiles, 1, out + ((size_t)b * T + s_lo) * kHeads * kVHead,
            (size_t)kHeads * kVHead, kVHead);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

// ------------------------------------------------------------------------------------------------
// Split form for long sequences: queries 0..split-1 of each sequence through the head-major path
// (their keys and values formed per head, only for rows < split), queries split..T-1 through the
// latent form. The head-major cost of query s grows with s (all causal tiles are scored) while
// the latent cost is fixed by the top-k; measured on the long workload the two meet near
// s = 3.9 K, so split = min(T, 4 K) rounded down to a multiple of 256.
// ------------------------------------------------------------------------------------------------
#ifndef LAT_SPLIT_X4
#define LAT_SPLIT_X4 16   // split = (LAT_SPLIT_X4 / 4) * K
#endif
int latent_auto_split(int T, int K) {
    const long long s = ((long long)LAT_SPLIT_X4 * K / 4) / 256 * 256;
    return s >= T ? T : (int)s;
}

// When every row takes the head-major path (split = T) its buffers hold all B sequences and the
// calls are batched; otherwise one sequence's buffers are reused for each sequence in turn.
AutoWorkspace auto_workspace(int B, int T, int K) {
    AutoWorkspace a;
    a.split = latent_auto_split(T, K);
    const size_t nseq = a.split == T ? (size_t)B : 1;
    size_t off = 0;
    a.kv = off;       off += align256(nseq * kHeads * a.split * 256 * 2);
    a.bitmap = off;   off += align256(attn_select_bytes((int)nseq, a.split));
    a.latent = off;   off += a.split < T ? latent_workspace(B, T, K, a.split).bytes : 0;
    a.bytes = off;
    return a;
}

hipError_t launch_sparse_attn_auto(const uint16_t* q, const uint16_t* c_kv, const uint16_t* k_pe,
                                   const uint16_t* w_ukv, const int32_t* topk, int B, int T, int K, float scale,
                                   uint16_t* out, void* workspace, hipStream_t stream) {
    const AutoWorkspace a = auto_workspace(B, T, K);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint16_t* kvp = reinterpret_cast<uint16_t*>(ws + a.kv);
    uint32_t* bm = reinterpret_cast<uint32_t*>(ws + a.bitmap);
    hipError_t e = hipSuccess;
    if (a.split == T) {   // the head-major path for every row, all sequences at once
        if ((e = launch_gemm_kv_up(c_kv, w_ukv, B, T, kvp, stream)) != hipSuccess) return e;
        if ((e = launch_attn_select(topk, B, T, K, bm, stream)) != hipSuccess) return e;
        return launch_sparse_attn(q, kvp, k_pe, bm, B, T, scale, out, stream);
    }
    // rows 0..split-1 of sequence b are a contiguous prefix of each per-token tensor, so each
    // sequence's prefix is a one-sequence problem of length split; kv and bitmap are reused
    for (int b = 0; b < B && a.split > 0; ++b) {
        const int S = a.split;
        if ((e = launch_gemm_kv_up(c_kv + (size_t)b * T * kLora, w_ukv, 1, S, kvp, stream)) != hipSuccess) return e;
        if ((e = launch_attn_select(topk + (size_t)b * T * K, 1, S, K, bm, stream)) != hipSuccess) return e;
        if ((e = launch_sparse_attn(q + (size_t)b * T * kHeads * kQkHead, kvp, k_pe + (size_t)b * T * kRope, bm, 1, S,
                                    scale, out + (size_t)b * T * kHeads * kVHead, stream)) != hipSuccess)
            return e;
    }
    if (a.split < T)
        e = launch_sparse_attn_latent(q, c_kv, k_pe, w_ukv, topk, B, T, K, a.split, scale, out, ws + a.latent, stream);
    return e;
}

}  // namespace mla
