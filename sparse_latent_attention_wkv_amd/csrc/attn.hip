// Sparse prefill attention over the top-k selection intersected with the causal mask.
//
// "DeepSeek-V3.2-Exp · Keys", MHA-prefill code excerpt: each head's key is its 128 non-rotary
// features followed by the 64-wide rotary key shared by all heads; scores are q.k times the
// softmax scale ("DeepSeek-V3.2-Exp · Scale scores": m^2/sqrt(192)); an index mask that is -inf
// except at the indexer's top-k positions, plus the causal mask, is added to every head's
// scores; softmax over keys; the weights mix the values.
//
// Three kernels:
//  * sel_bitmap: the index mask plus causal mask as bits, bitmap[b][t/32][s] bit t%32, shared by
//    all heads (one bit per (query, key) instead of a T x T float tensor).
//  * tile_flags: per 256-query tile, one bit per 64-key tile that holds an allowed key for at
//    least one of its queries.
//  * sparse_attn: flash-style attention on a persistent grid (one workgroup per compute unit)
//    that walks work items (b, h, a tile of 256 queries) in a fixed order; of the key tiles at or
//    before the item's queries, those whose flag is set are staged in LDS (key and value rows as
//    stored) and scored, and keys outside the selection are masked to -inf, so they get exactly
//    zero weight; tiles without a flag are skipped. Online softmax in fp32 (running max and sum
//    per query, base-2 exponentials), bf16 MFMA for q.k and p.v with fp32 accumulation.
//
// MFMA formulation: S^T = K . Q^T (32 keys x 32 queries per block), so lane l owns query
// (l % 32) and 16 of the block's keys; the row max and row sum are in-lane plus one exchange
// with lane l ^ 32. The probabilities are then already laid out as the B operand of
// O^T = V^T . P^T once the keys of each 16-key group are stored in V^T in the order the S^T
// accumulator holds them (keys 4g..4g+3 and 8+4g..8+4g+3 for lane half g).
#include <math.h>

#include <type_traits>

#include "mla_device.hpp"
#include "mla_launch.hpp"

namespace mla {

// ------------------------------------------------------------------------------------------------
// Selection bitmap.
// ------------------------------------------------------------------------------------------------
// Output layout [B][Wout][Tout] with Wout >= ceil(T/32) words per query and Tout >= T query
// columns; words and queries beyond the sequence are written as zero.
template <int QR>
__global__ __launch_bounds__(256) void sel_bitmap_kernel(const int32_t* __restrict__ topk, int T, int K,
                                                         int Wout, int Tout, uint32_t* __restrict__ bitmap) {
    extern __shared__ uint32_t rows_lds[];   // QR rows of Wout words (+1 pad word per row)
    const int WP = Wout + 1;
    const int s0 = blockIdx.x * QR, b = blockIdx.y;
    const int nrows = max(0, min(QR, T - s0));
    for (int i = threadIdx.x; i < QR * WP; i += 256) rows_lds[i] = 0;
    __syncthreads();

    // The QR rows of topk are one contiguous block of nrows*K entries.
    const int32_t* base = topk + ((size_t)b * T + s0) * K;
    const int n = nrows * K;
    if ((K & 3) == 0) {
        const int n4 = n >> 2;
#pragma unroll 4
        for (int i = threadIdx.x; i < n4; i += 256) {
            const int4 v = reinterpret_cast<const int4*>(base)[i];
            const int e = i * 4;
            const int qi = e / K;          // the four entries share a row since K % 4 == 0
            const unsigned s = (unsigned)(s0 + qi);
            uint32_t* row = rows_lds + qi * WP;
            if ((unsigned)v.x <= s) atomicOr(row + (v.x >> 5), 1u << (v.x & 31));
            if ((unsigned)v.y <= s) atomicOr(row + (v.y >> 5), 1u << (v.y & 31));
            if ((unsigned)v.z <= s) atomicOr(row + (v.z >> 5), 1u << (v.z & 31));
            if ((unsigned)v.w <= s) atomicOr(row + (v.w >> 5), 1u << (v.w & 31));
        }
    } else {
#pragma unroll 4
        for (int i = threadIdx.x; i < n; i += 256) {
            const int t = base[i];
            const int qi = i / K;
            if ((unsigned)t <= (unsigned)(s0 + qi)) atomicOr(rows_lds + qi * WP + (t >> 5), 1u << (t & 31));
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < Wout * QR; i += 256) {
        const int qi = i % QR, w = i / QR;
        if (s0 + qi < Tout) bitmap[((size_t)b * Wout + w) * Tout + s0 + qi] = rows_lds[qi * WP + w];
    }
}

hipError_t launch_sel_bitmap(const int32_t* topk, int B, int T, int K, int Wout, int Tout,
                             uint32_t* bitmap, hipStream_t stream) {
    constexpr int QR = 8;
    const dim3 grid((Tout + QR - 1) / QR, B);
    const size_t lds = (size_t)QR * (Wout + 1) * sizeof(uint32_t);
    sel_bitmap_kernel<QR><<<grid, 256, lds, stream>>>(topk, T, K, Wout, Tout, bitmap);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Tile flags: bit (kt % 32) of flags[b][qt][kt / 32] is set when some query of the 256-query tile
// qt has an allowed key among the 64 keys of tile kt, i.e. when one of the words 2kt, 2kt+1 of one
// of its bitmap columns is nonzero. Block (qt, g, b) writes byte g of the row (key tiles
// 8g..8g+7; zero for tiles past the sequence); thread j reads column qt*256 + j of their 16
// words (each wave load is 256 consecutive bytes).
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tile_flags_kernel(const uint32_t* __restrict__ bitmap, int Wp, int Tpad,
                                                         int nqt, int FW, uint8_t* __restrict__ flags) {
    __shared__ uint32_t part[4];
    const int qt = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int w0 = 16 * g;
    const int nw = max(0, min(16, Wp - w0));
    const uint32_t* col = bitmap + ((size_t)b * Wp + w0) * Tpad + (size_t)qt * 256 + threadIdx.x;
    uint32_t bits = 0;
#pragma unroll 8
    for (int i = 0; i < nw; ++i)
        if (col[(size_t)i * Tpad] != 0u) bits |= 1u << (i >> 1);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) bits |= (uint32_t)__shfl_xor((int)bits, off, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = bits;
    __syncthreads();
    if (threadIdx.x == 0)
        flags[((size_t)b * nqt + qt) * FW * 4 + g] = (uint8_t)(part[0] | part[1] | part[2] | part[3]);
}

// ------------------------------------------------------------------------------------------------
// Attention.
// ------------------------------------------------------------------------------------------------
// Work item: 8 waves (two per SIMD) x 32 queries = 256 queries of one (b, h); a workgroup runs
// its items one after another.
//
// Key tiles of 64 keys (two 32-key blocks) rotate through three statically distinct LDS stages
// filled by direct global->LDS loads; tile kt+2 is loaded while tile kt is computed, and one
// barrier ends each tile.
//
// LDS stage, rows stored without padding, 16-byte chunks XOR-swizzled by row so that every
// operand read is bank-conflict free (LDS serves 256 B per clock: 16 lanes of a 16-byte read,
// 32 lanes of an 8-byte read):
//   kn [64 keys][128] bf16 (256 B rows), chunk ^= row & 15
//   kp [64 keys][64]  bf16 (128 B rows), chunk ^= (row >> 1) & 7
//   v  [64 keys][128] bf16 (256 B rows), chunk ^= 4 * (row & 3)
//   bm [2 words][256 queries] u32 (the tile's selection bits)
// V stays key-major; the transposing LDS read (ds_read_b64_tr_b16) delivers it as the
// [feature][key] operand of O^T = V^T . P^T. Within each 16-lane group that read gives lane i,
// slot k the element (i % 4) at the address of lane 4k + i/4, so a lane group addressing four
// key rows x four feature quads receives 16 features x 4 keys transposed.
//
// Software pipeline over 64-key tiles t of each wave:
//   X_t:  S(t+1) MFMAs (two chains)       |  exponentials, packing and sums of tile t
//   (rare) rescale O for tile t
//   Y_t:  P.V MFMAs of tile t (8 chains)  |  mask and row max of tile t+1
// so the matrix cores and the vector units of each wave have independent work, no wave runs a
// single dependent MFMA chain, and the two waves sharing a SIMD fill each other's stalls.
constexpr int kKT = 64;
constexpr int kWaves = 8;
constexpr int kQW = 32;                  // queries per wave
constexpr int kQT = kWaves * kQW;        // 256 queries per workgroup
constexpr int kMaxKeyTiles = 32768 / kKT; // key tiles of the longest accepted sequence

typedef short s16x4 __attribute__((ext_vector_type(4)));

struct Stage {
    uint16_t* kn;
    uint16_t* kp;
    uint16_t* v;
    uint32_t* bm;
    uint32_t kn_l, kp_l, v_l, bm_l;   // the same as 32-bit LDS addresses (load destinations)
};

__device__ __forceinline__ u32x4 lds_read16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ s16x4 lds_read_tr(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}
// vmcnt(0): every global->LDS load of this wave has landed
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x3F70); }

// max / sum over the two lanes l and l ^ 32
__device__ __forceinline__ float half_max(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Softmax part 1 for one 64-key tile held by this lane as two 32-key x 32-query S^T blocks
// (16 keys of its query each): keys outside the selection become -inf, then the tile's row max
// over both lane halves.
__device__ __forceinline__ void sm_mask(f32x16& s, uint32_t word, int half) {
    // accumulator r holds key 8*(r/4) + 4*half + (r%4) of the block
    const uint32_t w = word >> (4 * half);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int bit = 8 * (r >> 2) + (r & 3);
        const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe(w, bit, 1);
        s[r] = __uint_as_float((__float_as_uint(s[r]) & keep) | (0xFF800000u & ~keep));
    }
}
__device__ __forceinline__ float sm_max(const f32x16 s[2]) {
    float mx = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) mx = fmaxf(fmaxf(mx, s[0][r]), s[0][r + 1]);
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, s[1][r]), s[1][r + 1]);
    mx = fmaxf(mx, s[0][15]);
    return half_max(mx);
}

// Softmax part 2 for one tile: lazy running-max update (the max moves only when the tile's max
// exceeds it by more than 2^8 in base 2, so probabilities stay <= 256), rescale of the running
// sum, probabilities packed as the bf16 B operands of the value MFMAs, and their fp32 sum.
__device__ __forceinline__ void sm_exp(const f32x16 s[2], float mx, float c2, float& m_run, float& l_run,
                                       float& alpha, bf16x8 pf[2][2]) {
    const float mt = mx * c2;
    const bool need = mt > m_run + 8.0f;
    alpha = need ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;
    m_run = need ? mt : m_run;
    l_run *= alpha;
    const float nb = m_run == -INFINITY ? 0.f : -m_run;
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            u32x4 pk;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s[sb][8 * c + 2 * i], c2, nb));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s[sb][8 * c + 2 * i + 1], c2, nb));
                pk[i] = pack_bf16(p0, p1);
                acc0 += p0;
                acc1 += p1;
            }
            pf[sb][c] = as_bf16x8(pk);
        }
    l_run += acc0 + acc1;
}

__global__ __launch_bounds__(512) void sparse_attn_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ kv,
                                                          const uint16_t* __restrict__ kpe,
                                                          const uint32_t* __restrict__ bitmap,
                                                          const uint32_t* __restrict__ tflags, int T,
                                                          int Tpad, int Wp, int FW, int nqt, int BH,
                                                          int npairs, int units, float c2,
                                                          uint16_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint16_t knA[kKT * 128], knB[kKT * 128], knC[kKT * 128];
    __shared__ __attribute__((aligned(16))) uint16_t kpA[kKT * 64], kpB[kKT * 64], kpC[kKT * 64];
    __shared__ __attribute__((aligned(16))) uint16_t vA[kKT * 128], vB[kKT * 128], vC[kKT * 128];
    __shared__ __attribute__((aligned(16))) uint32_t bmA[2 * kQT], bmB[2 * kQT], bmC[2 * kQT];
    // each thread's fixed load offsets (four key/value rows, one rotary row), kept in LDS rather
    // than in registers: they are read once per tile
    __shared__ __attribute__((aligned(16))) uint32_t off_lds[kWaves * 64 * 5];
    // the item's key tiles to score, ascending, and their count; the flag rows of the current
    // and the next item (lane l of wave 0 loads word min(l, FW - 1) of a row)
    __shared__ uint16_t kt_list[kMaxKeyTiles];
    __shared__ int kt_count;
    __shared__ uint32_t flag_lds[2][64];
    const Stage stA{knA, kpA, vA, bmA, lds_addr(knA), lds_addr(kpA), lds_addr(vA), lds_addr(bmA)};
    const Stage stB{knB, kpB, vB, bmB, lds_addr(knB), lds_addr(kpB), lds_addr(vB), lds_addr(bmB)};
    const Stage stC{knC, kpC, vC, bmC, lds_addr(knC), lds_addr(kpC), lds_addr(vC), lds_addr(bmC)};

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, col = lane & 31;

    // Persistent schedule. A unit is a pair of query tiles of one (b, h): tile nqt-1-p (the
    // longer) then tile p, so under the causal mask every unit costs about the same number of
    // key tiles. Workgroups are dealt to the 8 XCDs round-robin, so workgroup w sits on XCD
    // w % 8 and takes the units u = w, w + G, ... (G a multiple of 8), all of that XCD: unit u
    // covers head bh = u % 8 + 8 * g and the pair (k % npairs + j0) % npairs, k = u / 8,
    // g = k / npairs, where j0 is the step (u0 / G) at which the head's first unit u0 runs. The
    // workgroups of one XCD run the pairs of a few heads side by side and in step, so those heads'
    // keys and values are shared through that XCD's L2; the rotation by j0 hands a workgroup a
    // different pair at each step (every pair once when npairs divides G / 8), so when skipped
    // key tiles make the pairs' costs differ, the workgroups' totals still even out.
    // (BH is a multiple of 8, so every unit names a head below BH.)
    auto unit_of = [&](int u, int& bh, int& pr) {
        const int k_ = u >> 3;
        const int grp = k_ / npairs;
        bh = (u & 7) + 8 * grp;
        const int j0 = ((u & 7) + 8 * grp * npairs) / (int)gridDim.x;
        pr = (k_ - grp * npairs + j0) % npairs;
    };
    // Wave 0 loads each item's row of key-tile flags into LDS one item ahead (the first one here),
    // so building an item's tile list waits for no global load: a row loaded during an item has
    // landed by that item's first tile-end wait.
    auto load_flags = [&](int slot, int fb, int fqt) {
        dma4_lds(tflags + ((size_t)fb * nqt + fqt) * FW, (uint32_t)min(lane, FW - 1) * 4u,
                 lds_addr(&flag_lds[slot][0]));
    };
    if (wave == 0) {
        int bh0, pr0;
        unit_of(blockIdx.x, bh0, pr0);
        load_flags(0, bh0 / kHeads, nqt - 1 - pr0);
        wait_vm0();
    }
    int fslot = 0;
    for (int u = blockIdx.x; u < units; u += gridDim.x) {
    int bh, pr;
    unit_of(u, bh, pr);
    if (bh >= BH) continue;
    const int b = bh / kHeads, h = bh - b * kHeads;
    for (int item = 0; item < 2; ++item) {
    const int qt = item == 0 ? nqt - 1 - pr : pr;
    if (item == 1 && qt == nqt - 1 - pr) break;   // odd count: the middle tile stands alone
    const int q0 = qt * kQT;
    const int wq0 = q0 + wave * kQW;
    const int qrow = wq0 + col;

    const uint16_t* kvh = kv + (size_t)bh * T * 256;
    const uint16_t* kpeb = kpe + (size_t)b * T * kRope;
    const uint32_t* bmb = bitmap + (size_t)b * Wp * Tpad;

    // Q^T fragments (B operand of S^T = K . Q^T): lane holds query qrow, features kc*16 + 8*half.
    bf16x8 qf[12];
    {
        const uint16_t* src = q + (((size_t)b * T + qrow) * kHeads + h) * kQkHead + half * 8;
#pragma unroll
        for (int kc = 0; kc < 12; ++kc)
            qf[kc] = as_bf16x8(qrow < T ? load16(src + kc * 16) : u32x4{0, 0, 0, 0});
    }

    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    // ---- global -> LDS loads of one tile. Each wave instruction moves 1 KB (64 lanes x 16 B) to
    // consecutive LDS; the swizzle is applied by choosing which source chunk each lane fetches.
    //   waves 0-3: kn rows 16w..16w+15 (4 instructions); waves 4-7: v rows 16(w-4).. (4);
    //   every wave: kp rows 8w..8w+7 (1); waves 0-1: bm word w of the tile (1).
    // Per-lane byte offsets are taken from the head's (or sequence's) first row, so the scalar
    // bases stay fixed and only the tile's first key t0 enters each offset; a row past the
    // sequence (last tile only) is clamped to the last key (never selected). Offsets stay below
    // 2^32: at most 32768 rows of 512 bytes, and 2 * ceil(T/64) * Tpad * 4 bytes of bitmap.
    const int r16 = lane >> 4;
    uint32_t chunk_off[4];   // bytes within the key row
    const bool kn_wave = wave < 4;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int lc = kn_wave ? (lane & 15) ^ ((4 * k + r16) & 15) : (lane & 15) ^ (4 * r16);
        chunk_off[k] = (uint32_t)(lc * 16 + (kn_wave ? 0 : 2 * kNope));
    }
    const int kp_row = 8 * wave + (lane >> 3);
    {
        const uint32_t kp_chunk = (uint32_t)(((lane & 7) ^ ((kp_row >> 1) & 7)) << 4);
        *reinterpret_cast<u32x4*>(off_lds + 4 * tid) = u32x4{chunk_off[0], chunk_off[1], chunk_off[2], chunk_off[3]};
        off_lds[kWaves * 64 * 4 + tid] = kp_chunk;
    }
    auto issue_tile = [&](const Stage& st, int kt) {
        const u32x4 ch = *reinterpret_cast<const u32x4*>(off_lds + 4 * tid);
        const uint32_t kp_ch = off_lds[kWaves * 64 * 4 + tid];
        const int t0 = kt * kKT;
        const uint32_t dst = kn_wave ? st.kn_l : st.v_l;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int row = 16 * (wave & 3) + 4 * k + r16;
            dma16_lds(kvh, (uint32_t)min(t0 + row, T - 1) * 512u + ch[k],
                      dst + (uint32_t)((16 * (wave & 3) + 4 * k) * 128 * 2));
        }
        dma16_lds(kpeb, (uint32_t)min(t0 + kp_row, T - 1) * (2u * kRope) + kp_ch,
                  st.kp_l + (uint32_t)(8 * wave * 64 * 2));
        if (wave < 2)
            dma16_lds(bmb + q0, (uint32_t)((kt * 2 + wave) * Tpad) * 4u + (uint32_t)lane * 16,
                      st.bm_l + (uint32_t)(wave * kQT * 4));
    };

    // ---- per-lane LDS read offsets (bytes).
    // K operand: key row (sub*32 + col), 16-byte chunk (2*kc + half) of the row, swizzled.
    int kn_off[8], kpr_off[4], v_off[4];
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) kn_off[kc] = col * 256 + (((2 * kc + half) ^ (col & 15)) << 4);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) kpr_off[kc] = col * 128 + (((2 * kc + half) ^ ((col >> 1) & 7)) << 4);
    // V operand via the transposing read: lane group g = lane/16, i = lane%16; the lane addresses
    // key row (16c + 8n + 4*(g/2) + i/4) and feature quad 32dt + 16*(g%2) + 4*(i%4).
    {
        const int g = lane >> 4, i = lane & 15, k = i >> 2, qq = i & 3;
        const int key = 4 * (g >> 1) + k;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const int lc = 4 * dt + 2 * (g & 1) + (qq >> 1);
            v_off[dt] = key * 256 + ((lc ^ (4 * k)) << 4) + (qq & 1) * 8;
        }
    }
    const int bm_lane = wave * kQW + col;

    // S^T for both 32-key blocks of a tile: two independent MFMA chains sharing the Q operand.
    auto s_tile = [&](const Stage& st, f32x16 s[2]) {
        const uint8_t* kn = reinterpret_cast<const uint8_t*>(st.kn);
        const uint8_t* kp = reinterpret_cast<const uint8_t*>(st.kp);
        auto rd = [&](int j, int blk) -> bf16x8 {
            return j < 8 ? as_bf16x8(lds_read16(kn + blk * 32 * 256 + kn_off[j]))
                         : as_bf16x8(lds_read16(kp + blk * 32 * 128 + kpr_off[j - 8]));
        };
        s[0] = f32x16{};
        s[1] = f32x16{};
        // the 24 key operands (step j, block b) in order 2j + b, each read three MFMAs ahead
        bf16x8 r0 = rd(0, 0), r1 = rd(0, 1), r2 = rd(1, 0);
#pragma unroll
        for (int i = 0; i < 24; ++i) {
            const int j = i >> 1, blk = i & 1;
            bf16x8 nx = r2;   // unused past the last step
            if (i + 3 < 24) nx = rd((i + 3) >> 1, (i + 3) & 1);
            s[blk] = mfma32x32x16(r0, qf[j], s[blk]);
            r0 = r1;
            r1 = r2;
            r2 = nx;
        }
    };
    auto pv_tile = [&](const Stage& st, const bf16x8 pf[2][2]) {
        const uint8_t* vb = reinterpret_cast<const uint8_t*>(st.v);
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const s16x4 lo = lds_read_tr(vb + v_off[dt] + (32 * sb + 16 * c) * 256);
                    const s16x4 hi = lds_read_tr(vb + v_off[dt] + (32 * sb + 16 * c + 8) * 256);
                    const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    o[dt] = mfma32x32x16(a, pf[sb][c], o[dt]);
                }
            }
    };
    auto mask_tile = [&](const Stage& st, f32x16 s[2]) {
        sm_mask(s[0], st.bm[bm_lane], half);
        sm_mask(s[1], st.bm[kQT + bm_lane], half);
        return sm_max(s);
    };

    // Pipeline state carried between tiles: masked scores and row max of the next tile.
    f32x16 s_cur[2];
    float mx_cur;

    // One tile t in stage `cur` (values) with tile t+1 in `nxt` (keys, selection bits) and tile
    // t+2 loading into `ld`.
    //   X_t: S(t+1) MFMAs | exponentials of t;  rare O rescale;  Y_t: P.V of t | mask, max of t+1
    // Key tile to load at the start of tile i (entry i + 2 of the list), read from LDS at the start
    // of the tile before, so the read completes under that tile's work.
    int kt_ahead = 0;
    auto tile = [&](int i, int n, const Stage& cur, const Stage& nxt, const Stage& ld) {
        const int kt_load = __builtin_amdgcn_readfirstlane(kt_ahead);
        kt_ahead = kt_list[min(i + 3, n - 1)];
        if (i + 2 < n) issue_tile(ld, kt_load);
        f32x16 s_nx[2];
        bf16x8 pf[2][2];
        float alpha;
        s_tile(nxt, s_nx);
        sm_exp(s_cur, mx_cur, c2, m_run, l_run, alpha, pf);
        if (__any(alpha != 1.0f)) {
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
        }
        pv_tile(cur, pf);
        mx_cur = mask_tile(nxt, s_nx);
        s_cur[0] = s_nx[0];
        s_cur[1] = s_nx[1];
        wait_vm0();
        __syncthreads();
    };

    // Key tiles at or before the item's last query whose flag is set, listed in ascending order by
    // wave 0 (lane l looks at tiles 8l..8l+7). An item without any allowed key gets the list {0}:
    // tile 0's selection bits are then all clear, so every weight is zero and its rows are zeros.
    const int q_last = min(T, q0 + kQT) - 1;
    const int nkt = q_last / kKT + 1;
    if (wave == 0) {
        const int t8 = 8 * lane;
        uint32_t f = 0;
        if (t8 < nkt) {
            f = (flag_lds[fslot][lane >> 2] >> (8 * (lane & 3))) & 0xFFu;
            if (nkt - t8 < 8) f &= (1u << (nkt - t8)) - 1u;
        }
        // the next item: tile pr of this unit, else the first tile of the workgroup's next unit
        if (item == 0 && pr != nqt - 1 - pr) {
            load_flags(fslot ^ 1, b, pr);
        } else if (u + (int)gridDim.x < units) {
            int nbh, npr;
            unit_of(u + (int)gridDim.x, nbh, npr);
            load_flags(fslot ^ 1, nbh / kHeads, nqt - 1 - npr);
        }
        const int c = __builtin_popcount(f);
        int incl = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off, 64);
            if (lane >= off) incl += y;
        }
        int pos = incl - c;
        while (f) {
            kt_list[pos++] = (uint16_t)(t8 + __builtin_ctz(f));
            f &= f - 1u;
        }
        const int total = __shfl(incl, 63, 64);
        if (lane == 0) {
            if (total == 0) kt_list[0] = 0;
            kt_count = total > 0 ? total : 1;
        }
    }
    fslot ^= 1;
    __syncthreads();
    const int n = __builtin_amdgcn_readfirstlane(kt_count);

    issue_tile(stA, __builtin_amdgcn_readfirstlane((int)kt_list[0]));
    if (n > 1) issue_tile(stB, __builtin_amdgcn_readfirstlane((int)kt_list[1]));
    kt_ahead = kt_list[min(2, n - 1)];
    wait_vm0();
    __syncthreads();
    s_tile(stA, s_cur);
    mx_cur = mask_tile(stA, s_cur);
    for (int i = 0; i < n; i += 3) {
        tile(i, n, stA, stB, stC);
        if (i + 1 >= n) break;
        tile(i + 1, n, stB, stC, stA);
        if (i + 2 >= n) break;
        tile(i + 2, n, stC, stA, stB);
    }

    // Epilogue: the two lane halves hold partial sums over different keys of the same query.
    // A query with no allowed key has l_tot = 0 and o = 0: its row is written as zeros.
    const float l_tot = half_sum(l_run);
    if (qrow < T) {
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        uint16_t* dst = out + (((size_t)b * T + qrow) * kHeads + h) * kVHead;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 v;
                v[0] = pack_bf16(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv);
                v[1] = pack_bf16(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv);
                store8(dst + dt * 32 + 8 * g + 4 * half, v);
            }
    }
    }   // items of the unit
    }   // units
}

int attn_bitmap_words(int T) { return 2 * ((T + kKT - 1) / kKT); }
int attn_bitmap_cols(int T) { return (T + kQT - 1) / kQT * kQT; }
int attn_flag_words(int T) { return ((T + kKT - 1) / kKT + 31) / 32; }
size_t attn_select_bytes(int B, int T) {
    const size_t bm = (size_t)B * attn_bitmap_words(T) * attn_bitmap_cols(T) * 4;
    const size_t fl = (size_t)B * ((T + kQT - 1) / kQT) * attn_flag_words(T) * 4;
    return bm + ((fl + 255) & ~(size_t)255);
}

hipError_t launch_attn_select(const int32_t* topk, int B, int T, int K, uint32_t* sel, hipStream_t stream) {
    const int Wp = attn_bitmap_words(T), Tpad = attn_bitmap_cols(T);
    hipError_t e = launch_sel_bitmap(topk, B, T, K, Wp, Tpad, sel, stream);
    if (e != hipSuccess) return e;
    const int nqt = Tpad / kQT, FW = attn_flag_words(T);
    tile_flags_kernel<<<dim3(nqt, 4 * FW, B), 256, 0, stream>>>(
        sel, Wp, Tpad, nqt, FW, reinterpret_cast<uint8_t*>(sel + (size_t)B * Wp * Tpad));
    return hipGetLastError();
}

hipError_t launch_sparse_attn(const uint16_t* q, const uint16_t* kv, const uint16_t* k_pe,
                              const uint32_t* sel, int B, int T, float scale, uint16_t* out,
                              hipStream_t stream) {
    const int nqt = (T + kQT - 1) / kQT;
    const int npairs = (nqt + 1) / 2;
    const int BH = B * kHeads;
    const int units = 8 * ((BH + 7) / 8) * npairs;     // a multiple of 8
    // one workgroup per compute unit (the LDS use admits one), a multiple of 8
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n >= 8) cus = n;
    }
    const int G = min(units, cus / 8 * 8);
    const float c2 = (float)((double)scale * 1.4426950408889634);   // scale * log2(e)
    const int Wp = attn_bitmap_words(T), Tpad = attn_bitmap_cols(T);
    sparse_attn_kernel<<<G, kWaves * 64, 0, stream>>>(q, kv, k_pe, sel, sel + (size_t)B * Wp * Tpad, T, Tpad,
                                                      Wp, attn_flag_words(T), nqt, BH, npairs, units, c2,
                                                      out);
    return hipGetLastError();
}

}  // namespace mla
