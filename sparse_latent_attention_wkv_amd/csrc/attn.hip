// Sparse prefill attention over the top-k selection intersected with the causal mask.
//
// "DeepSeek-V3.2-Exp · Keys", MHA-prefill code excerpt: each head's key is its 128 non-rotary
// features followed by the 64-wide rotary key shared by all heads; scores are q.k times the
// softmax scale ("DeepSeek-V3.2-Exp · Scale scores": m^2/sqrt(192)); an index mask that is -inf
// except at the indexer's top-k positions, plus the causal mask, is added to every head's
// scores; softmax over keys; the weights mix the values.
//
// Two kernels:
//  * sel_bitmap: the index mask plus causal mask as bits, bitmap[b][t/32][s] bit t%32, shared by
//    all heads (one bit per (query, key) instead of a T x T float tensor).
//  * sparse_attn: flash-style attention. One workgroup owns (b, h, a tile of queries); key tiles
//    of 64 are staged in LDS (K as [key][192], V transposed as [128][key]); a key block that no
//    query of a wave selects is skipped, selected-but-not-all blocks are scored and masked to
//    -inf, so masked keys get exactly zero weight. Online softmax in fp32 (running max and sum
//    per query, base-2 exponentials), bf16 MFMA for q.k and p.v with fp32 accumulation.
//
// MFMA formulation: S^T = K . Q^T (32 keys x 32 queries per block), so lane l owns query
// (l % 32) and 16 of the block's keys; the row max and row sum are in-lane plus one exchange
// with lane l ^ 32. The probabilities are then already laid out as the B operand of
// O^T = V^T . P^T once the keys of each 16-key group are stored in V^T in the order the S^T
// accumulator holds them (keys 4g..4g+3 and 8+4g..8+4g+3 for lane half g).
#include <math.h>

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
// Attention.
// ------------------------------------------------------------------------------------------------
// Workgroup: 8 waves (two per SIMD) x 32 queries = 256 queries of one (b, h). Key tiles of 64
// are double-buffered in LDS; the next tile's global loads are in flight while the current tile
// is computed, and one barrier per tile separates the stages.
//
// LDS stage (bytes), rows stored without padding and 16-byte chunks XOR-swizzled by row so the
// MFMA operand reads are bank-conflict free:
//   Kn  [64 keys][128] bf16, chunk ^= row & 15                   16384
//   Kp  [64 keys][64]  bf16, chunk ^= row & 7                     8192
//   V   [64 keys][128] bf16, chunk ^= 2 * (row & 3)              16384
//   Bm  [2 words][256 queries] u32 (selection bits of the tile)   2048
// V stays key-major; the transposing LDS read (ds_read_b64_tr_b16) delivers it as the
// [feature][key] operand of O^T = V^T . P^T. Within each 16-lane group that read gives lane i,
// slot k the element (i % 4) at the address of lane 4k + i/4, so a lane group addressing four
// key rows x four feature quads receives 16 features x 4 keys transposed.
constexpr int kKT = 64;
constexpr int kWaves = 8;
constexpr int kQT = kWaves * 32;
constexpr int kOffKn = 0, kOffKp = 16384, kOffV = 24576, kOffBm = 40960, kStage = 43008;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ u32x4 lds_read16(const lds_u8* p) {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p);
}
__device__ __forceinline__ void lds_write16(lds_u8* p, const u32x4& v) {
    *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(p) = v;
}
__device__ __forceinline__ uint32_t lds_read4(const lds_u8* p) {
    return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(p);
}
__device__ __forceinline__ s16x4 lds_read_tr(const lds_u8* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
}

// max over the two lanes l and l ^ 32
__device__ __forceinline__ float half_max(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__global__ __launch_bounds__(512) void sparse_attn_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ kv,
                                                          const uint16_t* __restrict__ kpe,
                                                          const uint32_t* __restrict__ bitmap, int T,
                                                          int Tpad, int Wp, int nqt, float c2,
                                                          uint16_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint8_t smem_generic[2 * kStage];
    lds_u8* smem = (lds_u8*)smem_generic;

    // Workgroups are dealt to the 8 XCDs round-robin. Every query tile of one (b, h) goes to
    // the same XCD so the head's keys and values stay in that XCD's L2; within a head the
    // longest (latest) query tiles start first.
    const int wg = blockIdx.x;
    const int xcd = wg & 7, j = wg >> 3;
    const int bh = xcd + 8 * (j / nqt);
    const int qt = nqt - 1 - (j % nqt);
    const int b = bh / kHeads, h = bh - b * kHeads;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, col = lane & 31;
    const int q0 = qt * kQT;
    const int wq0 = q0 + wave * 32;
    const int wq_last = min(T - 1, wq0 + 31);
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

    // ---- staging: 2 Kn + 1 Kp + 2 V chunks per thread, plus 1 bitmap chunk for threads < 128.
    u32x4 r_kn[2], r_kp, r_v[2], r_bm;
    auto gload = [&](int kt) {
        const int t0 = kt * kKT;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + 512 * i, row = c >> 4, lc = c & 15;
            const int t = min(t0 + row, T - 1);
            r_kn[i] = load16(kvh + (size_t)t * 256 + lc * 8);
            r_v[i] = load16(kvh + (size_t)t * 256 + kNope + lc * 8);
        }
        {
            const int row = tid >> 3, lc = tid & 7;
            const int t = min(t0 + row, T - 1);
            r_kp = load16(kpeb + (size_t)t * kRope + lc * 8);
        }
        if (tid < 128) {
            const int ww = tid >> 6, q4 = (tid & 63) * 4;
            r_bm = load16(bmb + (size_t)(kt * 2 + ww) * Tpad + q0 + q4);
        }
    };
    auto lstore = [&](int stage) {
        lds_u8* base = smem + stage * kStage;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + 512 * i, row = c >> 4, lc = c & 15;
            lds_write16(base + kOffKn + row * 256 + ((lc ^ (row & 15)) << 4), r_kn[i]);
            lds_write16(base + kOffV + row * 256 + ((lc ^ ((row & 3) << 1)) << 4), r_v[i]);
        }
        {
            const int row = tid >> 3, lc = tid & 7;
            lds_write16(base + kOffKp + row * 128 + ((lc ^ (row & 7)) << 4), r_kp);
        }
        if (tid < 128) {
            const int ww = tid >> 6, q4 = (tid & 63) * 4;
            lds_write16(base + kOffBm + (ww * 256 + q4) * 4, r_bm);
        }
    };

    // ---- per-lane LDS read offsets.
    // K operand: key row (sub*32 + col), 16-byte chunk (2*kc + half) of the row, swizzled.
    int kn_off[8], kp_off[4];
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) kn_off[kc] = kOffKn + col * 256 + (((2 * kc + half) ^ (col & 15)) << 4);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) kp_off[kc] = kOffKp + col * 128 + (((2 * kc + half) ^ (col & 7)) << 4);
    // V operand via the transposing read: lane group g = lane/16, i = lane%16; the lane
    // addresses key row (16c + 8n + 4*(g/2) + i/4) and feature quad 32dt + 16*(g%2) + 4*(i%4).
    int v_off[4];
    {
        const int g = lane >> 4, i = lane & 15, k = i >> 2, qq = i & 3;
        const int key = 4 * (g >> 1) + k;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const int lc = 4 * dt + 2 * (g & 1) + (qq >> 1);
            v_off[dt] = kOffV + key * 256 + ((lc ^ (k << 1)) << 4) + (qq & 1) * 8;
        }
    }
    const int bm_off = kOffBm + (wave * 32 + col) * 4;

    const int q_last = min(T, q0 + kQT) - 1;
    const int nkt = q_last / kKT + 1;

    gload(0);
    lstore(0);
    if (nkt > 1) gload(1);
    __syncthreads();

    for (int kt = 0; kt < nkt; ++kt) {
        const lds_u8* base = smem + (kt & 1) * kStage;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int kb = kt * kKT + sub * 32;
            if (kb > wq_last) break;                      // keys all in this wave's future
            const uint32_t word = lds_read4(base + bm_off + sub * 1024);
            if (!__any(word != 0u)) continue;             // no query of this wave selects here
            const bool full = __all(word == 0xFFFFFFFFu);

            // S^T block: 32 keys x 32 queries, 192 features.
            f32x16 s = f32x16{};
            const lds_u8* kb_base = base + sub * 32 * 256;
            const lds_u8* kp_base = base + sub * 32 * 128;
#pragma unroll
            for (int kc = 0; kc < 8; ++kc)
                s = mfma32x32x16(as_bf16x8(lds_read16(kb_base + kn_off[kc])), qf[kc], s);
#pragma unroll
            for (int kc = 0; kc < 4; ++kc)
                s = mfma32x32x16(as_bf16x8(lds_read16(kp_base + kp_off[kc])), qf[8 + kc], s);

            if (!full) {
                // accumulator r holds key 8*(r/4) + 4*half + (r%4) of the block
                const uint32_t w = word >> (4 * half);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int bit = 8 * (r >> 2) + (r & 3);
                    const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe(w, bit, 1);
                    s[r] = __uint_as_float((__float_as_uint(s[r]) & keep) | (0xFF800000u & ~keep));
                }
            }
            float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
            for (int r = 3; r < 15; r += 2) mx = fmaxf(fmaxf(mx, s[r]), s[r + 1]);
            mx = fmaxf(mx, s[15]);
            const float mt = half_max(mx) * c2;

            // Lazy rescale: the running max moves only when the block's max exceeds it by more
            // than 2^8, so probabilities stay <= 256 and the O rescale is rare.
            const bool need = mt > m_run + 8.0f;
            if (__any(need)) {
                const float alpha = need ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;
                if (need) m_run = mt;
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
            }
            const float nb = m_run == -INFINITY ? 0.f : -m_run;
            float p[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c2, nb));
            float rs = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) rs += p[r];
            l_run += rs;
            bf16x8 pf[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                u32x4 pk;
#pragma unroll
                for (int i = 0; i < 4; ++i) pk[i] = pack_bf16(p[8 * c + 2 * i], p[8 * c + 2 * i + 1]);
                pf[c] = as_bf16x8(pk);
            }

            // O^T += V^T . P^T over the block's 32 keys, two 16-key steps.
            const lds_u8* v_base = base + sub * 32 * 256;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const s16x4 lo = lds_read_tr(v_base + v_off[dt] + (16 * c) * 256);
                    const s16x4 hi = lds_read_tr(v_base + v_off[dt] + (16 * c + 8) * 256);
                    typedef short s16x8 __attribute__((ext_vector_type(8)));
                    const s16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    o[dt] = mfma32x32x16(__builtin_bit_cast(bf16x8, a), pf[c], o[dt]);
                }
            }
        }

        if (kt + 1 < nkt) {
            lstore((kt + 1) & 1);
            if (kt + 2 < nkt) gload(kt + 2);
        }
        __syncthreads();
    }

    // Epilogue: the two lane halves hold partial sums over different keys of the same query.
    const float l_tot = half_sum(l_run);
    if (qrow < T) {
        const float inv = 1.0f / l_tot;
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
}

int attn_bitmap_words(int T) { return 2 * ((T + kKT - 1) / kKT); }
int attn_bitmap_cols(int T) { return (T + kQT - 1) / kQT * kQT; }

hipError_t launch_sparse_attn(const uint16_t* q, const uint16_t* kv, const uint16_t* k_pe,
                              const uint32_t* bitmap, int B, int T, float scale, uint16_t* out,
                              hipStream_t stream) {
    const int nqt = (T + kQT - 1) / kQT;
    const float c2 = (float)((double)scale * 1.4426950408889634);   // scale * log2(e)
    const dim3 grid(B * kHeads * nqt);
    sparse_attn_kernel<<<grid, 512, 0, stream>>>(q, kv, k_pe, bitmap, T, attn_bitmap_cols(T),
                                                 attn_bitmap_words(T), nqt, c2, out);
    return hipGetLastError();
}

}  // namespace mla
