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
template <int QR>
__global__ __launch_bounds__(256) void sel_bitmap_kernel(const int32_t* __restrict__ topk, int T, int K,
                                                         int W, uint32_t* __restrict__ bitmap) {
    extern __shared__ uint32_t rows_lds[];   // QR rows of W words (+1 pad word per row)
    const int WP = W + 1;
    const int s0 = blockIdx.x * QR, b = blockIdx.y;
    const int nrows = min(QR, T - s0);
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
    for (int i = threadIdx.x; i < W * QR; i += 256) {
        const int qi = i % QR, w = i / QR;
        if (qi < nrows) bitmap[((size_t)b * W + w) * T + s0 + qi] = rows_lds[qi * WP + w];
    }
}

hipError_t launch_sel_bitmap(const int32_t* topk, int B, int T, int K, uint32_t* bitmap,
                             hipStream_t stream) {
    constexpr int QR = 8;
    const int W = (T + 31) / 32;
    const dim3 grid((T + QR - 1) / QR, B);
    const size_t lds = (size_t)QR * (W + 1) * sizeof(uint32_t);
    sel_bitmap_kernel<QR><<<grid, 256, lds, stream>>>(topk, T, K, W, bitmap);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Attention.
// ------------------------------------------------------------------------------------------------
constexpr int kKT = 64;                 // keys per LDS tile
constexpr int kKsRow = kQkHead + 8;     // 200 bf16 = 400 B per staged key row
constexpr int kVtRow = kKT + 8;         // 72 bf16 = 144 B per staged value feature row

// Position of key k (0..63) of a tile inside a V^T row: within each group of 16 keys the four
// quads are stored in the order 0, 2, 1, 3, so keys {4g..4g+3, 8+4g..8+4g+3} are contiguous.
__device__ __forceinline__ int vt_pos(int k) {
    const int quad = (k >> 2) & 3;
    const int pq = (quad == 1) ? 2 : (quad == 2) ? 1 : quad;
    return (k & ~15) + pq * 4 + (k & 3);
}

template <int QB>
__global__ __launch_bounds__(256) void sparse_attn_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ kv,
                                                          const uint16_t* __restrict__ kpe,
                                                          const uint32_t* __restrict__ bitmap, int T,
                                                          int nqt, float c2, uint16_t* __restrict__ out) {
    constexpr int QT = 4 * 32 * QB;     // queries per workgroup
    __shared__ __attribute__((aligned(16))) uint16_t Ks[kKT * kKsRow];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[kVHead * kVtRow];

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
    const int W = (T + 31) >> 5;
    const int q0 = qt * QT;
    const int wq0 = q0 + wave * 32 * QB;
    const int wq_last = min(T - 1, wq0 + 32 * QB - 1);

    const uint16_t* kvh = kv + (size_t)bh * T * 256;
    const uint16_t* kpeb = kpe + (size_t)b * T * kRope;
    const uint32_t* bmb = bitmap + (size_t)b * W * T;

    // Q^T fragments (B operand): lane holds query wq0 + 32*qb + col, features kc*16 + 8*half ...
    bf16x8 qf[QB][12];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qrow = wq0 + qb * 32 + col;
        const uint16_t* src = q + (((size_t)b * T + qrow) * kHeads + h) * kQkHead + half * 8;
#pragma unroll
        for (int kc = 0; kc < 12; ++kc)
            qf[qb][kc] = as_bf16x8(qrow < T ? load16(src + kc * 16) : u32x4{0, 0, 0, 0});
    }

    f32x16 o[QB][4];
    float m_run[QB], l_run[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[qb][dt] = f32x16{};
        m_run[qb] = -INFINITY;
        l_run[qb] = 0.f;
    }

    // Staging assignment. K: 64 keys x 24 chunks of 16 B (16 from the head's non-rotary key,
    // 8 from the shared rotary key), six chunks per thread. V: thread owns 4 consecutive keys
    // x 8 consecutive value features and writes them transposed.
    const int v_dg = tid & 15, v_kg = tid >> 4;
    const int v_dst = v_dg * 8 * kVtRow + vt_pos(v_kg * 4);
    u32x4 kst[6], vst[4];

    auto gload = [&](int t0) {
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            const int c = tid + 256 * i, key = c / 24, part = c - key * 24;
            const int t = t0 + key;
            u32x4 v = {0, 0, 0, 0};
            if (t < T) v = part < 16 ? load16(kvh + (size_t)t * 256 + part * 8)
                                     : load16(kpeb + (size_t)t * kRope + (part - 16) * 8);
            kst[i] = v;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int t = t0 + v_kg * 4 + k;
            vst[k] = t < T ? load16(kvh + (size_t)t * 256 + kNope + v_dg * 8) : u32x4{0, 0, 0, 0};
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            const int c = tid + 256 * i, key = c / 24, part = c - key * 24;
            *reinterpret_cast<u32x4*>(&Ks[key * kKsRow + part * 8]) = kst[i];
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint32_t sel = e ? 0x07060302u : 0x05040100u;
                u32x2 w;
                w[0] = __builtin_amdgcn_perm(vst[1][jj], vst[0][jj], sel);
                w[1] = __builtin_amdgcn_perm(vst[3][jj], vst[2][jj], sel);
                *reinterpret_cast<u32x2*>(&Vt[v_dst + (2 * jj + e) * kVtRow]) = w;
            }
        }
    };

    const int q_last = min(T, q0 + QT) - 1;
    const int nkt = q_last / kKT + 1;

    gload(0);
    lstore();
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
        if (kt + 1 < nkt) gload((kt + 1) * kKT);

#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int kbase = kt * kKT + sub * 32;
            if (kbase > wq_last) continue;          // every key is in this wave's future

            uint32_t word[QB];
            bool any = false;
            bool full[QB];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int qrow = wq0 + qb * 32 + col;
                word[qb] = qrow < T ? bmb[(size_t)(kbase >> 5) * T + qrow] : 0u;
                any |= __any(word[qb] != 0u);
                full[qb] = __all(word[qb] == 0xFFFFFFFFu);
            }
            if (!any) continue;                     // no query of this wave selects a key here

            // S^T block: 32 keys x 32 queries per query block.
            f32x16 s[QB];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[qb] = f32x16{};
            const uint16_t* kfrag = &Ks[(sub * 32 + col) * kKsRow + half * 8];
#pragma unroll
            for (int kc = 0; kc < 12; ++kc) {
                const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(kfrag + kc * 16));
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) s[qb] = mfma32x32x16(a, qf[qb][kc], s[qb]);
            }

            bf16x8 pf[QB][2];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                if (!full[qb]) {
                    // Accumulator r of this lane is key 8*(r/4) + 4*half + (r%4) of the block.
                    const uint32_t w = word[qb] >> (4 * half);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int bit = 8 * (r >> 2) + (r & 3);
                        s[qb][r] = ((w >> bit) & 1u) ? s[qb][r] : -INFINITY;
                    }
                }
                float mx = s[qb][0];
#pragma unroll
                for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[qb][r]);
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                const float m_new = fmaxf(m_run[qb], mx * c2);
                const float base = m_new == -INFINITY ? 0.f : m_new;
                float p[16];
                float rs = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    p[r] = __builtin_amdgcn_exp2f(fmaf(s[qb][r], c2, -base));
                    rs += p[r];
                }
                rs += __shfl_xor(rs, 32, 64);
                const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - base);
                l_run[qb] = l_run[qb] * alpha + rs;
                m_run[qb] = m_new;
                if (__any(alpha != 1.f)) {
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) o[qb][dt][r] *= alpha;
                }
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    u32x4 pk;
#pragma unroll
                    for (int i = 0; i < 4; ++i) pk[i] = pack_bf16(p[8 * c + 2 * i], p[8 * c + 2 * i + 1]);
                    pf[qb][c] = as_bf16x8(pk);
                }
            }

            // O^T += V^T . P^T over the block's 32 keys (two 16-key reduction steps).
            const uint16_t* vfrag = &Vt[col * kVtRow + sub * 32 + half * 8];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const bf16x8 a =
                        as_bf16x8(*reinterpret_cast<const u32x4*>(vfrag + dt * 32 * kVtRow + c * 16));
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) o[qb][dt] = mfma32x32x16(a, pf[qb][c], o[qb][dt]);
                }
            }
        }

        __syncthreads();
        if (kt + 1 < nkt) {
            lstore();
            __syncthreads();
        }
    }

    // Epilogue: out[b, s, h, d] = O / l; lane owns features 8g + 4*half + 0..3 of each 32 block.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qrow = wq0 + qb * 32 + col;
        if (qrow >= T) continue;
        const float inv = 1.0f / l_run[qb];
        uint16_t* dst = out + (((size_t)b * T + qrow) * kHeads + h) * kVHead;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 v;
                v[0] = pack_bf16(o[qb][dt][4 * g] * inv, o[qb][dt][4 * g + 1] * inv);
                v[1] = pack_bf16(o[qb][dt][4 * g + 2] * inv, o[qb][dt][4 * g + 3] * inv);
                store8(dst + dt * 32 + 8 * g + 4 * half, v);
            }
    }
}

hipError_t launch_sparse_attn(const uint16_t* q, const uint16_t* kv, const uint16_t* k_pe,
                              const uint32_t* bitmap, int B, int T, float scale, uint16_t* out,
                              hipStream_t stream) {
    constexpr int QB = 1;
    constexpr int QT = 4 * 32 * QB;
    const int nqt = (T + QT - 1) / QT;
    const float c2 = (float)((double)scale * 1.4426950408889634);   // scale * log2(e)
    const dim3 grid(B * kHeads * nqt);
    sparse_attn_kernel<QB><<<grid, 256, 0, stream>>>(q, kv, k_pe, bitmap, T, nqt, c2, out);
    return hipGetLastError();
}

}  // namespace mla
