// FP8 round trip of the latent and the key-value cache writes, fused into the norm/rotary pass;
// the V4.1 window-KV front end (norm, rotary tail, round trip, ring buffer) in the same kernel.
//
// "DeepSeek-V3.2-Exp · Key-value down-projection", KV-cache evidence: each call passes the
// normalised latent through a block fp8 quantiser (blocks of 128 features) and back — the fp8
// values times their block's scale in float, cast to bf16 — and stores it with the rotated key
// in two caches at the call's positions; the up-projection then consumes the rounded latent.
// "DeepSeek V4.1 · Key-value RMSNorm", window-KV excerpt: RMSNorm (eps 1e-20) of the 512-wide
// projection output, rotary on its last 64 features, the same round trip over the whole vector,
// then a ring buffer of `window` positions, position p in slot p mod window.
//
// The quantiser's body is not on the pages. This one: e4m3 (largest finite value 448); block
// scale s = amax / 448 in fp32, or that rounded up to a power of two; code = the e4m3 value
// nearest to x / s (the correctly rounded fp32 quotient), ties to the even code; result
// bf16(code * s). A block of zeros keeps scale 1. x / s can exceed 448 by one rounding of the
// division; it then rounds to 448 (464 is the midpoint to the grid's next step, the NaN code).
//
// Layout: one wave per row; on large calls four rows per wave with every load issued before any
// arithmetic (the norm/rotary kernel's scheme), on decode-sized calls one. Lane l holds features 8l..8l+7, so one 128-feature block is a
// group of 16 lanes and its largest magnitude is a 4-step exchange inside the group. One pass
// reads the projection output once and writes the rounded latent, the rotated key and the cache
// rows (plus, if asked, the vector before the round trip).
#include "mla_device.hpp"
#include "mla_launch.hpp"

namespace mla {

// Correctly rounded fp32 quotient x / s from rc = RN(1 / s), the block's reciprocal: two
// correction steps with exact remainders (fma). The first turns x * rc (within 1.5 ulp) into a
// quotient within half an ulp plus a negligible amount, i.e. a faithful one; from a faithful
// quotient and the correctly rounded reciprocal, one more step gives the correctly rounded
// quotient (Markstein's theorem on division by fused multiply-add). Valid while nothing over- or
// underflows: callers keep s >= 2^-100, and |x / s| <= 464; quotients in the fp32 subnormal range
// are far below the smallest e4m3 step and become code 0 either way. The remainder steps turn a
// quotient of -0 into +0; the sign of x (s > 0) is put back, as the division keeps it.
__device__ __forceinline__ float quotient_rn(float x, float s, float rc) {
    const float y0 = x * rc;
    const float y1 = fmaf(fmaf(-s, y0, x), rc, y0);
    return copysignf(fmaf(fmaf(-s, y1, x), rc, y1), x);
}

// Two quotients to their nearest e4m3 values (round to nearest even, the finite-only e4m3 format
// of the gfx950 conversion instructions), dequantised with the block scale and packed to bf16.
__device__ __forceinline__ uint32_t e4m3_round_trip2(float q0, float q1, float sc) {
    const int p = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
    return pack_bf16(__builtin_amdgcn_cvt_f32_fp8(p, 0) * sc, __builtin_amdgcn_cvt_f32_fp8(p, 1) * sc);
}

// Block scale from the block's largest magnitude: amax / 448 (fp32), or the smallest power of
// two not below it; 1 for a block of zeros.
__device__ __forceinline__ float fp8_block_scale(float amax, int pow2) {
    if (amax == 0.0f) return 1.0f;
    // RN(amax / 448) from the correctly rounded constant RN(1 / 448); amax is a bf16 value of at
    // least 2^-133, far from over- and underflow of the quotient's steps.
    const float s = quotient_rn(amax, 448.0f, 1.0f / 448.0f);
    if (!pow2) return s;
    int e;
    const float m = frexpf(s, &e);    // s = m * 2^e, 0.5 <= m < 1
    return m == 0.5f ? s : ldexpf(1.0f, e);
}

struct Fp8FrontArgs {
    const uint16_t* src;     // [rows][stride]: 576 (latent | rotary key) or 512 (window form)
    int rows, stride;
    int T;                   // positions per batch row; row r is batch r / T, position start + r % T
    int start_pos;
    const float* gain;       // [512]
    float eps;
    const float* rope_cs;    // [positions][32][2] (cos, sin) by absolute position
    int pow2_scale;
    uint16_t* out;           // [rows][512] after the round trip
    uint16_t* pre;           // [rows][512] before it, or null
    uint16_t* k_pe;          // [rows][64] rotated key (latent form)
    uint16_t* cache;         // latent form [.][cache_len][512]; window form [.][cache_len][512]
    uint16_t* pe_cache;      // latent form [.][cache_len][64]
    int cache_len;           // latent form: positions per cache row; window form: the window
};

template <bool WINDOW, int RPW>
__global__ __launch_bounds__(256) void fp8_front_kernel(Fp8FrontArgs A) {
    const int lane = threadIdx.x & 63;
    // wave-uniform, so the row arithmetic below stays in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row0 = (blockIdx.x * 4 + wave) * RPW;
    // Window form: lanes 56..63 hold the rotary tail (features 448..511), four pairs each.
    const bool tail = WINDOW && lane >= 56;

    u32x4 v[RPW];
    uint32_t pe[RPW];
    float2 cs[RPW];
    f32x4 cw[RPW][2];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int row = row0 + i;
        if (row < A.rows) {
            const uint16_t* r = A.src + (size_t)row * A.stride;
            v[i] = load16(r + lane * 8);
            const size_t pos = (size_t)A.start_pos + (row % A.T);
            if (!WINDOW && lane < 32) {
                pe[i] = *reinterpret_cast<const uint32_t*>(r + kLora + 2 * lane);
                cs[i] = *reinterpret_cast<const float2*>(A.rope_cs + (pos * 32 + lane) * 2);
            }
            if (tail) {
                const float* c = A.rope_cs + (pos * 32 + 4 * (lane - 56)) * 2;
                cw[i][0] = *reinterpret_cast<const f32x4*>(c);
                cw[i][1] = *reinterpret_cast<const f32x4*>(c + 4);
            }
        }
    }
    const f32x4 g0 = *reinterpret_cast<const f32x4*>(A.gain + lane * 8);
    const f32x4 g1 = *reinterpret_cast<const f32x4*>(A.gain + lane * 8 + 4);
    const float g[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};

#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int row = row0 + i;
        if (row >= A.rows) break;
        float x[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = bf16lo(v[i][j]);
            x[2 * j + 1] = bf16hi(v[i][j]);
        }
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) ss = fmaf(x[j], x[j], ss);
        ss = wave_sum(ss);
        const float rs = rsqrtf(ss * (1.0f / kLora) + A.eps);
        // The normalised vector in bf16 (the norm's output dtype), then the rotary tail.
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = pack_bf16(g[2 * j] * (x[2 * j] * rs), g[2 * j + 1] * (x[2 * j + 1] * rs));
        if (tail) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float re = bf16lo(o[j]), im = bf16hi(o[j]);
                const float c = cw[i][j >> 1][2 * (j & 1)], s = cw[i][j >> 1][2 * (j & 1) + 1];
                o[j] = pack_bf16(re * c - im * s, re * s + im * c);
            }
        }
        if (A.pre) store16(A.pre + (size_t)row * kLora + lane * 8, o);

        // Block fp8 round trip: largest magnitude over the 16 lanes of the block, scale,
        // quantise, dequantise.
        float y[8];
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            y[2 * j] = bf16lo(o[j]);
            y[2 * j + 1] = bf16hi(o[j]);
            amax = fmaxf(amax, fmaxf(fabsf(y[2 * j]), fabsf(y[2 * j + 1])));
        }
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
        const float sc = fp8_block_scale(amax, A.pow2_scale);
        float q[8];
        if (sc >= 0x1p-100f) {
            const float rc = __fdiv_rn(1.0f, sc);
#pragma unroll
            for (int j = 0; j < 8; ++j) q[j] = quotient_rn(y[j], sc, rc);
        } else {    // blocks whose largest magnitude is below ~2^-91: plain division
#pragma unroll
            for (int j = 0; j < 8; ++j) q[j] = __fdiv_rn(y[j], sc);
        }
        u32x4 d;
#pragma unroll
        for (int j = 0; j < 4; ++j) d[j] = e4m3_round_trip2(q[2 * j], q[2 * j + 1], sc);
        store16(A.out + (size_t)row * kLora + lane * 8, d);

        const int b = row / A.T, t = row - b * A.T;
        if (!WINDOW) {
            const size_t crow = (size_t)b * A.cache_len + A.start_pos + t;
            store16(A.cache + crow * kLora + lane * 8, d);
            if (lane < 32) {
                const float re = bf16lo(pe[i]), im = bf16hi(pe[i]);
                const float c = cs[i].x, s = cs[i].y;
                const uint32_t k = pack_bf16(re * c - im * s, re * s + im * c);
                *reinterpret_cast<uint32_t*>(A.k_pe + (size_t)row * kRope + 2 * lane) = k;
                *reinterpret_cast<uint32_t*>(A.pe_cache + crow * kRope + 2 * lane) = k;
            }
        } else if (t >= A.T - A.cache_len) {
            // Only the last `window` positions of the call reach the ring buffer.
            const int slot = (int)(((size_t)A.start_pos + t) % (size_t)A.cache_len);
            store16(A.cache + ((size_t)b * A.cache_len + slot) * kLora + lane * 8, d);
        }
    }
}

namespace {
// Four rows per wave keep enough loads in flight to stream at HBM rate on large calls; below
// 16K rows (decode-sized calls) one row per wave spreads the work over more of the chip, which
// shortens the call.
template <bool WINDOW>
hipError_t launch_fp8_front(const Fp8FrontArgs& a, hipStream_t stream) {
    if (a.rows >= 16384) {
        constexpr int R = 4;
        fp8_front_kernel<WINDOW, R><<<dim3((a.rows + 4 * R - 1) / (4 * R)), 256, 0, stream>>>(a);
    } else {
        fp8_front_kernel<WINDOW, 1><<<dim3((a.rows + 3) / 4), 256, 0, stream>>>(a);
    }
    return hipGetLastError();
}
}  // namespace

hipError_t launch_kv_norm_rope_cache(const uint16_t* kv_raw, int B, int T, int start_pos,
                                     const float* gain, float eps, const float* rope_cs,
                                     int pow2_scale, uint16_t* c_kv, uint16_t* c_norm,
                                     uint16_t* k_pe, uint16_t* kv_cache, uint16_t* pe_cache,
                                     int cache_len, hipStream_t stream) {
    Fp8FrontArgs a{kv_raw, B * T, kKvAOut, T, start_pos, gain, eps, rope_cs, pow2_scale,
                   c_kv, c_norm, k_pe, kv_cache, pe_cache, cache_len};
    return launch_fp8_front<false>(a, stream);
}

hipError_t launch_window_kv(const uint16_t* kv_raw, int B, int S, int start_pos, const float* gain,
                            float eps, const float* rope_cs, int pow2_scale, int window,
                            uint16_t* out, uint16_t* pre, uint16_t* cache, hipStream_t stream) {
    Fp8FrontArgs a{kv_raw, B * S, kLora, S, start_pos, gain, eps, rope_cs, pow2_scale,
                   out, pre, nullptr, cache, nullptr, window};
    return launch_fp8_front<true>(a, stream);
}

}  // namespace mla
