// Latent RMSNorm and rotary rotation of the shared key (bandwidth-bound step of the front end).
//
// "DeepSeek V4.1 · Key-value RMSNorm" (formula and RMSNorm excerpt): per row, the fp32 mean of
// squares over the 512 latent features, y = gain * x * rsqrt(mean + eps), cast back to bf16.
// "DeepSeek-V3.2-Exp · Key-value down-projection" (MLA key-value excerpt): the 576-wide
// projection output splits into the 512 latent and the 64-wide rotary key; the key is rotated
// by the position's freqs_cis entry, adjacent pairs read as complex numbers.
//
// Layout: one wave per row, four rows per wave with all their loads issued before any arithmetic
// (enough bytes in flight per wave to stream at HBM rate). Lane l reads latent features
// 8l..8l+7 with one 16-byte load; lanes 0..31 also rotate pair l of the rotary key (one 4-byte
// load, one 8-byte table load). The mean of squares is a 64-lane butterfly sum.
#include "mla_device.hpp"
#include "mla_launch.hpp"

namespace mla {

template <bool ROPE, int ROWS_PER_WAVE>
__global__ __launch_bounds__(256) void norm_rope_kernel(const uint16_t* __restrict__ src, int rows,
                                                        int stride, const float* __restrict__ gain,
                                                        float eps, const float* __restrict__ rope_cs,
                                                        int T, uint16_t* __restrict__ c_kv,
                                                        uint16_t* __restrict__ k_pe) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row0 = (blockIdx.x * 4 + wave) * ROWS_PER_WAVE;

    // Issue every load of this wave's rows before any arithmetic.
    u32x4 v[ROWS_PER_WAVE];
    uint32_t pe[ROWS_PER_WAVE];
    float2 cs[ROWS_PER_WAVE];
#pragma unroll
    for (int i = 0; i < ROWS_PER_WAVE; ++i) {
        const int row = row0 + i;
        if (row < rows) {
            const uint16_t* r = src + (size_t)row * stride;
            v[i] = load16(r + lane * 8);
            if (ROPE && lane < 32) {
                pe[i] = *reinterpret_cast<const uint32_t*>(r + kLora + 2 * lane);
                cs[i] = *reinterpret_cast<const float2*>(rope_cs + ((size_t)(row % T) * 32 + lane) * 2);
            }
        }
    }
    const f32x4 g0 = *reinterpret_cast<const f32x4*>(gain + lane * 8);
    const f32x4 g1 = *reinterpret_cast<const f32x4*>(gain + lane * 8 + 4);
    const float g[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};

#pragma unroll
    for (int i = 0; i < ROWS_PER_WAVE; ++i) {
        const int row = row0 + i;
        if (row >= rows) break;
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
        const float ms = ss * (1.0f / kLora);
        const float rs = rsqrtf(ms + eps);
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = pack_bf16(g[2 * j] * (x[2 * j] * rs), g[2 * j + 1] * (x[2 * j + 1] * rs));
        store16(c_kv + (size_t)row * kLora + lane * 8, o);
        if (ROPE && lane < 32) {
            const float re = bf16lo(pe[i]), im = bf16hi(pe[i]);
            const float c = cs[i].x, s = cs[i].y;
            const float ore = re * c - im * s;
            const float oim = re * s + im * c;
            *reinterpret_cast<uint32_t*>(k_pe + (size_t)row * kRope + 2 * lane) = pack_bf16(ore, oim);
        }
    }
}

hipError_t launch_norm_rope(const uint16_t* src, int rows, int stride, bool rope, const float* gain,
                            float eps, const float* rope_cs, int T, uint16_t* c_kv, uint16_t* k_pe,
                            hipStream_t stream) {
    constexpr int R = 4;
    const int per_block = 4 * R;
    const dim3 grid((rows + per_block - 1) / per_block);
    if (rope)
        norm_rope_kernel<true, R><<<grid, 256, 0, stream>>>(src, rows, stride, gain, eps, rope_cs, T,
                                                            c_kv, k_pe);
    else
        norm_rope_kernel<false, R><<<grid, 256, 0, stream>>>(src, rows, stride, gain, eps, rope_cs,
                                                             T, c_kv, k_pe);
    return hipGetLastError();
}

// Rotary table: (cos, sin) of t * theta^(-2i/64), evaluated in fp64 and rounded to fp32.
__global__ __launch_bounds__(256) void rope_table_kernel(int T, double theta, float* __restrict__ cs) {
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= T * 32) return;
    const int t = idx >> 5, i = idx & 31;
    const double inv_freq = pow(theta, -2.0 * i / 64.0);
    const double phi = (double)t * inv_freq;
    double s, c;
    sincos(phi, &s, &c);
    cs[2 * idx] = (float)c;
    cs[2 * idx + 1] = (float)s;
}

hipError_t launch_rope_table(int T, double theta, float* rope_cs, hipStream_t stream) {
    const int n = T * 32;
    rope_table_kernel<<<(n + 255) / 256, 256, 0, stream>>>(T, theta, rope_cs);
    return hipGetLastError();
}

}  // namespace mla
