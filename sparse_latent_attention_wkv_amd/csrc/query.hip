// Query RMSNorm of the query path (the two GEMMs around it are gemm_big_kernel in
// gemm_big.hip).
//
// "DeepSeek V4.1 · Key-value RMSNorm" (formula and RMSNorm excerpt): per row, the fp32 mean of
// squares, y = gain * x * rsqrt(mean + eps), cast back to bf16; "DeepSeek-V3.2-Exp · Key-value
// down-projection" (MLA constructor excerpt): q_norm is such an RMSNorm over the q_lora_rank
// features of wq_a's output (1536 here).
//
// One wave per row; lane l holds features 512k + 8l .. 512k + 8l + 7 for k < 3 (three 16-byte
// loads, each wave instruction reading 1 KB of consecutive bytes); the mean of squares is a
// 64-lane butterfly sum.
#include "mla_device.hpp"
#include "mla_launch.hpp"

namespace mla {

__global__ __launch_bounds__(256) void rms_norm_q_kernel(const uint16_t* __restrict__ qa, int rows,
                                                         const float* __restrict__ gain, float eps,
                                                         uint16_t* __restrict__ qr) {
    constexpr int PARTS = kQRank / 512;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= rows) return;
    const uint16_t* src = qa + (size_t)row * kQRank + lane * 8;
    u32x4 v[PARTS];
#pragma unroll
    for (int k = 0; k < PARTS; ++k) v[k] = load16(src + 512 * k);
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < PARTS; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float lo = bf16lo(v[k][j]), hi = bf16hi(v[k][j]);
            ss = fmaf(lo, lo, ss);
            ss = fmaf(hi, hi, ss);
        }
    ss = wave_sum(ss);
    const float rs = rsqrtf(__fdiv_rn(ss, (float)kQRank) + eps);
    uint16_t* dst = qr + (size_t)row * kQRank + lane * 8;
#pragma unroll
    for (int k = 0; k < PARTS; ++k) {
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(gain + 512 * k + lane * 8);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(gain + 512 * k + lane * 8 + 4);
        const float g[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = pack_bf16(g[2 * j] * (bf16lo(v[k][j]) * rs), g[2 * j + 1] * (bf16hi(v[k][j]) * rs));
        store16(dst + 512 * k, o);
    }
}

hipError_t launch_rms_norm_q(const uint16_t* qa, int rows, const float* gain, float eps,
                             uint16_t* qr, hipStream_t stream) {
    rms_norm_q_kernel<<<dim3((rows + 3) / 4), 256, 0, stream>>>(qa, rows, gain, eps, qr);
    return hipGetLastError();
}

}  // namespace mla
