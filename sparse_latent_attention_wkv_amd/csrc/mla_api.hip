// C ABI of libmla.so (declared in include/mla.h): argument validation, the device check and the
// kernel sequence of each call. Validation happens before any HIP call, so a rejected call has
// no side effects.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/mla.h"
#include "mla_launch.hpp"

namespace {

thread_local int g_last_hip_error = 0;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
    const void* p;
    size_t bytes;
};

bool overlap(Span a, Span b) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// True if any output overlaps any other span (inputs or outputs).
bool any_alias(const Span* outs, int nout, const Span* ins, int nin) {
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j)
            if (overlap(outs[i], ins[j])) return true;
        for (int j = i + 1; j < nout; ++j)
            if (overlap(outs[i], outs[j])) return true;
    }
    return false;
}

bool pos_finite(float v) { return isfinite(v) && v > 0.f; }

// Per-device cache of "is this a gfx950": 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

int check_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0) {
        g_last_hip_error = (int)e;
        return MLA_E_DEVICE;
    }
    if (dev < kMaxDevices) {
        const int c = g_arch_ok[dev].load(std::memory_order_relaxed);
        if (c == 1) return MLA_OK;
        if (c == 2) return MLA_E_DEVICE;
    }
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return MLA_E_DEVICE;
    }
    const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? MLA_OK : MLA_E_DEVICE;
}

int launched(hipError_t e) {
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return MLA_E_LAUNCH;
    }
    return MLA_OK;
}

constexpr size_t kBf16 = 2;

int validate_norm_rope(const void* kv_raw, int rows, int row_stride, int has_rope, const float* gain,
                       float eps, const float* rope_cs, int T, const void* c_kv, const void* k_pe) {
    if (!kv_raw || !gain || !c_kv) return MLA_E_NULL;
    if (has_rope && (!rope_cs || !k_pe)) return MLA_E_NULL;
    if (rows < 1 || rows > MLA_MAX_ROWS) return MLA_E_SHAPE;
    if (row_stride != MLA_KV_A_OUT && row_stride != MLA_KV_LORA) return MLA_E_SHAPE;
    if (has_rope && (row_stride != MLA_KV_A_OUT || T < 1 || T > MLA_MAX_ROWS)) return MLA_E_SHAPE;
    if (!aligned16(kv_raw) || !aligned16(gain) || !aligned16(c_kv)) return MLA_E_ALIGN;
    if (has_rope && (!aligned16(rope_cs) || !aligned16(k_pe))) return MLA_E_ALIGN;
    if (!pos_finite(eps)) return MLA_E_ARG;
    const Span ins[] = {{kv_raw, (size_t)rows * row_stride * kBf16},
                        {gain, MLA_KV_LORA * sizeof(float)},
                        {rope_cs, has_rope ? (size_t)T * 64 * sizeof(float) : 0}};
    const Span outs[] = {{c_kv, (size_t)rows * MLA_KV_LORA * kBf16},
                         {k_pe, has_rope ? (size_t)rows * MLA_ROPE * kBf16 : 0}};
    if (any_alias(outs, 2, ins, 3)) return MLA_E_ALIAS;
    return MLA_OK;
}

// Checks shared by the cached front end and the window form: B*T rows at positions
// start_pos..start_pos+T-1, the rotary table covering them, the scale format.
int validate_positions(int B, int T, int start_pos, int scale_fmt, float eps) {
    if (B < 1 || T < 1 || (size_t)B * T > (size_t)MLA_MAX_ROWS) return MLA_E_SHAPE;
    if (start_pos < 0 || (int64_t)start_pos + T > (int64_t)MLA_MAX_ROWS) return MLA_E_SHAPE;
    if (!pos_finite(eps) || (scale_fmt != 0 && scale_fmt != 1)) return MLA_E_ARG;
    return MLA_OK;
}

int validate_norm_rope_cache(const void* kv_raw, int B, int T, int start_pos, const float* gain,
                             float eps, const float* rope_cs, int scale_fmt, const void* c_kv,
                             const void* k_pe, const void* kv_cache, const void* pe_cache,
                             int cache_batch, int cache_len, const void* c_norm,
                             bool kv_raw_is_output) {
    if (!kv_raw || !gain || !rope_cs || !c_kv || !k_pe || !kv_cache || !pe_cache) return MLA_E_NULL;
    int st = validate_positions(B, T, start_pos, scale_fmt, eps);
    if (st != MLA_OK) return st;
    if (cache_batch < B || cache_len < 1 || (int64_t)start_pos + T > cache_len) return MLA_E_SHAPE;
    if (!aligned16(kv_raw) || !aligned16(gain) || !aligned16(rope_cs) || !aligned16(c_kv) ||
        !aligned16(k_pe) || !aligned16(kv_cache) || !aligned16(pe_cache) ||
        (c_norm && !aligned16(c_norm)))
        return MLA_E_ALIGN;
    const size_t M = (size_t)B * T;
    const Span raw = {kv_raw, M * MLA_KV_A_OUT * kBf16};
    const Span ins[] = {raw,
                        {gain, MLA_KV_LORA * sizeof(float)},
                        {rope_cs, (size_t)(start_pos + T) * 64 * sizeof(float)}};
    const Span outs[] = {{c_kv, M * MLA_KV_LORA * kBf16},
                         {k_pe, M * MLA_ROPE * kBf16},
                         {kv_cache, (size_t)cache_batch * cache_len * MLA_KV_LORA * kBf16},
                         {pe_cache, (size_t)cache_batch * cache_len * MLA_ROPE * kBf16},
                         {c_norm, c_norm ? M * MLA_KV_LORA * kBf16 : 0},
                         {kv_raw_is_output ? kv_raw : nullptr, kv_raw_is_output ? raw.bytes : 0}};
    // kv_raw is an input of the norm step; when the call also produces it, it counts as an
    // output (checked against every other buffer) instead.
    if (any_alias(outs, 6, kv_raw_is_output ? ins + 1 : ins, kv_raw_is_output ? 2 : 3))
        return MLA_E_ALIAS;
    return MLA_OK;
}

int validate_topk(const int32_t* topk, int B, int T, int K) {
    if (!topk) return MLA_E_NULL;
    if (B < 1 || T < 1 || K < 1 || T > MLA_MAX_T || K > 65536) return MLA_E_SHAPE;
    if ((size_t)B * T > (size_t)MLA_MAX_ROWS) return MLA_E_SHAPE;
    if (!aligned16(topk)) return MLA_E_ALIGN;
    return MLA_OK;
}

// Selection data as the attention kernel reads it: the bitmap (padded so every staged tile is in
// bounds) and the key-tile flags.
size_t attn_bitmap_bytes(int B, int T) { return mla::attn_select_bytes(B, T); }
// Bitmap as mla_selection_bitmap returns it, [B][ceil(T/32)][T].
size_t plain_bitmap_bytes(int B, int T) { return (size_t)B * ((T + 31) / 32) * T * sizeof(uint32_t); }

// Scratch of mla_sparse_prefill_attn_noalloc: the selection bitmap and key-tile flags live in this fixed array
// instead of a caller workspace. Each device holds its own copy for the life of the process. In
// host code `scratch` names a host-side stand-in, not the device copy: the device address comes
// from hipGetSymbolAddress, once per device, and only that address is handed to kernels.
constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) uint32_t scratch[kScratchBytes / sizeof(uint32_t)];

std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];

// Device address of this device's scratch (the current device), or nullptr on failure.
void* scratch_address(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            g_last_hip_error = (int)e;
            return nullptr;
        }
        g_scratch_dev[dev] = p;
    }
    return g_scratch_dev[dev];
}

}  // namespace

extern "C" {

int mla_kv_norm_rope(const void* kv_raw, int rows, int row_stride, int has_rope, const float* gain,
                     float eps, const float* rope_cs, int T, void* c_kv, void* k_pe, void* stream) {
    int st = validate_norm_rope(kv_raw, rows, row_stride, has_rope, gain, eps, rope_cs, T, c_kv, k_pe);
    if (st != MLA_OK) return st;
    if ((st = check_device()) != MLA_OK) return st;
    return launched(mla::launch_norm_rope(static_cast<const uint16_t*>(kv_raw), rows, row_stride,
                                          has_rope != 0, gain, eps, rope_cs, has_rope ? T : 1,
                                          static_cast<uint16_t*>(c_kv), static_cast<uint16_t*>(k_pe),
                                          static_cast<hipStream_t>(stream)));
}

int mla_kv_latent(const void* x, const void* w_dkv, const float* kv_gain, float eps,
                  const float* rope_cs, int B, int T, void* kv_raw, void* c_kv, void* k_pe,
                  void* stream) {
    if (!x || !w_dkv || !kv_gain || !rope_cs || !kv_raw || !c_kv || !k_pe) return MLA_E_NULL;
    if (B < 1 || T < 1 || (size_t)B * T > (size_t)MLA_MAX_ROWS) return MLA_E_SHAPE;
    if (!aligned16(x) || !aligned16(w_dkv) || !aligned16(kv_gain) || !aligned16(rope_cs) ||
        !aligned16(kv_raw) || !aligned16(c_kv) || !aligned16(k_pe))
        return MLA_E_ALIGN;
    if (!pos_finite(eps)) return MLA_E_ARG;
    const size_t M = (size_t)B * T;
    const Span ins[] = {{x, M * MLA_HIDDEN * kBf16},
                        {w_dkv, (size_t)MLA_KV_A_OUT * MLA_HIDDEN * kBf16},
                        {kv_gain, MLA_KV_LORA * sizeof(float)},
                        {rope_cs, (size_t)T * 64 * sizeof(float)}};
    const Span outs[] = {{kv_raw, M * MLA_KV_A_OUT * kBf16},
                         {c_kv, M * MLA_KV_LORA * kBf16},
                         {k_pe, M * MLA_ROPE * kBf16}};
    if (any_alias(outs, 3, ins, 4)) return MLA_E_ALIAS;
    int st = check_device();
    if (st != MLA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = launched(mla::launch_gemm_kv_down(static_cast<const uint16_t*>(x),
                                           static_cast<const uint16_t*>(w_dkv), (int)M,
                                           static_cast<uint16_t*>(kv_raw), s));
    if (st != MLA_OK) return st;
    return launched(mla::launch_norm_rope(static_cast<const uint16_t*>(kv_raw), (int)M, MLA_KV_A_OUT,
                                          true, kv_gain, eps, rope_cs, T, static_cast<uint16_t*>(c_kv),
                                          static_cast<uint16_t*>(k_pe), s));
}

int mla_kv_norm_rope_cache(const void* kv_raw, int B, int T, int start_pos, const float* gain,
                           float eps, const float* rope_cs, int scale_fmt, void* c_kv, void* k_pe,
                           void* kv_cache, void* pe_cache, int cache_batch, int cache_len,
                           void* c_norm, void* stream) {
    int st = validate_norm_rope_cache(kv_raw, B, T, start_pos, gain, eps, rope_cs, scale_fmt, c_kv,
                                      k_pe, kv_cache, pe_cache, cache_batch, cache_len, c_norm,
                                      false);
    if (st != MLA_OK) return st;
    if ((st = check_device()) != MLA_OK) return st;
    return launched(mla::launch_kv_norm_rope_cache(
        static_cast<const uint16_t*>(kv_raw), B, T, start_pos, gain, eps, rope_cs, scale_fmt,
        static_cast<uint16_t*>(c_kv), static_cast<uint16_t*>(c_norm), static_cast<uint16_t*>(k_pe),
        static_cast<uint16_t*>(kv_cache), static_cast<uint16_t*>(pe_cache), cache_len,
        static_cast<hipStream_t>(stream)));
}

int mla_kv_latent_cache(const void* x, const void* w_dkv, const float* kv_gain, float eps,
                        const float* rope_cs, int B, int T, int start_pos, int scale_fmt,
                        void* kv_raw, void* c_kv, void* k_pe, void* kv_cache, void* pe_cache,
                        int cache_batch, int cache_len, void* c_norm, void* stream) {
    if (!x || !w_dkv) return MLA_E_NULL;
    int st = validate_norm_rope_cache(kv_raw, B, T, start_pos, kv_gain, eps, rope_cs, scale_fmt,
                                      c_kv, k_pe, kv_cache, pe_cache, cache_batch, cache_len,
                                      c_norm, true);
    if (st != MLA_OK) return st;
    if (!aligned16(x) || !aligned16(w_dkv)) return MLA_E_ALIGN;
    const size_t M = (size_t)B * T;
    // The weights and activations must not overlap any output either.
    const Span ins[] = {{x, M * MLA_HIDDEN * kBf16},
                        {w_dkv, (size_t)MLA_KV_A_OUT * MLA_HIDDEN * kBf16}};
    const Span outs[] = {{kv_raw, M * MLA_KV_A_OUT * kBf16},
                         {c_kv, M * MLA_KV_LORA * kBf16},
                         {k_pe, M * MLA_ROPE * kBf16},
                         {kv_cache, (size_t)cache_batch * cache_len * MLA_KV_LORA * kBf16},
                         {pe_cache, (size_t)cache_batch * cache_len * MLA_ROPE * kBf16},
                         {c_norm, c_norm ? M * MLA_KV_LORA * kBf16 : 0}};
    if (any_alias(outs, 6, ins, 2)) return MLA_E_ALIAS;
    if ((st = check_device()) != MLA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = launched(mla::launch_gemm_kv_down(static_cast<const uint16_t*>(x),
                                           static_cast<const uint16_t*>(w_dkv), (int)M,
                                           static_cast<uint16_t*>(kv_raw), s));
    if (st != MLA_OK) return st;
    return launched(mla::launch_kv_norm_rope_cache(
        static_cast<const uint16_t*>(kv_raw), B, T, start_pos, kv_gain, eps, rope_cs, scale_fmt,
        static_cast<uint16_t*>(c_kv), static_cast<uint16_t*>(c_norm), static_cast<uint16_t*>(k_pe),
        static_cast<uint16_t*>(kv_cache), static_cast<uint16_t*>(pe_cache), cache_len, s));
}

int mla_window_kv(const void* kv_raw, int B, int S, int start_pos, const float* gain, float eps,
                  const float* rope_cs, int scale_fmt, int window, void* kv_out,
                  void* window_cache, int cache_batch, void* kv_pre, void* stream) {
    if (!kv_raw || !gain || !rope_cs || !kv_out || !window_cache) return MLA_E_NULL;
    int st = validate_positions(B, S, start_pos, scale_fmt, eps);
    if (st != MLA_OK) return st;
    if (window < 1 || cache_batch < B) return MLA_E_SHAPE;
    if ((size_t)cache_batch * window > (size_t)MLA_MAX_ROWS) return MLA_E_SHAPE;
    if (!aligned16(kv_raw) || !aligned16(gain) || !aligned16(rope_cs) || !aligned16(kv_out) ||
        !aligned16(window_cache) || (kv_pre && !aligned16(kv_pre)))
        return MLA_E_ALIGN;
    const size_t M = (size_t)B * S;
    const Span ins[] = {{kv_raw, M * MLA_KV_LORA * kBf16},
                        {gain, MLA_KV_LORA * sizeof(float)},
                        {rope_cs, (size_t)(start_pos + S) * 64 * sizeof(float)}};
    const Span outs[] = {{kv_out, M * MLA_KV_LORA * kBf16},
                         {window_cache, (size_t)cache_batch * window * MLA_KV_LORA * kBf16},
                         {kv_pre, kv_pre ? M * MLA_KV_LORA * kBf16 : 0}};
    if (any_alias(outs, 3, ins, 3)) return MLA_E_ALIAS;
    if ((st = check_device()) != MLA_OK) return st;
    return launched(mla::launch_window_kv(
        static_cast<const uint16_t*>(kv_raw), B, S, start_pos, gain, eps, rope_cs, scale_fmt, window,
        static_cast<uint16_t*>(kv_out), static_cast<uint16_t*>(kv_pre),
        static_cast<uint16_t*>(window_cache), static_cast<hipStream_t>(stream)));
}

int mla_q_path(const void* x, const void* w_qa, const float* q_gain, float eps, const void* w_qb,
               const float* rope_cs, int B, int T, int start_pos, int q_rank, void* qa, void* qr,
               void* q, void* stream) {
    if (!x || !w_qa || !q_gain || !w_qb || !rope_cs || !qa || !qr || !q) return MLA_E_NULL;
    int st = validate_positions(B, T, start_pos, 0, eps);
    if (st != MLA_OK) return st;
    if (q_rank != MLA_Q_LORA) return MLA_E_SHAPE;
    if (!aligned16(x) || !aligned16(w_qa) || !aligned16(q_gain) || !aligned16(w_qb) ||
        !aligned16(rope_cs) || !aligned16(qa) || !aligned16(qr) || !aligned16(q))
        return MLA_E_ALIGN;
    const size_t M = (size_t)B * T;
    const Span ins[] = {{x, M * MLA_HIDDEN * kBf16},
                        {w_qa, (size_t)MLA_Q_LORA * MLA_HIDDEN * kBf16},
                        {q_gain, MLA_Q_LORA * sizeof(float)},
                        {w_qb, (size_t)MLA_HEADS * MLA_QK_HEAD * MLA_Q_LORA * kBf16},
                        {rope_cs, (size_t)(start_pos + T) * 64 * sizeof(float)}};
    const Span outs[] = {{qa, M * MLA_Q_LORA * kBf16},
                         {qr, M * MLA_Q_LORA * kBf16},
                         {q, M * MLA_HEADS * MLA_QK_HEAD * kBf16}};
    if (any_alias(outs, 3, ins, 5)) return MLA_E_ALIAS;
    if ((st = check_device()) != MLA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = launched(mla::launch_gemm_q_a(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_qa),
                                       (int)M, static_cast<uint16_t*>(qa), s));
    if (st != MLA_OK) return st;
    st = launched(mla::launch_rms_norm_q(static_cast<const uint16_t*>(qa), (int)M, q_gain, eps,
                                         static_cast<uint16_t*>(qr), s));
    if (st != MLA_OK) return st;
    return launched(mla::launch_gemm_q_b_rope(static_cast<const uint16_t*>(qr),
                                              static_cast<const uint16_t*>(w_qb), (int)M,
                                              static_cast<uint16_t*>(q), rope_cs, T, start_pos, s));
}

int mla_rope_table(int T, float theta, float* rope_cs, void* stream) {
    if (!rope_cs) return MLA_E_NULL;
    if (T < 1 || T > MLA_MAX_ROWS) return MLA_E_SHAPE;
    if (!aligned16(rope_cs)) return MLA_E_ALIGN;
    if (!pos_finite(theta)) return MLA_E_ARG;
    int st = check_device();
    if (st != MLA_OK) return st;
    return launched(mla::launch_rope_table(T, (double)theta, rope_cs, static_cast<hipStream_t>(stream)));
}

int mla_kv_up(const void* c_kv, const void* w_ukv, int B, int T, void* kv, void* stream) {
    if (!c_kv || !w_ukv || !kv) return MLA_E_NULL;
    if (B < 1 || T < 1 || (size_t)B * T > (size_t)MLA_MAX_ROWS) return MLA_E_SHAPE;
    if (!aligned16(c_kv) || !aligned16(w_ukv) || !aligned16(kv)) return MLA_E_ALIGN;
    const size_t M = (size_t)B * T;
    const Span ins[] = {{c_kv, M * MLA_KV_LORA * kBf16}, {w_ukv, (size_t)MLA_KV_B_OUT * MLA_KV_LORA * kBf16}};
    const Span outs[] = {{kv, M * MLA_KV_B_OUT * kBf16}};
    if (any_alias(outs, 1, ins, 2)) return MLA_E_ALIAS;
    int st = check_device();
    if (st != MLA_OK) return st;
    return launched(mla::launch_gemm_kv_up(static_cast<const uint16_t*>(c_kv),
                                           static_cast<const uint16_t*>(w_ukv), B, T,
                                           static_cast<uint16_t*>(kv), static_cast<hipStream_t>(stream)));
}

size_t mla_attn_workspace_bytes(int B, int T, int K) {
    if (validate_topk(reinterpret_cast<const int32_t*>(16), B, T, K) != MLA_OK) return 0;
    return (attn_bitmap_bytes(B, T) + 255) & ~(size_t)255;
}

int mla_selection_bitmap(const int32_t* topk, int B, int T, int K, uint32_t* bitmap, void* stream) {
    int st = validate_topk(topk, B, T, K);
    if (st != MLA_OK) return st;
    if (!bitmap) return MLA_E_NULL;
    if (!aligned16(bitmap)) return MLA_E_ALIGN;
    const Span ins[] = {{topk, (size_t)B * T * K * sizeof(int32_t)}};
    const Span outs[] = {{bitmap, plain_bitmap_bytes(B, T)}};
    if (any_alias(outs, 1, ins, 1)) return MLA_E_ALIAS;
    if ((st = check_device()) != MLA_OK) return st;
    return launched(mla::launch_sel_bitmap(topk, B, T, K, (T + 31) / 32, T, bitmap,
                                           static_cast<hipStream_t>(stream)));
}

int mla_attn_prepare(const int32_t* topk, int B, int T, int K, void* workspace, size_t ws_bytes,
                     void* stream) {
    int st = validate_topk(topk, B, T, K);
    if (st != MLA_OK) return st;
    if (!workspace) return MLA_E_NULL;
    if (!aligned16(workspace)) return MLA_E_ALIGN;
    if (ws_bytes < attn_bitmap_bytes(B, T)) return MLA_E_WORKSPACE;
    const Span ins[] = {{topk, (size_t)B * T * K * sizeof(int32_t)}};
    const Span outs[] = {{workspace, attn_bitmap_bytes(B, T)}};
    if (any_alias(outs, 1, ins, 1)) return MLA_E_ALIAS;
    if ((st = check_device()) != MLA_OK) return st;
    return launched(mla::launch_attn_select(topk, B, T, K, static_cast<uint32_t*>(workspace),
                                            static_cast<hipStream_t>(stream)));
}

namespace {
int validate_attn_prepared(const void* q, const void* kv, const void* k_pe, int B, int T,
                           float softmax_scale, const void* out, const void* workspace,
                           size_t ws_bytes) {
    if (!q || !kv || !k_pe || !out || !workspace) return MLA_E_NULL;
    if (B < 1 || T < 1 || T > MLA_MAX_T || (size_t)B * T > (size_t)MLA_MAX_ROWS) return MLA_E_SHAPE;
    if (!aligned16(q) || !aligned16(kv) || !aligned16(k_pe) || !aligned16(out) || !aligned16(workspace))
        return MLA_E_ALIGN;
    if (!pos_finite(softmax_scale)) return MLA_E_ARG;
    if (ws_bytes < attn_bitmap_bytes(B, T)) return MLA_E_WORKSPACE;
    const size_t M = (size_t)B * T;
    const Span ins[] = {{q, M * MLA_HEADS * MLA_QK_HEAD * kBf16},
                        {kv, M * MLA_HEADS * 256 * kBf16},
                        {k_pe, M * MLA_ROPE * kBf16},
                        {workspace, attn_bitmap_bytes(B, T)}};
    const Span outs[] = {{out, M * MLA_HEADS * MLA_V_HEAD * kBf16}};
    if (any_alias(outs, 1, ins, 4)) return MLA_E_ALIAS;
    return MLA_OK;
}
}  // namespace

int mla_sparse_prefill_attn_prepared(const void* q, const void* kv, const void* k_pe, int B, int T,
                                     float softmax_scale, void* out, const void* workspace,
                                     size_t ws_bytes, void* stream) {
    int st = validate_attn_prepared(q, kv, k_pe, B, T, softmax_scale, out, workspace, ws_bytes);
    if (st != MLA_OK) return st;
    if ((st = check_device()) != MLA_OK) return st;
    return launched(mla::launch_sparse_attn(static_cast<const uint16_t*>(q),
                                            static_cast<const uint16_t*>(kv),
                                            static_cast<const uint16_t*>(k_pe),
                                            static_cast<const uint32_t*>(workspace), B, T,
                                            softmax_scale, static_cast<uint16_t*>(out),
                                            static_cast<hipStream_t>(stream)));
}

int mla_sparse_prefill_attn(const void* q, const void* kv, const void* k_pe, const int32_t* topk,
                            int B, int T, int K, float softmax_scale, void* out, void* workspace,
                            size_t ws_bytes, void* stream) {
    int st = validate_topk(topk, B, T, K);
    if (st != MLA_OK) return st;
    if ((st = validate_attn_prepared(q, kv, k_pe, B, T, softmax_scale, out, workspace, ws_bytes)) != MLA_OK)
        return st;
    const size_t M = (size_t)B * T;
    const Span ins[] = {{q, M * MLA_HEADS * MLA_QK_HEAD * kBf16},
                        {kv, M * MLA_HEADS * 256 * kBf16},
                        {k_pe, M * MLA_ROPE * kBf16},
                        {topk, M * K * sizeof(int32_t)}};
    const Span outs[] = {{out, M * MLA_HEADS * MLA_V_HEAD * kBf16}, {workspace, attn_bitmap_bytes(B, T)}};
    if (any_alias(outs, 2, ins, 4)) return MLA_E_ALIAS;
    if ((st = check_device()) != MLA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t* bm = static_cast<uint32_t*>(workspace);
    st = launched(mla::launch_attn_select(topk, B, T, K, bm, s));
    if (st != MLA_OK) return st;
    return launched(mla::launch_sparse_attn(static_cast<const uint16_t*>(q),
                                            static_cast<const uint16_t*>(kv),
                                            static_cast<const uint16_t*>(k_pe), bm, B, T,
                                            softmax_scale, static_cast<uint16_t*>(out), s));
}

int mla_check_topk(const int32_t* topk, int B, int T, int K, int64_t* counts, void* stream) {
    int st = validate_topk(topk, B, T, K);
    if (st != MLA_OK) return st;
    if (!counts) return MLA_E_NULL;
    if (!aligned16(counts)) return MLA_E_ALIGN;
    const Span ins[] = {{topk, (size_t)B * T * K * sizeof(int32_t)}};
    const Span outs[] = {{counts, 4 * sizeof(int64_t)}};
    if (any_alias(outs, 1, ins, 1)) return MLA_E_ALIAS;
    if ((st = check_device()) != MLA_OK) return st;
    return launched(mla::launch_check_topk(topk, B, T, K, counts, static_cast<hipStream_t>(stream)));
}

int mla_sparse_prefill_attn_noalloc(const void* q, const void* kv, const void* k_pe, const int32_t* topk,
                                    int B, int T, int K, float softmax_scale, void* out, void* stream) {
    int st = validate_topk(topk, B, T, K);
    if (st != MLA_OK) return st;
    if (!q || !kv || !k_pe || !out) return MLA_E_NULL;
    if (!aligned16(q) || !aligned16(kv) || !aligned16(k_pe) || !aligned16(out)) return MLA_E_ALIGN;
    if (!pos_finite(softmax_scale)) return MLA_E_ARG;
    if (attn_bitmap_bytes(B, T) > kScratchBytes) return MLA_E_SCRATCH;
    const size_t M = (size_t)B * T;
    const Span ins[] = {{q, M * MLA_HEADS * MLA_QK_HEAD * kBf16},
                        {kv, M * MLA_HEADS * 256 * kBf16},
                        {k_pe, M * MLA_ROPE * kBf16},
                        {topk, M * K * sizeof(int32_t)}};
    const Span outs[] = {{out, M * MLA_HEADS * MLA_V_HEAD * kBf16}};
    if (any_alias(outs, 1, ins, 4)) return MLA_E_ALIAS;
    if ((st = check_device()) != MLA_OK) return st;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MLA_E_DEVICE;
    uint32_t* bm = static_cast<uint32_t*>(scratch_address(dev));
    if (!bm) return MLA_E_DEVICE;
    // every word of the bitmap and flag regions the attention reads is written by the selection
    // kernels (bitmap zeros past the sequence), so the scratch needs no clearing between calls
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = launched(mla::launch_attn_select(topk, B, T, K, bm, s));
    if (st != MLA_OK) return st;
    return launched(mla::launch_sparse_attn(static_cast<const uint16_t*>(q),
                                            static_cast<const uint16_t*>(kv),
                                            static_cast<const uint16_t*>(k_pe), bm, B, T,
                                            softmax_scale, static_cast<uint16_t*>(out), s));
}

size_t mla_noalloc_scratch_bytes(int B, int T) {
    if (validate_topk(reinterpret_cast<const int32_t*>(16), B, T, 1) != MLA_OK) return 0;
    return attn_bitmap_bytes(B, T);
}

int mla_selection_list_stride(int T, int K) {
    if (validate_topk(reinterpret_cast<const int32_t*>(16), 1, T, K) != MLA_OK) return 0;
    return mla::latent_list_stride(T, K);
}

int mla_selection_lists(const int32_t* topk, int B, int T, int K, int32_t* lists, int32_t* counts,
                        void* stream) {
    int st = validate_topk(topk, B, T, K);
    if (st != MLA_OK) return st;
    if (!lists || !counts) return MLA_E_NULL;
    if (!aligned16(lists) || !aligned16(counts)) return MLA_E_ALIGN;
    const size_t M = (size_t)B * T;
    const Span ins[] = {{topk, M * K * sizeof(int32_t)}};
    const Span outs[] = {{lists, M * mla::latent_list_stride(T, K) * sizeof(int32_t)},
                         {counts, M * sizeof(int32_t)}};
    if (any_alias(outs, 2, ins, 1)) return MLA_E_ALIAS;
    if ((st = check_device()) != MLA_OK) return st;
    return launched(mla::launch_sel_list(topk, B, T, K, lists, counts, static_cast<hipStream_t>(stream)));
}

size_t mla_attn_latent_workspace_bytes(int B, int T, int K) {
    if (validate_topk(reinterpret_cast<const int32_t*>(16), B, T, K) != MLA_OK) return 0;
    return mla::latent_workspace(B, T, K, 0).bytes;
}

int mla_sparse_prefill_attn_latent(const void* q, const void* c_kv, const void* k_pe, const void* w_ukv,
                                   const int32_t* topk, int B, int T, int K, float softmax_scale,
                                   void* out, void* workspace, size_t ws_bytes, void* stream) {
    int st = validate_topk(topk, B, T, K);
    if (st != MLA_OK) return st;
    if (!q || !c_kv || !k_pe || !w_ukv || !out || !workspace) return MLA_E_NULL;
    if (!aligned16(q) || !aligned16(c_kv) || !aligned16(k_pe) || !aligned16(w_ukv) || !aligned16(out) ||
        !aligned16(workspace))
        return MLA_E_ALIGN;
    if (!pos_finite(softmax_scale)) return MLA_E_ARG;
    const size_t need = mla::latent_workspace(B, T, K, 0).bytes;
    if (ws_bytes < need) return MLA_E_WORKSPACE;
    const size_t M = (size_t)B * T;
    const Span ins[] = {{q, M * MLA_HEADS * MLA_QK_HEAD * kBf16},
                        {c_kv, M * MLA_KV_LORA * kBf16},
                        {k_pe, M * MLA_ROPE * kBf16},
                        {w_ukv, (size_t)MLA_KV_B_OUT * MLA_KV_LORA * kBf16},
                        {topk, M * K * sizeof(int32_t)}};
    const Span outs[] = {{out, M * MLA_HEADS * MLA_V_HEAD * kBf16}, {workspace, need}};
    if (any_alias(outs, 2, ins, 5)) return MLA_E_ALIAS;
    if ((st = check_device()) != MLA_OK) return st;
    return launched(mla::launch_sparse_attn_latent(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(c_kv), static_cast<const uint16_t*>(k_pe),
        static_cast<const uint16_t*>(w_ukv), topk, B, T, K, 0, softmax_scale, static_cast<uint16_t*>(out), workspace,
        static_cast<hipStream_t>(stream)));
}

int mla_attn_auto_split(int T, int K) {
    if (validate_topk(reinterpret_cast<const int32_t*>(16), 1, T, K) != MLA_OK) return -1;
    return mla::latent_auto_split(T, K);
}

size_t mla_attn_auto_workspace_bytes(int B, int T, int K) {
    if (validate_topk(reinterpret_cast<const int32_t*>(16), B, T, K) != MLA_OK) return 0;
    return mla::auto_workspace(B, T, K).bytes;
}

int mla_sparse_prefill_attn_auto(const void* q, const void* c_kv, const void* k_pe, const void* w_ukv,
                                 const int32_t* topk, int B, int T, int K, float softmax_scale, void* out,
                                 void* workspace, size_t ws_bytes, void* stream) {
    int st = validate_topk(topk, B, T, K);
    if (st != MLA_OK) return st;
    if (!q || !c_kv || !k_pe || !w_ukv || !out || !workspace) return MLA_E_NULL;
    if (!aligned16(q) || !aligned16(c_kv) || !aligned16(k_pe) || !aligned16(w_ukv) || !aligned16(out) ||
        !aligned16(workspace))
        return MLA_E_ALIGN;
    if (!pos_finite(softmax_scale)) return MLA_E_ARG;
    const size_t need = mla::auto_workspace(B, T, K).bytes;
    if (ws_bytes < need) return MLA_E_WORKSPACE;
    const size_t M = (size_t)B * T;
    const Span ins[] = {{q, M * MLA_HEADS * MLA_QK_HEAD * kBf16},
                        {c_kv, M * MLA_KV_LORA * kBf16},
                        {k_pe, M * MLA_ROPE * kBf16},
                        {w_ukv, (size_t)MLA_KV_B_OUT * MLA_KV_LORA * kBf16},
                        {topk, M * K * sizeof(int32_t)}};
    const Span outs[] = {{out, M * MLA_HEADS * MLA_V_HEAD * kBf16}, {workspace, need}};
    if (any_alias(outs, 2, ins, 5)) return MLA_E_ALIAS;
    if ((st = check_device()) != MLA_OK) return st;
    return launched(mla::launch_sparse_attn_auto(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(c_kv), static_cast<const uint16_t*>(k_pe),
        static_cast<const uint16_t*>(w_ukv), topk, B, T, K, softmax_scale, static_cast<uint16_t*>(out), workspace,
        static_cast<hipStream_t>(stream)));
}

float mla_default_softmax_scale(void) {
    const double m = 1.0 + 0.1 * log(40.0);
    return (float)(m * m / sqrt(192.0));
}

const char* mla_status_string(int status) {
    switch (status) {
        case MLA_OK: return "MLA_OK";
        case MLA_E_NULL: return "MLA_E_NULL: a required pointer is NULL";
        case MLA_E_SHAPE: return "MLA_E_SHAPE: unsupported shape";
        case MLA_E_ALIGN: return "MLA_E_ALIGN: pointer not 16-byte aligned";
        case MLA_E_WORKSPACE: return "MLA_E_WORKSPACE: workspace too small";
        case MLA_E_DEVICE: return "MLA_E_DEVICE: current device is not gfx950";
        case MLA_E_LAUNCH: return "MLA_E_LAUNCH: kernel launch failed";
        case MLA_E_ARG: return "MLA_E_ARG: eps/theta/scale must be finite and positive";
        case MLA_E_ALIAS: return "MLA_E_ALIAS: an output overlaps another buffer";
        case MLA_E_SCRATCH:
            return "MLA_E_SCRATCH: the problem needs more than the fixed scratch of the no-allocation entry point";
        default: return "unknown status";
    }
}

int mla_last_hip_error(void) { return g_last_hip_error; }

const char* mla_build_info(void) { return "libmla gfx950 (hipcc " __clang_version__ ")"; }

}  // extern "C"
