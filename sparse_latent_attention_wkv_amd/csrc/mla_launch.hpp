// Host-side launchers of the gfx950 kernels (internal to libmla.so; the C ABI in include/mla.h
// validates arguments and then calls these).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

hipError_t launch_norm_rope(const uint16_t* src, int rows, int stride, bool rope, const float* gain,
                            float eps, const float* rope_cs, int T, uint16_t* c_kv, uint16_t* k_pe,
                            hipStream_t stream);
hipError_t launch_rope_table(int T, double theta, float* rope_cs, hipStream_t stream);
// Norm/rotary pass with the fp8 round trip of the latent and the cache writes (rows b*T + t at
// position start_pos + t), and the window-KV form (ring buffer of `window` positions).
hipError_t launch_kv_norm_rope_cache(const uint16_t* kv_raw, int B, int T, int start_pos,
                                     const float* gain, float eps, const float* rope_cs,
                                     int pow2_scale, uint16_t* c_kv, uint16_t* c_norm,
                                     uint16_t* k_pe, uint16_t* kv_cache, uint16_t* pe_cache,
                                     int cache_len, hipStream_t stream);
hipError_t launch_window_kv(const uint16_t* kv_raw, int B, int S, int start_pos, const float* gain,
                            float eps, const float* rope_cs, int pow2_scale, int window,
                            uint16_t* out, uint16_t* pre, uint16_t* cache, hipStream_t stream);
hipError_t launch_gemm_kv_down(const uint16_t* x, const uint16_t* w_dkv, int M, uint16_t* kv_raw,
                               hipStream_t stream);
// Query path: x . W_qa^T (7168 -> 1536), the query RMSNorm, then qr . W_qb^T (1536 -> 128 x 192)
// with the rotary part of every head rotated at position start_pos + (row % T).
hipError_t launch_gemm_q_a(const uint16_t* x, const uint16_t* w_qa, int M, uint16_t* qa,
                           hipStream_t stream);
hipError_t launch_gemm_q_b_rope(const uint16_t* qr, const uint16_t* w_qb, int M, uint16_t* q,
                                const float* rope_cs, int T, int start_pos, hipStream_t stream);
hipError_t launch_rms_norm_q(const uint16_t* qa, int rows, const float* gain, float eps,
                             uint16_t* qr, hipStream_t stream);
hipError_t launch_gemm_kv_up(const uint16_t* c_kv, const uint16_t* w_ukv, int B, int T, uint16_t* kv,
                             hipStream_t stream);
// Selection bitmap [B][Wout][Tout] (Wout >= ceil(T/32), Tout >= T; the excess is zero-filled).
hipError_t launch_sel_bitmap(const int32_t* topk, int B, int T, int K, int Wout, int Tout,
                             uint32_t* bitmap, hipStream_t stream);
// Counts of a selection's entries outside [-1, T), later than their query, repeated, and of
// rows left with no allowed key (counts: device int64 [4], overwritten).
hipError_t launch_check_topk(const int32_t* topk, int B, int T, int K, int64_t* counts, hipStream_t stream);
// Bitmap geometry the attention kernel reads: words per query column and query columns.
int attn_bitmap_words(int T);
int attn_bitmap_cols(int T);
// Words of key-tile flags per 256-query tile.
int attn_flag_words(int T);
// The attention's selection data: the bitmap [B][attn_bitmap_words][attn_bitmap_cols] followed by
// the key-tile flags [B][ceil(T/256)][attn_flag_words]; bytes, and the two kernels that write it.
size_t attn_select_bytes(int B, int T);
hipError_t launch_attn_select(const int32_t* topk, int B, int T, int K, uint32_t* sel, hipStream_t stream);
hipError_t launch_sparse_attn(const uint16_t* q, const uint16_t* kv, const uint16_t* k_pe,
                              const uint32_t* sel, int B, int T, float scale, uint16_t* out,
                              hipStream_t stream);


// Latent-space attention (long sequences): selection lists, workspace layout, launch sequence
// for the queries s_lo..T-1 of every sequence.
int latent_list_stride(int T, int K);
hipError_t launch_sel_list(const int32_t* topk, int B, int T, int K, int32_t* lists, int32_t* counts,
                           hipStream_t stream);
struct LatentWorkspace {
    size_t wukT, counts, flags, lists, qlat, olat, bytes;   // byte offsets into the workspace, total
};
LatentWorkspace latent_workspace(int B, int T, int K, int s_lo);
hipError_t launch_sparse_attn_latent(const uint16_t* q, const uint16_t* c_kv, const uint16_t* k_pe,
                                     const uint16_t* w_ukv, const int32_t* topk, int B, int T, int K, int s_lo,
                                     float scale, uint16_t* out, void* workspace, hipStream_t stream);
// Split form: head-major for queries < split, latent form for the rest.
int latent_auto_split(int T, int K);
struct AutoWorkspace {
    int split;
    size_t kv, bitmap, latent, bytes;
};
AutoWorkspace auto_workspace(int B, int T, int K);
hipError_t launch_sparse_attn_auto(const uint16_t* q, const uint16_t* c_kv, const uint16_t* k_pe,
                                   const uint16_t* w_ukv, const int32_t* topk, int B, int T, int K, float scale,
                                   uint16_t* out, void* workspace, hipStream_t stream);

}  // namespace mla
