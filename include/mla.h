/*
 * mla.h - C ABI of the MI355X (gfx950) sparse latent-attention prefill library (libmla.so).
 *
 * The library computes the DeepSeek-V3.2-Exp sparse multi-head latent-attention prefill as the
 * model-atlas pages describe it:
 *
 *   mla_kv_latent            x -> joint KV down-projection (512 latent + 64 rotary key),
 *                            fp32 RMSNorm of the latent, rotary rotation of the shared key
 *                            ("DeepSeek-V3.2-Exp · Key-value down-projection": formula and the
 *                            MLA key-value code excerpt; "DeepSeek V4.1 · Key-value RMSNorm":
 *                            formula and the RMSNorm code excerpt).
 *   mla_kv_up                latent -> 128 heads of [128 non-rotary key | 128 value]
 *                            ("DeepSeek-V3.2-Exp · Keys": MHA-prefill code excerpt;
 *                            "DeepSeek-V3.2-Exp · Split value heads": [B,T,16384] -> [B,128,T,128]).
 *   mla_sparse_prefill_attn  scores over [k_nope | k_pe] times the softmax scale, restricted to
 *                            the top-k selection intersected with the causal mask, softmax over
 *                            keys, value mixing ("DeepSeek-V3.2-Exp · Keys": MHA-prefill code
 *                            excerpt; "DeepSeek-V3.2-Exp · Scale scores": formula).
 *   mla_kv_latent_cache      mla_kv_latent plus the FP8 round trip of the latent and the
 *                            latent / rotary-key cache writes (the down-projection page's
 *                            KV-cache evidence).
 *   mla_window_kv            V4.1 window keys/values: norm, rotary tail, FP8 round trip, ring
 *                            buffer ("DeepSeek V4.1 · Key-value RMSNorm": window-KV excerpt).
 *   mla_q_path               the query path: wq_a, q_norm, wq_b, rotary of each head's rotary
 *                            part (the MLA constructor excerpt's query modules).
 *
 * Conventions for every call
 *  - Pointers marked (device) are HIP device pointers; all tensors are dense, row-major,
 *    contiguous, and must be 16-byte aligned. bf16 tensors are passed as raw 16-bit storage.
 *  - The caller owns every buffer (inputs, outputs, workspace). The library allocates no memory
 *    and keeps no state beyond a per-device architecture check.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream). Calls only enqueue
 *    work on it and return; nothing is synchronised. Device faults surface at the caller's next
 *    synchronisation.
 *  - Return value: MLA_OK (0) or a negative MLA_E_* code. On a negative code nothing was
 *    enqueued. Argument checks run before any HIP call. MLA_E_LAUNCH reports a HIP launch
 *    failure; mla_last_hip_error() then returns the hipError_t of this thread's last failure.
 *  - Outputs must not overlap inputs.
 *  - Model dimensions are fixed at compile time (the MLA constructor excerpt and the pages'
 *    shapes): hidden 7168, latent 512, rotary 64, 128 heads, 192 = 128 + 64 query/key features,
 *    128 value features.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_HIDDEN 7168
#define MLA_KV_LORA 512
#define MLA_ROPE 64
#define MLA_KV_A_OUT 576      /* MLA_KV_LORA + MLA_ROPE rows of the down-projection weight */
#define MLA_HEADS 128
#define MLA_QK_NOPE 128
#define MLA_QK_HEAD 192       /* MLA_QK_NOPE + MLA_ROPE */
#define MLA_V_HEAD 128
#define MLA_KV_B_OUT 32768    /* MLA_HEADS * (MLA_QK_NOPE + MLA_V_HEAD) */
#define MLA_Q_LORA 1536       /* q_lora_rank: not on the pages; the library's fixed reading */
#define MLA_MAX_T 32768       /* longest sequence the selection/attention calls accept */
#define MLA_MAX_ROWS (1 << 24)

enum {
    MLA_OK = 0,
    MLA_E_NULL = -1,       /* a required pointer is NULL */
    MLA_E_SHAPE = -2,      /* B, T, K, rows or a stride outside the supported range */
    MLA_E_ALIGN = -3,      /* a pointer is not 16-byte aligned */
    MLA_E_WORKSPACE = -4,  /* workspace smaller than mla_attn_workspace_bytes() */
    MLA_E_DEVICE = -5,     /* current device is not gfx950, or no device */
    MLA_E_LAUNCH = -6,     /* a kernel launch failed (see mla_last_hip_error) */
    MLA_E_ARG = -7,        /* eps, theta or softmax_scale not finite and > 0 */
    MLA_E_ALIAS = -8,      /* an output overlaps an input or another output */
    MLA_E_SCRATCH = -9     /* beyond the fixed scratch of mla_sparse_prefill_attn_noalloc */
};

/* Bytes of device scratch mla_sparse_prefill_attn_noalloc holds on each device it runs on: 32 MiB
 * for the selection bitmap and 128 KiB for the key-tile flags. */
#define MLA_NOALLOC_SCRATCH_BYTES ((32u << 20) + (128u << 10))

/*
 * Joint KV down-projection, latent RMSNorm and rotary key (one call for the front end).
 *   x        (device) bf16 [B, T, 7168]
 *   w_dkv    (device) bf16 [576, 7168], stored [out, in] as the Linear excerpt holds weights;
 *            rows 0..511 produce the latent, rows 512..575 the shared rotary key.
 *   kv_gain  (device) fp32 [512], the RMSNorm learned gain.
 *   eps      RMSNorm epsilon (1e-6 is the RMSNorm class default used by the V3.2 kv_norm).
 *   rope_cs  (device) fp32 [T, 32, 2]: (cos, sin) of t * theta^(-2i/64) for t < T, i < 32
 *            (the pages' freqs_cis; build it with mla_rope_table).
 *   kv_raw   (device, out) bf16 [B, T, 576], the down-projection output (fp32 accumulation,
 *            one rounding to bf16).
 *   c_kv     (device, out) bf16 [B, T, 512] = bf16(gain * x / sqrt(mean(x^2) + eps)), computed in
 *            fp32 from kv_raw[..., :512].
 *   k_pe     (device, out) bf16 [B, T, 64]: kv_raw[..., 512:] with pairs (2i, 2i+1) rotated as
 *            complex numbers by angle t * theta^(-2i/64), fp32 arithmetic.
 * Errors: MLA_E_NULL, MLA_E_SHAPE (B, T < 1, B*T > MLA_MAX_ROWS), MLA_E_ALIGN, MLA_E_ARG,
 *         MLA_E_ALIAS, MLA_E_DEVICE, MLA_E_LAUNCH.
 */
int mla_kv_latent(const void* x, const void* w_dkv, const float* kv_gain, float eps,
                  const float* rope_cs, int B, int T, void* kv_raw, void* c_kv, void* k_pe,
                  void* stream);

/*
 * The norm/rotary step alone (the second half of mla_kv_latent), also used for the V4.1
 * window-KV decode norm ("DeepSeek V4.1 · Key-value RMSNorm": eps = 1e-20, in/out [B, 1, 512]).
 *   kv_raw      (device) bf16 [rows, row_stride]; row_stride is 576 (latent + rotary key) or
 *               512 (latent only).
 *   has_rope    nonzero: rotate kv_raw[r, 512:576] into k_pe[r] at position r % T (requires
 *               row_stride 576, rope_cs and k_pe); zero: no rotary output (rope_cs, k_pe, T unused).
 *   gain, eps   as for mla_kv_latent.
 *   c_kv        (device, out) bf16 [rows, 512];  k_pe (device, out) bf16 [rows, 64].
 * Errors: as mla_kv_latent.
 */
int mla_kv_norm_rope(const void* kv_raw, int rows, int row_stride, int has_rope,
                     const float* gain, float eps, const float* rope_cs, int T, void* c_kv,
                     void* k_pe, void* stream);

/*
 * Rotary table for positions 0..T-1: rope_cs[t][i] = (cos, sin)(t * theta^(-2i/64)), i < 32,
 * evaluated in fp64 on the device and rounded to fp32 (the pages pass this table, freqs_cis,
 * into the rotary helper; the model-args excerpt sets rope_theta = 10000).
 *   rope_cs (device, out) fp32 [T, 32, 2].
 * Errors: MLA_E_NULL, MLA_E_SHAPE (T < 1 or T > MLA_MAX_ROWS), MLA_E_ARG, MLA_E_DEVICE,
 *         MLA_E_LAUNCH.
 */
int mla_rope_table(int T, float theta, float* rope_cs, void* stream);

/*
 * Latent front end with the FP8 round trip of the latent and the key-value cache writes
 * ("DeepSeek-V3.2-Exp · Key-value down-projection": the MLA key-value excerpt, then the
 * KV-cache evidence: the normalised latent is quantised to fp8 in blocks of 128 features and
 * brought back — fp8 values times the block scale in float, cast to bf16 — and stored with the
 * rotated key in two caches at positions start_pos..start_pos+T-1; the up-projection consumes
 * the rounded latent). The quantiser is not on the pages; this library's: e4m3 (largest value
 * 448), scale s = amax/448 in fp32 (scale_fmt 0) or that rounded up to a power of two
 * (scale_fmt 1), code = e4m3 value nearest to x/s (correctly rounded fp32 division, ties to the
 * even code), result bf16(code * s); a block of zeros stays zero.
 *   x, w_dkv, kv_gain, eps  as for mla_kv_latent.
 *   rope_cs     (device) fp32 [start_pos + T, 32, 2]: the table of mla_rope_table, indexed by
 *               absolute position (row t of the call is position start_pos + t).
 *   start_pos   first position of the call, >= 0.
 *   kv_raw      (device, out) bf16 [B, T, 576]: the down-projection output.
 *   c_kv        (device, out) bf16 [B, T, 512]: the rounded latent (input of mla_kv_up).
 *   k_pe        (device, out) bf16 [B, T, 64]: the rotated key.
 *   kv_cache    (device, in/out) bf16 [cache_batch, cache_len, 512]; rows [b, start_pos + t]
 *               for b < B, t < T receive c_kv[b, t]; every other row is left as it was.
 *   pe_cache    (device, in/out) bf16 [cache_batch, cache_len, 64]; the same rows receive k_pe.
 *   cache_batch >= B;  cache_len >= start_pos + T.
 *   c_norm      (device, out, may be NULL) bf16 [B, T, 512]: the normalised latent before the
 *               round trip.
 * Errors: MLA_E_NULL, MLA_E_SHAPE (B, T < 1, B*T > MLA_MAX_ROWS, start_pos < 0, the cache too
 *         small, start_pos + T > MLA_MAX_ROWS), MLA_E_ALIGN, MLA_E_ARG (eps, or scale_fmt not 0
 *         or 1), MLA_E_ALIAS, MLA_E_DEVICE, MLA_E_LAUNCH.
 */
int mla_kv_latent_cache(const void* x, const void* w_dkv, const float* kv_gain, float eps,
                        const float* rope_cs, int B, int T, int start_pos, int scale_fmt,
                        void* kv_raw, void* c_kv, void* k_pe, void* kv_cache, void* pe_cache,
                        int cache_batch, int cache_len, void* c_norm, void* stream);

/*
 * The norm/rotary/round-trip/cache step alone (the second half of mla_kv_latent_cache), from a
 * down-projection output kv_raw (device) bf16 [B, T, 576]. Other arguments and errors as for
 * mla_kv_latent_cache.
 */
int mla_kv_norm_rope_cache(const void* kv_raw, int B, int T, int start_pos, const float* gain,
                           float eps, const float* rope_cs, int scale_fmt, void* c_kv, void* k_pe,
                           void* kv_cache, void* pe_cache, int cache_batch, int cache_len,
                           void* c_norm, void* stream);

/*
 * Query path ("DeepSeek-V3.2-Exp · Key-value down-projection": MLA constructor excerpt with wq_a,
 * q_norm and wq_b; "DeepSeek-V3.2-Exp · Keys": MHA-prefill excerpt, q = [q_nope | q_pe] per head,
 * and the indexer's qr argument). The forward is not on the pages; this library's reading:
 * qa = bf16(x . W_qa^T), qr = bf16(q_gain * qa * rsqrt(mean(qa^2) + eps)) in fp32, q = bf16(qr .
 * W_qb^T) viewed [B, T, 128, 192], and features 128..191 of every head (q_pe) rotated as the
 * shared key is (pairs (2i, 2i+1) as complex numbers, angle (start_pos + t) * theta^(-2i/64),
 * fp32 arithmetic on the bf16 values, rounded to bf16).
 *   x          (device) bf16 [B, T, 7168].
 *   w_qa       (device) bf16 [1536, 7168], [out, in].
 *   q_gain     (device) fp32 [1536];  eps (host) finite and > 0 (the RMSNorm default is 1e-6).
 *   w_qb       (device) bf16 [128 * 192, 1536], [out, in]; output feature h*192 + j is head h's
 *              feature j (j < 128 non-rotary, j >= 128 rotary).
 *   rope_cs    (device) fp32 [start_pos + T, 32, 2] (mla_rope_table), by absolute position.
 *   q_rank     must be MLA_Q_LORA (1536).
 *   qa         (device, out) bf16 [B, T, 1536]: the wq_a output.
 *   qr         (device, out) bf16 [B, T, 1536]: the normalised low-rank query (the indexer's input).
 *   q          (device, out) bf16 [B, T, 128, 192]: the query mla_sparse_prefill_attn takes.
 * Errors: MLA_E_NULL, MLA_E_SHAPE (B, T < 1, B*T > MLA_MAX_ROWS, start_pos < 0, q_rank),
 *         MLA_E_ALIGN, MLA_E_ARG (eps), MLA_E_ALIAS, MLA_E_DEVICE, MLA_E_LAUNCH.
 */
int mla_q_path(const void* x, const void* w_qa, const float* q_gain, float eps, const void* w_qb,
               const float* rope_cs, int B, int T, int start_pos, int q_rank, void* qa, void* qr,
               void* q, void* stream);

/*
 * V4.1 window keys/values ("DeepSeek V4.1 · Key-value RMSNorm", formula and window-KV excerpt):
 * RMSNorm of the 512-wide projection output (the page's eps is 1e-20), rotary on its last 64
 * features in place (pairs (2i, 2i+1) of the tail as complex numbers, angle
 * position * theta^(-2i/64)), the FP8 round trip of mla_kv_latent_cache over the whole vector
 * (rotary tail included), then the ring-buffer writes: position p = start_pos + s goes to slot
 * p mod window, for the last min(S, window) positions of the call (the page's prefill branch
 * at start_pos 0 and its one-position decode branch both write exactly these).
 *   kv_raw        (device) bf16 [B, S, 512].
 *   gain, eps     (device) fp32 [512]; eps finite and > 0 (host).
 *   rope_cs       (device) fp32 [start_pos + S, 32, 2], by absolute position.
 *   scale_fmt     0 or 1, as for mla_kv_latent_cache.
 *   window        ring size, >= 1.
 *   kv_out        (device, out) bf16 [B, S, 512]: the rounded vectors (the page's window_kv in
 *                 prefill).
 *   window_cache  (device, in/out) bf16 [cache_batch, window, 512]; slots not written keep
 *                 their contents.
 *   kv_pre        (device, out, may be NULL) bf16 [B, S, 512]: the vectors before the round trip.
 * Errors: MLA_E_NULL, MLA_E_SHAPE (B, S, window < 1, B*S > MLA_MAX_ROWS, start_pos < 0,
 *         cache_batch < B, start_pos + S > MLA_MAX_ROWS), MLA_E_ALIGN, MLA_E_ARG, MLA_E_ALIAS,
 *         MLA_E_DEVICE, MLA_E_LAUNCH.
 */
int mla_window_kv(const void* kv_raw, int B, int S, int start_pos, const float* gain, float eps,
                  const float* rope_cs, int scale_fmt, int window, void* kv_out,
                  void* window_cache, int cache_batch, void* kv_pre, void* stream);

/*
 * KV up-projection into head-major keys and values.
 *   c_kv   (device) bf16 [B, T, 512]
 *   w_ukv  (device) bf16 [32768, 512], [out, in]; output feature h*256 + j is head h's
 *          non-rotary key feature j for j < 128 and its value feature j - 128 otherwise.
 *   kv     (device, out) bf16 [B, 128, T, 256]: kv[b, h, t, :] = bf16(c_kv[b, t] . W[h*256 : h*256+256]^T)
 *          with fp32 accumulation.
 * Errors: MLA_E_NULL, MLA_E_SHAPE, MLA_E_ALIGN, MLA_E_ALIAS, MLA_E_DEVICE, MLA_E_LAUNCH.
 */
int mla_kv_up(const void* c_kv, const void* w_ukv, int B, int T, void* kv, void* stream);

/*
 * Bytes of workspace mla_sparse_prefill_attn needs: the selection bitmap in the layout the
 * attention kernel reads, 4 * B * (2 * ceil(T/64)) * (256 * ceil(T/256)) bytes (rounded up to
 * 256). Returns 0 for shapes the call would reject.
 */
size_t mla_attn_workspace_bytes(int B, int T, int K);

/*
 * Selection intersected with the causal mask, as a bitmap (the MHA-prefill excerpt's scattered
 * index mask plus causal mask, stored as bits).
 *   topk    (device) int32 [B, T, K]: key positions per query. Entries outside [0, T) select
 *           nothing (-1 marks an empty slot); repeated entries select once; entries > s are
 *           removed by the causal mask.
 *   bitmap  (device, out) uint32 [B, ceil(T/32), T]: bit (t % 32) of bitmap[b][t / 32][s] is
 *           set iff t is one of row s's entries and t <= s.
 * Errors: MLA_E_NULL, MLA_E_SHAPE (B, T, K < 1, T > MLA_MAX_T, K > 65536), MLA_E_ALIGN,
 *         MLA_E_DEVICE, MLA_E_LAUNCH.
 */
int mla_selection_bitmap(const int32_t* topk, int B, int T, int K, uint32_t* bitmap, void* stream);

/*
 * Validity report of a top-k selection (a debug aid; the attention calls never need it). The
 * MHA-prefill code excerpt of "DeepSeek-V3.2-Exp · Keys" scatters the indexer's top-k indices into
 * a -inf index mask and adds the causal mask; the attention calls read each entry the same way
 * (outside [0, T): selects nothing, -1 marking an empty slot; later than the query: removed by the
 * causal mask; repeated: selected once), so no entry is an error to them and none is reported by
 * them. This call counts, over all B * T rows:
 *   counts[0]  entries outside [-1, T) (neither a key position nor the empty-slot marker),
 *   counts[1]  entries t with s < t < T (later than their query s),
 *   counts[2]  repeats of an allowed entry within its row (each occurrence after the first),
 *   counts[3]  rows whose allowed set is empty (the attention calls write zeros for such a row).
 *   topk    (device) int32 [B, T, K], as for mla_selection_bitmap.
 *   counts  (device, out) int64 [4], overwritten. The call is asynchronous like every other:
 *           synchronise the stream before reading the counts.
 * Errors: MLA_E_NULL, MLA_E_SHAPE (as mla_selection_bitmap), MLA_E_ALIGN, MLA_E_ALIAS,
 *         MLA_E_DEVICE, MLA_E_LAUNCH.
 */
int mla_check_topk(const int32_t* topk, int B, int T, int K, int64_t* counts, void* stream);

/*
 * Sparse prefill attention.
 *   q        (device) bf16 [B, T, 128, 192], each head's query as [128 non-rotary | 64 rotary]
 *            (the excerpt concatenates q_nope and q_pe in that order).
 *   kv       (device) bf16 [B, 128, T, 256] from mla_kv_up.
 *   k_pe     (device) bf16 [B, T, 64], shared by all heads (appended to every head's key).
 *   topk     (device) int32 [B, T, K], as for mla_selection_bitmap.
 *   softmax_scale  multiplies q.k (mla_default_softmax_scale() gives m^2/sqrt(192)).
 *   out      (device, out) bf16 [B, T, 128, 128]:
 *            out[b,s,h] = sum_{t in A(b,s)} softmax_t(scale * q[b,s,h] . k[b,h,t]) v[b,h,t],
 *            fp32 scores, softmax and accumulation; A(b,s) = selected keys with t <= s.
 *            Keys outside A(b,s) receive exactly zero weight.
 *   workspace, ws_bytes  (device) scratch of at least mla_attn_workspace_bytes(B, T, K) bytes;
 *            its contents on entry do not matter and are overwritten.
 * A query with no allowed key (outside the pages' contract: their -inf mask would give NaN there)
 * gets an output row of zeros; mla_check_topk counts such rows.
 * Errors: MLA_E_NULL, MLA_E_SHAPE, MLA_E_ALIGN, MLA_E_WORKSPACE, MLA_E_ARG, MLA_E_ALIAS,
 *         MLA_E_DEVICE, MLA_E_LAUNCH.
 */
int mla_sparse_prefill_attn(const void* q, const void* kv, const void* k_pe, const int32_t* topk,
                            int B, int T, int K, float softmax_scale, void* out, void* workspace,
                            size_t ws_bytes, void* stream);

/*
 * mla_sparse_prefill_attn in two calls, so that the selection step (which depends only on the
 * top-k indices) can run on another stream while the projections run:
 * mla_attn_prepare builds the selection bitmap (the excerpt's index mask intersected with the
 * causal mask, in the attention kernel's layout) and, per 256 queries, a flag per 64-key tile
 * that holds any allowed key, into the workspace; it reads only topk. The attention scores only
 * flagged tiles: with a selection that leaves whole tiles empty (local or block-structured
 * selections) the work shrinks with it.
 *   topk, B, T, K       as for mla_sparse_prefill_attn.
 *   workspace, ws_bytes (device, out) at least mla_attn_workspace_bytes(B, T, K) bytes.
 * Errors: MLA_E_NULL, MLA_E_SHAPE, MLA_E_ALIGN, MLA_E_WORKSPACE, MLA_E_ALIAS, MLA_E_DEVICE,
 *         MLA_E_LAUNCH.
 */
int mla_attn_prepare(const int32_t* topk, int B, int T, int K, void* workspace, size_t ws_bytes,
                     void* stream);

/*
 * The attention of mla_sparse_prefill_attn from a workspace that mla_attn_prepare filled for the
 * same B and T (the caller orders the two calls, e.g. with an event when they run on different
 * streams; the workspace is only read here). Arguments as for mla_sparse_prefill_attn.
 * Errors: MLA_E_NULL, MLA_E_SHAPE, MLA_E_ALIGN, MLA_E_WORKSPACE, MLA_E_ARG, MLA_E_ALIAS,
 *         MLA_E_DEVICE, MLA_E_LAUNCH.
 */
int mla_sparse_prefill_attn_prepared(const void* q, const void* kv, const void* k_pe, int B, int T,
                                     float softmax_scale, void* out, const void* workspace,
                                     size_t ws_bytes, void* stream);

/*
 * mla_sparse_prefill_attn for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same kernels and result,
 * with the selection bitmap and key-tile flags kept in a fixed device array of
 * MLA_NOALLOC_SCRATCH_BYTES that the library holds on each device for the life of the process,
 * instead of a caller workspace. The call allocates nothing (no hipMalloc, no library allocation)
 * and only enqueues work.
 *   q, kv, k_pe, topk, B, T, K, softmax_scale, out   as for mla_sparse_prefill_attn.
 * Limit: mla_noalloc_scratch_bytes(B, T) (the bitmap, 4 * B * (2 * ceil(T/64)) * (256 * ceil(T/256))
 * bytes, then 4 * B * ceil(T/256) * ceil(T/2048) bytes of flags rounded up to 256) must fit the
 * scratch (a bitmap of B * T^2 / 8 <= 32 MiB for T a multiple of 256: B <= 16 at T = 4096, B = 1 at
 * T = 16384); larger problems are rejected with MLA_E_SCRATCH before anything is enqueued.
 * Every call on one device shares that device's scratch: calls that may overlap on one device
 * (different streams, or different threads without ordering) race, and must be serialised by the
 * caller. The scratch keeps the last call's bitmap and flags; nothing in it has to start at zero.
 * Errors: MLA_E_NULL, MLA_E_SHAPE, MLA_E_ALIGN, MLA_E_ARG, MLA_E_ALIAS, MLA_E_SCRATCH, MLA_E_DEVICE,
 *         MLA_E_LAUNCH.
 */
int mla_sparse_prefill_attn_noalloc(const void* q, const void* kv, const void* k_pe, const int32_t* topk,
                                    int B, int T, int K, float softmax_scale, void* out, void* stream);

/* Scratch bytes mla_sparse_prefill_attn_noalloc needs for B sequences of length T (0 for shapes the
 * attention calls reject). */
size_t mla_noalloc_scratch_bytes(int B, int T);

/*
 * Row stride (entries) of the selection lists: ceil(min(T, K) / 64) * 64. Returns 0 for shapes the
 * list call would reject.
 */
int mla_selection_list_stride(int T, int K);

/*
 * Selection intersected with the causal mask, as sorted lists (the same set as
 * mla_selection_bitmap: the MHA-prefill excerpt's scattered index mask plus causal mask).
 *   topk    (device) int32 [B, T, K], as for mla_selection_bitmap.
 *   lists   (device, out) int32 [B, T, L], L = mla_selection_list_stride(T, K): row (b, s) holds
 *           the distinct allowed key positions t <= s in increasing order, then 0 up to the next
 *           multiple of 64 (entries after that are not written).
 *   counts  (device, out) int32 [B, T]: the number of allowed keys of each row.
 * Errors: MLA_E_NULL, MLA_E_SHAPE, MLA_E_ALIGN, MLA_E_ALIAS, MLA_E_DEVICE, MLA_E_LAUNCH.
 */
int mla_selection_lists(const int32_t* topk, int B, int T, int K, int32_t* lists, int32_t* counts,
                        void* stream);

/*
 * Bytes of workspace mla_sparse_prefill_attn_latent needs (a transposed copy of the key half of
 * W_UKV, the selection lists, the absorbed queries and the latent outputs:
 * about 16.8 MB + B*T*(4*L + 262152) bytes). Returns 0 for shapes the call would reject.
 */
size_t mla_attn_latent_workspace_bytes(int B, int T, int K);

/*
 * Sparse prefill attention computed in the latent space, for long sequences: the same result as
 * mla_kv_up followed by mla_sparse_prefill_attn, up to rounding, without forming per-head keys
 * and values. "DeepSeek-V3.2-Exp · Keys", MHA-prefill code excerpt: per head, the non-rotary key
 * and the value are the two halves of wkv_b applied to the normalised latent; regrouping the
 * products (not shown on the pages) scores every head against the shared 576-wide rows
 * [c_kv | k_pe] of the selected keys only:
 *   q_lat[h] = bf16(W_UK[h]^T q_nope[h]) (fp32 accumulation), scores = scale * [q_lat | q_pe] . [c_kv | k_pe],
 *   o_lat[h] = bf16(sum_t softmax_t * c_kv[t]),  out[h] = bf16(W_UV[h] o_lat[h]) (fp32 accumulation),
 * W_UK[h] = w_ukv rows h*256 .. h*256+127, W_UV[h] = rows h*256+128 .. h*256+255.
 *   q        (device) bf16 [B, T, 128, 192] as for mla_sparse_prefill_attn.
 *   c_kv     (device) bf16 [B, T, 512];  k_pe (device) bf16 [B, T, 64] (from mla_kv_latent).
 *   w_ukv    (device) bf16 [32768, 512] as for mla_kv_up.
 *   topk     (device) int32 [B, T, K] as for mla_selection_bitmap.
 *   softmax_scale, out  as for mla_sparse_prefill_attn (out [B, T, 128, 128] bf16).
 *   workspace, ws_bytes  (device) at least mla_attn_latent_workspace_bytes(B, T, K) bytes,
 *            contents on entry irrelevant.
 * As for mla_sparse_prefill_attn, a query with no allowed key gets an output row of zeros.
 * Errors: MLA_E_NULL, MLA_E_SHAPE, MLA_E_ALIGN, MLA_E_WORKSPACE, MLA_E_ARG, MLA_E_ALIAS,
 *         MLA_E_DEVICE, MLA_E_LAUNCH.
 */
int mla_sparse_prefill_attn_latent(const void* q, const void* c_kv, const void* k_pe, const void* w_ukv,
                                   const int32_t* topk, int B, int T, int K, float softmax_scale,
                                   void* out, void* workspace, size_t ws_bytes, void* stream);

/*
 * First query row mla_sparse_prefill_attn_auto hands to the latent form: min(T, 4K) rounded down
 * to a multiple of 256 (T: every row takes the head-major path). -1 for rejected shapes.
 */
int mla_attn_auto_split(int T, int K);

/* Bytes of workspace mla_sparse_prefill_attn_auto needs (0 for rejected shapes). */
size_t mla_attn_auto_workspace_bytes(int B, int T, int K);

/*
 * The same attention from the latent rows, split by query position: rows s < split
 * (mla_attn_auto_split) take the head-major form — per-head keys and values of rows < split, as
 * mla_kv_up computes them, then the same kernels as mla_sparse_prefill_attn — and rows s >= split
 * the latent form of mla_sparse_prefill_attn_latent. Under causality a query below split never
 * sees a key at or above it, so each part is the pages' computation on its rows ("DeepSeek-V3.2-Exp
 * · Keys", MHA-prefill excerpt). The head-major cost of a query grows with its position (every
 * causal key tile is scored) while the latent cost is set by the top-k; split is where they meet.
 * Arguments, results and errors as for mla_sparse_prefill_attn_latent, with the workspace from
 * mla_attn_auto_workspace_bytes.
 */
int mla_sparse_prefill_attn_auto(const void* q, const void* c_kv, const void* k_pe, const void* w_ukv,
                                 const int32_t* topk, int B, int T, int K, float softmax_scale, void* out,
                                 void* workspace, size_t ws_bytes, void* stream);

/* m^2 / sqrt(192) with m = 1 + 0.1 ln 40, rounded to fp32 ("DeepSeek-V3.2-Exp · Scale scores"). */
float mla_default_softmax_scale(void);

/* Static string naming a status code. */
const char* mla_status_string(int status);

/* hipError_t of this thread's last failed HIP call inside the library (0 if none). */
int mla_last_hip_error(void);

/* Static string describing the build (target architecture, compiler). */
const char* mla_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
