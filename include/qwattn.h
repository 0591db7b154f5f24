/*
 * libqwattn -- the Qwen3 attention-sublayer core on AMD MI355X (gfx950).
 *
 *   QK-Norm   per-head RMSNorm of Q and K: each head vector of head_dim values is
 *             divided by sqrt(mean of its squares + eps) and multiplied by a learned
 *             gamma of length head_dim (one for Q, one for K, shared by all heads);
 *             the variance is taken in fp32.
 *             ["7.2 Qwen3 全规模实现" §7.2.1 RMSNorm and GQA+QKNorm;
 *              "Qwen3" notes, section "QK-Norm"; "第 20 章 Qwen3 与 Qwen3.5" §20.1]
 *   RoPE      rotate-half: dims i and i + head_dim/2 of a head vector at position p
 *             turn by the angle p * theta^(-2i/head_dim).
 *             ["7.2 Qwen3 全规模实现" §7.2.1 RoPE]
 *   order     QK-Norm first, then RoPE (the order four of the five pages print);
 *             params.order = 1 selects RoPE first, then QK-Norm, the order
 *             "Transformer 20. Qwen 3 架构拆解" §2.2 describes.  The RMS is the same
 *             either way (RoPE keeps norms); the orders differ in whether gamma
 *             scales the dims before or after the rotation.
 *   attention causal softmax(Q K^T / sqrt(head_dim)) V per query head t, reading
 *             KV head floor(t / g), g = n_q_heads / n_kv_heads.
 *             ["Transformer 20. Qwen 3 架构拆解" §2.2; "7.2 Qwen3 全规模实现" §7.2.1 GQA]
 *   cache     holds K after norm and RoPE, and V; a new key is rotated at its own
 *             position start_pos and never again.
 *             ["Qwen3" notes, Qwen3Attention excerpt; "第 20 章 Qwen3 与 Qwen3.5" §20.3]
 *
 * Gated global-attention layers (Qwen3-Next, Qwen3.5; params.head_dim = 256)
 *             ["14. Qwen 家族：从 QKV 偏置到混合注意力", section on Qwen3-Next;
 *              "第 20 章 Qwen3 与 Qwen3.5" §20.4]:
 *   norm      zero-centred: the scale is 1 + w (params.norm_offset = 1);
 *   RoPE      partial: only the first rotary_dim coordinates turn, as rotate-half
 *             pairs (i, i + rotary_dim/2) at frequencies theta^(-2i/rotary_dim);
 *             the others pass unchanged (rotary_dim 64 of 256);
 *   gate      q_proj gives 2 * head_dim values per query head, the query then the
 *             gate (params.output_gate = 1); the attention output of that head is
 *             multiplied elementwise by sigmoid(gate).
 *
 * Conventions for every entry point
 *   - Device pointers are device memory of the current HIP device; host pointers
 *     are read during the call only.  The library allocates and frees nothing:
 *     scratch memory comes from the caller's `workspace`, sized by the
 *     *_workspace_size functions.  All device buffers stay the caller's.
 *   - Tensors are token-major and contiguous, head_dim (d) innermost:
 *     q [n_tok][n_q_heads][d] (or [n_tok][n_q_heads][2d] with output_gate),
 *     k and v [n_tok][n_kv_heads][d], out [n_tok][n_q_heads][d].  Every tensor
 *     of a call has the call's dtype, gamma included; math is fp32; outputs
 *     have the input dtype.  Base pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     on it in order and the call returns without synchronising.  Only kernel
 *     launches (and the optional timing events) are enqueued -- no allocation,
 *     copy or memset -- so calls may be captured into a HIP graph; launch
 *     sizes follow the host-side lengths, so a captured graph is valid for the
 *     lengths it was captured with.
 *   - Every argument is validated before anything is enqueued: on any error the
 *     call returns a non-zero status, launches nothing and writes nothing (the
 *     cache included), as an over-long append must leave the cache and the
 *     position unchanged ["第 20 章 Qwen3 与 Qwen3.5" §20.9].  A failed launch
 *     returns QWATTN_ERR_HIP; qwattn_last_error() gives the text (per thread).
 *   - Calls are reentrant; concurrent calls must not share a workspace.
 */
#ifndef QWATTN_H
#define QWATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QWATTN_ABI_VERSION 6
#define QWATTN_HEAD_DIM 128        /* Qwen3 layers                  */
#define QWATTN_HEAD_DIM_GATED 256  /* gated Qwen3-Next / 3.5 layers */

typedef enum {
  QWATTN_OK = 0,
  QWATTN_ERR_INVALID_ARG = 1,  /* bad shape, pointer, alignment or length array   */
  QWATTN_ERR_UNSUPPORTED = 2,  /* valid but not implemented (head_dim 64, ...)    */
  QWATTN_ERR_CAPACITY = 3,     /* a sequence would not fit in the cache           */
  QWATTN_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required      */
  QWATTN_ERR_HIP = 5           /* a HIP runtime call or launch failed             */
} qwattn_status;

typedef enum {
  QWATTN_F32 = 0,
  QWATTN_BF16 = 1,
  /* Not dtypes: they give the enum the range of int32, so that any value a
   * caller passes is a valid qwattn_dtype inside the (C++) library and is
   * rejected with QWATTN_ERR_INVALID_ARG rather than being undefined. */
  QWATTN_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  QWATTN_DTYPE_RANGE_MAX_ = 2147483647
} qwattn_dtype;

typedef struct {
  int32_t n_q_heads;    /* query heads, > 0 and <= 32768                           */
  int32_t n_kv_heads;   /* KV heads, > 0, divides n_q_heads; g = n_q / n_kv <= 128,
                           and <= 16 for a bf16 decode                            */
  int32_t head_dim;     /* 128, or 256 for the gated layers                        */
  float eps;            /* RMSNorm epsilon (1e-6 for Qwen3), >= 0                  */
  double rope_theta;    /* RoPE base (1e6 dense Qwen3, 1e7 for the MoE models), > 1 */
  float softmax_scale;  /* 0 => 1/sqrt(head_dim)                                   */
  int32_t order;        /* 0 = QK-Norm then RoPE, 1 = RoPE then QK-Norm            */
  int32_t rotary_dim;   /* leading coordinates RoPE turns; 0 => head_dim.  head_dim
                           128: 128; head_dim 256: 32, 64, 128 or 256            */
  float norm_offset;    /* QK-Norm scale = norm_offset + gamma: 0 (Qwen3), or 1 (the
                           zero-centred norm); head_dim 128: 0                   */
  int32_t output_gate;  /* 1: q holds [query | gate] per head (2 * head_dim values)
                           and out = attention * sigmoid(gate); head_dim 128: 0  */
} qwattn_params;

/* A KV cache: element (seq s, kv head h, slot j, dim d) of k_cache / v_cache is at
 * base + s*stride_seq + h*stride_head + j*stride_tok + d (strides in elements;
 * dim innermost and contiguous; stride_tok * elem_size and every other stride
 * must keep rows 16-byte aligned).  Slots 0 .. capacity-1 exist per sequence.
 * stride_tok * elem_size may be at most 64 MiB (QWATTN_ERR_UNSUPPORTED beyond:
 * the kernels address the rows of a 64-slot tile with 32-bit byte offsets), and
 * the last element a call can reach must lie within 2^56 elements of the base
 * (QWATTN_ERR_INVALID_ARG). */
typedef struct {
  int64_t stride_seq;
  int64_t stride_head;
  int64_t stride_tok;
  int32_t capacity;
} qwattn_cache_desc;

/* QK-Norm then RoPE on standalone rows.
 *   q [n_tok][n_q_heads][d] (with output_gate: [n_tok][n_q_heads][2d], whose gate
 *     halves are not read) and k [n_tok][n_kv_heads][d] (device): raw rows;
 *     either may be NULL (then its output must be NULL too).
 *   q_gamma, k_gamma [d] (device): the learned scales; required with q / k.
 *   positions [n_tok] (device int32, >= 0): position of each token row.
 *   q_out [n_tok][n_q_heads][d], k_out [n_tok][n_kv_heads][d] (device); may alias
 *     q, k (in place; not q with output_gate).
 * n_tok == 0 is a no-op.  Used on its own and to fill a cache with rotated keys. */
qwattn_status qwattn_qk_norm_rope(const qwattn_params* params, qwattn_dtype dtype,
                                  const void* q, const void* k,
                                  const void* q_gamma, const void* k_gamma,
                                  const int32_t* positions, int64_t n_tok,
                                  void* q_out, void* k_out, void* stream);

/* Causal GQA prefill over packed ragged sequences, with QK-Norm and RoPE fused.
 *   q [n_tok][n_q_heads][d] (output_gate: [n_tok][n_q_heads][2d]), k, v
 *     [n_tok][n_kv_heads][d] (device): raw rows of all sequences packed one after
 *     another.
 *   cu_seqlens [n_seq+1] (device int32) and cu_seqlens_host (host, same values):
 *     sequence s owns tokens cu[s] .. cu[s+1]-1 at positions 0 .. L_s-1; cu[0] = 0,
 *     non-decreasing, cu[n_seq] = n_tok.  Sequences never attend to each other.
 *   out [n_tok][n_q_heads][d] (device): attention output (gated, with
 *     output_gate), before o_proj.
 *   k_cache, v_cache, cache (optional, all NULL or all set): K after norm and RoPE
 *     and V of sequence s, token j go to slot j of cache sequence s; every
 *     L_s <= capacity.
 *   workspace (device, >= qwattn_prefill_workspace_size bytes, 256-byte aligned).
 * n_tok == 0 or n_seq == 0 is a no-op. */
qwattn_status qwattn_prefill(const qwattn_params* params, qwattn_dtype dtype,
                             const void* q, const void* k, const void* v,
                             const void* q_gamma, const void* k_gamma,
                             const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                             int32_t n_seq, void* out,
                             void* k_cache, void* v_cache, const qwattn_cache_desc* cache,
                             void* workspace, size_t workspace_bytes, void* stream);

/* One new token per sequence against a KV cache (split-K decode).
 *   q [n_seq][n_q_heads][d] (output_gate: [n_seq][n_q_heads][2d]), k, v
 *     [n_seq][n_kv_heads][d] (device): the raw new token of each sequence.
 *   k_cache, v_cache, cache: slots 0 .. start_pos[i]-1 of sequence i hold K after
 *     norm and RoPE and V.  The call normalises and rotates the new k at position
 *     start_pos[i], writes it and v into slot start_pos[i] (never re-rotating the
 *     old keys), and attends over the start_pos[i] + 1 keys.
 *   start_pos [n_seq] (device int32) and start_pos_host (host, same values):
 *     >= 0 and start_pos[i] + 1 <= capacity for every i, else QWATTN_ERR_CAPACITY
 *     with nothing written.
 *   out [n_seq][n_q_heads][d] (device).
 *   workspace (device, >= qwattn_decode_workspace_size bytes, 256-byte aligned).
 * n_seq == 0 is a no-op. */
qwattn_status qwattn_decode(const qwattn_params* params, qwattn_dtype dtype,
                            const void* q, const void* k, const void* v,
                            const void* q_gamma, const void* k_gamma,
                            void* k_cache, void* v_cache, const qwattn_cache_desc* cache,
                            const int32_t* start_pos, const int32_t* start_pos_host,
                            int32_t n_seq, void* out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* qwattn_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments, results and kernels, without a workspace.  Its scratch is a
 * fixed array of QWATTN_DECODE_NOALLOC_SCRATCH_BYTES in every device's global
 * memory, part of the library's code object (held from its load until the
 * process ends); the first call on a device looks its address up.  The call
 * allocates and frees nothing.
 *   Sizes whose qwattn_decode_workspace_size exceeds that maximum are rejected
 *   with QWATTN_ERR_WORKSPACE and nothing enqueued (at 32 query / 8 KV heads,
 *   head_dim 128, bf16: about 7.9 million cached keys in all for 64 sequences;
 *   use qwattn_decode beyond).
 *   Nothing in the scratch needs to start at zero.  All calls on one device
 *   share the array: calls that overlap in time on one device (different
 *   streams, or different threads) race and must be serialised by the caller.
 *   A failed lookup of the array returns QWATTN_ERR_HIP. */
#define QWATTN_DECODE_NOALLOC_SCRATCH_BYTES 67108864
qwattn_status qwattn_decode_noalloc(const qwattn_params* params, qwattn_dtype dtype,
                                    const void* q, const void* k, const void* v,
                                    const void* q_gamma, const void* k_gamma,
                                    void* k_cache, void* v_cache, const qwattn_cache_desc* cache,
                                    const int32_t* start_pos, const int32_t* start_pos_host,
                                    int32_t n_seq, void* out, void* stream);

/* Multi-token append (chunked prefill) against a KV cache: the new tokens of
 * each sequence attend to its cached keys and causally to each other, the mask
 * being rectangular from start_pos ["第 20 章 Qwen3 与 Qwen3.5" §20.3 (new K
 * rotated at its own positions, cached K never again) and §20.9 (appending a
 * prompt in chunks gives the single-pass result; an over-long append is
 * rejected and changes nothing)].
 *   q [n_new][n_q_heads][d] (output_gate: [n_new][n_q_heads][2d]), k, v
 *     [n_new][n_kv_heads][d] (device): raw rows of the new tokens of all
 *     sequences, packed one sequence after another.
 *   cu_new [n_seq+1] (device int32) and cu_new_host (host, same values): sequence
 *     s appends tokens cu_new[s] .. cu_new[s+1]-1; cu_new[0] = 0, non-decreasing.
 *   start_pos [n_seq] (device int32) and start_pos_host (host, same values): the
 *     number of tokens sequence s already holds; its new token j sits at position
 *     start_pos[s] + j.  >= 0, and start_pos[s] + n_s <= capacity for every s,
 *     else QWATTN_ERR_CAPACITY with nothing written.
 *   k_cache, v_cache, cache (required): slots 0 .. start_pos[s]-1 hold K after
 *     norm and RoPE and V; the call writes the new tokens' K (normed, rotated at
 *     their positions) and V into slots start_pos[s] .. start_pos[s]+n_s-1, then
 *     new token j attends to slots 0 .. start_pos[s]+j.
 *   out [n_new][n_q_heads][d] (device).
 *   workspace (device, >= qwattn_append_workspace_size bytes, 256-byte aligned).
 * With every start_pos 0 this is qwattn_prefill with a cache; one new token per
 * sequence is what qwattn_decode computes (there with a split-K kernel that
 * suits long caches).  n_seq == 0 or n_new == 0 is a no-op. */
qwattn_status qwattn_append(const qwattn_params* params, qwattn_dtype dtype,
                            const void* q, const void* k, const void* v,
                            const void* q_gamma, const void* k_gamma,
                            void* k_cache, void* v_cache, const qwattn_cache_desc* cache,
                            const int32_t* start_pos, const int32_t* start_pos_host,
                            const int32_t* cu_new, const int32_t* cu_new_host,
                            int32_t n_seq, void* out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* y = x W^T, the bias-free linear map of the sublayer's projections
 * ["Qwen3" notes, Qwen3Attention excerpt: q_proj, k_proj, v_proj, o_proj are
 * nn.Linear without bias; "7.2 Qwen3 全规模实现" §7.2.1 listing].
 *   x [m][k], w [n][k] (the weight as stored, out x in), y [m][n] (device, bf16,
 *   row-major, 16-byte aligned).  fp32 accumulation, y rounded to bf16.
 *   n a multiple of 128 and k a multiple of 64, k <= 8388608 (operand panels
 *   use 32-bit row offsets), m <= 2^31 - 1 (QWATTN_ERR_UNSUPPORTED else);
 *   m == 0 is a no-op.  Only QWATTN_BF16. */
qwattn_status qwattn_linear(qwattn_dtype dtype, const void* x, const void* w, int64_t m, int32_t n, int32_t k,
                            void* y, void* stream);

/* The whole attention sublayer of a Qwen3 layer over packed sequences (prefill),
 * or an append against the cache: q/k/v projections, QK-Norm, RoPE, causal GQA
 * attention, o_proj ["Qwen3" notes: qkv_proj -> split -> RMSNorm(Q, K) -> RoPE
 * -> attention -> o_proj; "7.2 Qwen3 全规模实现" §7.2.1 listing: heads
 * concatenated in order before out_proj].  With params.head_dim 256 it is the
 * gated global-attention sublayer of Qwen3-Next / Qwen3.5 ["14. Qwen 家族",
 * Qwen3-Next section: q_proj's width doubled, half query and half gate;
 * "第 20 章 Qwen3 与 Qwen3.5" §20.4: the split is inside each head].
 *   hidden: model width (a multiple of 128, <= 8388608, as is n_q_heads * head_dim:
 *     the projections' inner dimensions); x [n_tok][hidden] (device): the
 *     layer input rows, packed as for qwattn_prefill.
 *   w_qkv [n_q_heads * q_w + 2 n_kv_heads * head_dim][hidden] (device): the
 *     q_proj, k_proj and v_proj weights (each stored [out][in]) stacked in that
 *     order; q_w = head_dim, or 2 * head_dim with params.output_gate, where
 *     query head h owns q_proj outputs h*q_w .. h*q_w + q_w - 1: its query,
 *     then its gate.  Key and value head h own outputs h*head_dim ..
 *   w_o [hidden][n_q_heads * head_dim] (device): the o_proj weight.
 *   q_gamma, k_gamma [head_dim] (device).
 *   cu_seqlens / cu_seqlens_host, n_seq: as for qwattn_prefill.
 *   start_pos, start_pos_host: NULL for a prefill (positions 0 ..), or both set
 *     for an append (as for qwattn_append; the cache is then required).
 *   y [n_tok][hidden] (device): the sublayer output (before the residual add).
 *   k_cache, v_cache, cache: optional for a prefill, required for an append;
 *     the fused projection writes K after norm and RoPE and V straight into the
 *     slots of each token.
 *   workspace (device, >= qwattn_attention_layer_workspace_size, 256-byte
 *     aligned).
 * Only QWATTN_BF16 (QWATTN_ERR_UNSUPPORTED else); at head_dim 256 a
 * rotary_dim of at most 128.  fp32 accumulation in every product; q (and the
 * gate), k, v, the attention output and y are each rounded to bf16 once.
 * n_seq == 0 or n_tok == 0 is a no-op. */
qwattn_status qwattn_attention_layer(const qwattn_params* params, qwattn_dtype dtype, int32_t hidden,
                                     const void* x, const void* w_qkv, const void* w_o,
                                     const void* q_gamma, const void* k_gamma,
                                     const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int32_t n_seq,
                                     const int32_t* start_pos, const int32_t* start_pos_host,
                                     void* y, void* k_cache, void* v_cache, const qwattn_cache_desc* cache,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes qwattn_attention_layer needs (0 on invalid params). */
size_t qwattn_attention_layer_workspace_size(const qwattn_params* params, qwattn_dtype dtype, int32_t hidden,
                                             int32_t n_seq, int64_t n_tok, int32_t max_seqlen,
                                             int32_t with_cache);

/* Workspace bytes qwattn_append needs: n_new new tokens in all, at most max_new
 * in one sequence (0 on invalid params). */
size_t qwattn_append_workspace_size(const qwattn_params* params, qwattn_dtype dtype,
                                    int32_t n_seq, int64_t n_new, int32_t max_new);

/* Workspace bytes qwattn_prefill needs for these sizes (0 on invalid params).
 * with_cache != 0 when the call will pass a cache (the rotated K goes there). */
size_t qwattn_prefill_workspace_size(const qwattn_params* params, qwattn_dtype dtype,
                                     int32_t n_seq, int64_t n_tok, int32_t max_seqlen,
                                     int32_t with_cache);

/* Workspace bytes qwattn_decode needs for n_seq sequences whose start positions
 * sum to total_start_pos (0 on invalid params).  Non-decreasing in both: a
 * workspace sized for (n_seq, T) serves every call with n_seq sequences whose
 * start positions sum to T or less. */
size_t qwattn_decode_workspace_size(const qwattn_params* params, qwattn_dtype dtype,
                                    int32_t n_seq, int64_t total_start_pos);

/* Timing hook for benchmarks and profilers.  `begin` and `end` are hipEvent_t
 * handles (or both NULL to clear).  The calling thread's next qwattn_prefill,
 * qwattn_append, qwattn_decode, qwattn_linear or qwattn_attention_layer records
 * `begin` on its stream right before its dominant kernel (the attention kernel
 * of prefill and append, the split kernel of decode, the GEMM of linear, the
 * fused q/k/v projection of the sublayer) and `end` right after it, then clears
 * the hook.  Setting it enqueues nothing. */
qwattn_status qwattn_set_timing_events(void* begin, void* end);

/* ---- Measurement aids (not part of the attention path).  Reporting the
 * attention kernels against the rate this GPU sustains right now, beside the
 * published peaks: under a full MFMA load the clock sits well below its
 * maximum.  Both launch on `stream` and honour the timing hook above (begin
 * and end bracket the probe kernel); time them with it.  `sink` is device
 * memory of at least one float that the probe may write (only to keep its
 * work from being optimised away); it enqueues nothing else.
 *
 * qwattn_mfma_probe: on every compute unit one workgroup of four waves (one
 * per SIMD) runs a register-only loop of v_mfma_f32_32x32x16_bf16 over 8
 * independent accumulators, operands bf16 values that look random, iters
 * rounded up to a multiple of 4 (> 0 required).  Its work in flops is
 * qwattn_mfma_probe_flops(iters) (0 when the device cannot be queried).
 *
 * qwattn_hbm_read_probe: reads `bytes` (> 0, a multiple of 16) of device
 * memory at `src` (16-byte aligned) once with 16-byte nontemporal loads, eight
 * in flight per lane.
 *
 * Errors: QWATTN_ERR_INVALID_ARG (checked before anything is enqueued),
 * QWATTN_ERR_HIP on a failed launch or device query. */
qwattn_status qwattn_mfma_probe(int32_t iters, float* sink, void* stream);
double qwattn_mfma_probe_flops(int32_t iters);
qwattn_status qwattn_hbm_read_probe(const void* src, int64_t bytes, float* sink, void* stream);

const char* qwattn_status_str(qwattn_status status); /* static string             */
const char* qwattn_last_error(void);                 /* this thread's last detail */
int qwattn_abi_version(void);                        /* QWATTN_ABI_VERSION        */

#ifdef __cplusplus
}
#endif
#endif /* QWATTN_H */
