/*
 * duo.h -- C ABI of the DuoAttention head-split attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (arXiv 2410.10819) splits a layer's attention heads into
 * retrieval heads, which keep a full KV cache and run full causal softmax
 * attention, and streaming heads, which keep only the first `sink` tokens
 * and the most recent `recent` tokens and run attention under the
 * Lambda-shaped mask (xllm-io review "DuoAttention: Efficient Long-Context
 * LLM Inference with Retrieval and Streaming Heads", section 三 技术架构:
 * 整体框架 and 核心公式). Each layer holds two caches; Q/K/V of new tokens are
 * split along the head axis, each block attends separately and the outputs
 * are concatenated along heads (same page, section 三 推理流程). Prefill runs
 * in fixed-length chunks that fill both caches (same page, section 三
 * 预填充阶段; paperlayer summary of arXiv 2410.10819v1, section 2 Chunked
 * Pre-filling). Heads arrive pre-reordered so that retrieval heads form the
 * first contiguous block (xllm-io review, section 三 模型部署优化), and the
 * identification forward blends both attentions with one gate per KV head
 * (xllm-io review, section 三 核心公式; paperlayer summary, section 2).
 *
 * Conventions for every call:
 *   - Device pointers are plain HIP device addresses. The caller owns every
 *     device buffer (activations, both caches, the workspace); the library
 *     never allocates device memory. It allocates only the small host object
 *     behind duo_layer*, which duo_layer_destroy frees.
 *   - Activations are token-major: q and out are [B, T, Hq, D], k and v are
 *     [B, T, Hkv, D], densely packed. Query head h reads KV head h / G with
 *     G = Hq / Hkv. KV heads [0, Hr) are retrieval heads and [Hr, Hkv) are
 *     streaming heads, so query heads [0, Hr*G) are retrieval heads.
 *   - q and out are bf16. k and v are bf16 or fp16 (kv_dtype).
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream).
 *     No call synchronises the device. The token count is tracked on the
 *     host. A duo_layer must not be used from two threads at once, and calls
 *     on one layer must be ordered (same stream, or caller-side events).
 *   - Every call validates its arguments on the host first, including every
 *     condition a launch of the call depends on. On any status other than
 *     DUO_OK and DUO_ERR_HIP it enqueues nothing and leaves the layer state
 *     (token count, caches) unchanged. No C++ exception crosses this
 *     interface.
 *   - DUO_ERR_HIP reports a failed launch (an earlier asynchronous device
 *     fault may surface there). Calls made of several launches (prefill:
 *     cache append, then attention, then ring update; append: cache, then
 *     ring; decode of a ragged batch of more than 64 sequences: one launch
 *     per 64) may have enqueued the launches before the one that failed.
 *     The token count is then not advanced, but cache rows and ring slots of
 *     the new positions may already be written, overwriting ring slots that
 *     held older positions: the layer's caches are undefined and it must be
 *     refilled (or destroyed) before further use.
 *   - Pointers must be 16-byte aligned (DUO_ERR_LAYOUT otherwise).
 */
#ifndef DUO_H_
#define DUO_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DUO_OK = 0,
  DUO_ERR_INVALID_ARG = 1, /* null pointer, bad size or count */
  DUO_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. head_dim 96) */
  DUO_ERR_LAYOUT = 3,      /* misaligned pointer, non-contiguous head mask */
  DUO_ERR_CAPACITY = 4,    /* retrieval cache would overflow */
  DUO_ERR_HIP = 5          /* a HIP launch or API call failed */
} duo_status;

typedef enum {
  DUO_BF16 = 0,
  DUO_FP16 = 1,
  /* 4-bit codes per channel with one fp16 scale and one fp16 zero-point per
   * token, head and group of 32 channels (retrieval cache only). */
  DUO_INT4_G32 = 2
} duo_dtype;

typedef struct {
  int32_t batch;                /* B >= 1; every sequence has the same length */
  int32_t n_q_heads;            /* Hq, a multiple of n_kv_heads, Hq/Hkv <= 8 */
  int32_t n_kv_heads;           /* Hkv >= 1 */
  int32_t head_dim;             /* D: 64 or 128 */
  int32_t n_retrieval_kv_heads; /* Hr in [0, Hkv]: KV heads [0,Hr) are retrieval */
  int32_t sink;                 /* S >= 0 attention-sink tokens (16 at deployment) */
  int32_t recent;               /* R >= 1 recent tokens incl. the query (64) */
  int64_t retrieval_capacity;   /* max tokens held by the retrieval cache */
  duo_dtype kv_dtype;           /* dtype of k/v inputs and of the ring: BF16 | FP16 */
  duo_dtype retrieval_dtype;    /* kv_dtype, or INT4_G32 (then Hq/Hkv * D/32 <= 16) */
  float softmax_scale;          /* multiplies q.k before the softmax; finite, > 0 */
} duo_layer_desc;

/* Byte offsets of the arrays inside the caller-provided buffers.
 * Retrieval buffer, kv_dtype cache:
 *   K  [B][Hr][cap][D] elements at k_offset, V likewise at v_offset, then 32
 *   rows of padding that the decode step may read but never uses. One head's
 *   rows plus the padding must stay below 2^31 bytes: (cap + 32) * D * 2 <
 *   2^31, else DUO_ERR_UNSUPPORTED.
 * Retrieval buffer, INT4_G32 cache (cap32 = capacity rounded up to 32):
 *   K codes [B][Hr][cap32][D/2] bytes at k_offset, token-major: byte b of a
 *   row holds channel 2b in its low nibble and 2b+1 in its high nibble.
 *   V codes [B][Hr][cap32/32][16*D] bytes at v_offset, in 32-token blocks:
 *   for channel c and m in [0,16), the byte at offset
 *   16*(4*(16*(c/64) + c%16) + m/4) + 4*((c%64)/16) + m%4 of a block holds
 *   token m of the block in its low nibble and token m+16 in its high nibble.
 *   K scale/zero [B][Hr][cap32/32][D/32][32] words at k_sz_offset (block,
 *   32-channel group, token within the block), each word two fp16 values:
 *   scale in the low half, zero-point in the high half; V scale/zero likewise
 *   at v_sz_offset. A value decodes as fma(code, scale, zero) in fp32.
 *   One head's code array must stay below 2^31 bytes (cap32 * D/2 < 2^31).
 * Streaming buffer: ring K [B][Hs][S+R][D] kv_dtype at ring_k_offset, ring V
 *   at ring_v_offset, Hs = Hkv - Hr. Token position p lives in slot p if
 *   p < S, else in slot S + ((p - S) mod R).
 * Workspace: internal (split-K partials and arrival counters). */
typedef struct {
  size_t retrieval_bytes, streaming_bytes, workspace_bytes;
  size_t k_offset, v_offset, k_sz_offset, v_sz_offset;
  size_t ring_k_offset, ring_v_offset;
} duo_layout;

typedef struct duo_layer duo_layer; /* opaque host object */

/* Sizes and offsets of the buffers a layer needs. Host-only; no HIP call.
 * Errors: DUO_ERR_INVALID_ARG for a null pointer or a bad descriptor,
 * DUO_ERR_UNSUPPORTED for an unsupported head_dim, group size or dtype or a
 * batch or KV-head count above 65535, DUO_ERR_CAPACITY when a buffer of the layout would
 * exceed 2^62 bytes. */
duo_status duo_layer_layout(const duo_layer_desc* desc, duo_layout* layout);

/* Attach a layer to caller-owned device buffers of at least the sizes
 * duo_layer_layout reports (all 256-byte aligned). `n_tokens_existing`
 * tokens are taken to be already cached (0 for a fresh layer; a resumed
 * layer passes its previous count). The workspace is zero-filled on
 * `stream`. On success *out receives a new handle. */
duo_status duo_layer_init(duo_layer** out, const duo_layer_desc* desc, void* retrieval_buf,
                          void* streaming_buf, void* workspace, int64_t n_tokens_existing,
                          hipStream_t stream);

/* As duo_layer_init, for a batch whose sequences already hold different
 * token counts: n_tokens_existing[batch] (each within the capacity). Such a
 * ragged layer decodes every sequence at its own position (one launch per 64
 * sequences) and grows its sequences one at a time with
 * duo_append_kv_seq / duo_prefill_chunk_seq
 * (serving: sequences admitted at different times; paperlayer summary of
 * arXiv 2410.10819v1, section 4, and xllm-io review, section 三 推理流程). */
duo_status duo_layer_init_ragged(duo_layer** out, const duo_layer_desc* desc, void* retrieval_buf,
                                 void* streaming_buf, void* workspace,
                                 const int64_t* n_tokens_existing, hipStream_t stream);

/* Free the host object (never the caller's buffers). Null is accepted. */
duo_status duo_layer_destroy(duo_layer* layer);

/* Tokens currently cached by the layer (host counter): the largest count over
 * the batch's sequences, or -1 for null. */
int64_t duo_layer_tokens(const duo_layer* layer);

/* Tokens cached by sequence b, or -1 for null or b outside [0, batch). */
int64_t duo_layer_sequence_tokens(const duo_layer* layer, int32_t b);

/* Append `n_tokens` >= 1 tokens of K/V ([B, n_tokens, Hkv, D], kv_dtype)
 * at positions [n, n + n_tokens) without attending: retrieval heads write
 * their cache rows (quantising them for INT4_G32), streaming heads write the
 * ring slots of the positions that survive (the sinks and the last `recent`).
 * Defined by: xllm-io review "DuoAttention: Efficient Long-Context LLM
 * Inference with Retrieval and Streaming Heads", section 三 推理流程, 解码阶段
 * (each layer keeps a full cache for retrieval heads and a sink + recent cache
 * for streaming heads) and section 五 量化组合 (4-bit KV cache); the 4-bit
 * group encoding itself is this library's (the pages give none).
 * Used to fill a context. DUO_ERR_CAPACITY if n + n_tokens > capacity;
 * DUO_ERR_UNSUPPORTED while the sequences hold different counts (use
 * duo_append_kv_seq). */
duo_status duo_append_kv(duo_layer* layer, const void* k, const void* v, int32_t n_tokens,
                         hipStream_t stream);

/* Chunked prefill (xllm-io review, section 三 推理流程, 预填充阶段: chunked
 * pre-filling, streaming heads in linear time and constant memory, retrieval
 * heads with full attention; paperlayer summary of arXiv 2410.10819v1,
 * section 2 Chunked Pre-filling; the masks of section 三 核心公式)
 * of `chunk_len` >= 1 tokens at positions [n, n+chunk_len):
 * q [B, chunk_len, Hq, D] bf16, k/v [B, chunk_len, Hkv, D]. Retrieval heads
 * append the chunk to their cache and attend causally over positions
 * [0, n+chunk_len); streaming heads attend under the Lambda mask over the ring
 * as it was before the chunk plus the chunk, then the ring is updated.
 * Writes out [B, chunk_len, Hq, D] bf16 and advances the token count.
 * Every cache form is accepted: with an FP16 cache or ring the products take
 * q converted to fp16 (exact for magnitudes in fp16's normal range) and fp16
 * softmax weights; an INT4_G32 cache is attended in its decoded values
 * fma(code, scale, zero), rounded to fp16 (the chunk is quantised into the
 * cache first, so the chunk's own keys are decoded ones too).
 * Retrieval heads over a 16-bit cache (and the gate-blended forward and its
 * gate gradient below) take q multiplied by softmax_scale * log2(e) and
 * rounded once to the product type, which costs accuracy when logits are
 * large; DUO_EXACT_SCALE=1 in the environment, read at every launch, applies
 * the scale in fp32 instead.
 * DUO_ERR_CAPACITY if n + chunk_len > capacity; DUO_ERR_UNSUPPORTED while the
 * sequences hold different counts (use duo_prefill_chunk_seq). */
duo_status duo_prefill_chunk(duo_layer* layer, const void* q, const void* k, const void* v,
                             int32_t chunk_len, void* out, hipStream_t stream);

/* One decode step (xllm-io review, section 三 推理流程, 解码阶段: the new
 * token's Q/K/V split along heads, each head class attending over its own
 * cache, outputs concatenated along heads; masks of section 三 核心公式)
 * at position n: q [B, 1, Hq, D] bf16, k_new/v_new
 * [B, 1, Hkv, D]. The new token is appended to both caches, then every head
 * attends (retrieval: positions [0, n]; streaming: the sinks and the last
 * `recent` positions, the new one included). Writes out [B, 1, Hq, D] bf16.
 * Each sequence decodes at its own position n_b when the counts differ.
 * DUO_ERR_CAPACITY if the longest sequence is full. */
duo_status duo_decode(duo_layer* layer, const void* q, const void* k_new, const void* v_new,
                      void* out, hipStream_t stream);

/* duo_append_kv for sequence b alone: k/v [1, n_tokens, Hkv, D] at its
 * positions [n_b, n_b + n_tokens). DUO_ERR_INVALID_ARG for b outside
 * [0, batch) or n_tokens < 1, DUO_ERR_CAPACITY if it would pass the
 * capacity, DUO_ERR_UNSUPPORTED for batches above 64. */
duo_status duo_append_kv_seq(duo_layer* layer, int32_t b, const void* k, const void* v,
                             int32_t n_tokens, hipStream_t stream);

/* duo_prefill_chunk for sequence b alone: q [1, chunk_len, Hq, D], k/v
 * [1, chunk_len, Hkv, D], out [1, chunk_len, Hq, D], at its positions
 * [n_b, n_b + chunk_len). Errors as for duo_append_kv_seq and
 * duo_prefill_chunk. */
duo_status duo_prefill_chunk_seq(duo_layer* layer, int32_t b, const void* q, const void* k,
                                 const void* v, int32_t chunk_len, void* out, hipStream_t stream);

/* Stateless gate-blended forward used for head identification (xllm-io
 * review, section 三 核心公式, 混合注意力, and 检索头识别: one gate per KV
 * head blends full and Lambda-masked attention; paperlayer summary of arXiv
 * 2410.10819v1, section 2 Optimization-based Identification):
 * out_h = alpha[h/G] * full_h + (1 - alpha[h/G]) * streaming_h over one
 * sequence of `seq_len` tokens. q [B, T, Hq, D] bf16, k/v [B, T, Hkv, D]
 * (kv_dtype must be BF16), alpha [Hkv] fp32 on the device; the descriptor's
 * retrieval fields are ignored. A sequence whose K (or V) tensor holds
 * 2^31 bytes or more (seq_len * Hkv * D * 2) returns DUO_ERR_UNSUPPORTED. */
duo_status duo_mixed_forward(const duo_layer_desc* desc, const void* q, const void* k,
                             const void* v, const float* alpha, int32_t seq_len, void* out,
                             hipStream_t stream);

/* duo_mixed_forward with the streaming part under the block-sparse Lambda
 * mask used while training the gates (paperlayer summary of arXiv
 * 2410.10819v1, appendix A.1; its figure is missing, the reading is stated
 * here): with lambda_block = b = 64, query i may attend key j when j <= i and
 * (j / b < ceil(sink / b) or i / b - j / b < ceil(recent / b)) (integer
 * division). lambda_block = 0 is the token-level mask (duo_mixed_forward);
 * other values return DUO_ERR_UNSUPPORTED. */
duo_status duo_mixed_forward_block(const duo_layer_desc* desc, const void* q, const void* k,
                                   const void* v, const float* alpha, int32_t seq_len,
                                   int32_t lambda_block, void* out, hipStream_t stream);

/* Workspace (device memory, 16-byte aligned) that duo_mixed_alpha_grad needs
 * for seq_len tokens: one fp32 partial sum per attention block. Returns 0 for
 * an invalid descriptor or seq_len < 1. */
size_t duo_mixed_alpha_grad_workspace(const duo_layer_desc* desc, int32_t seq_len);

/* Gradient of the head-identification loss with respect to the gates of the
 * gate-blended forward (xllm-io review "DuoAttention: Efficient Long-Context
 * LLM Inference with Retrieval and Streaming Heads", section 三 核心公式:
 * the gate-blended attention, the distillation loss and the L1 term over the
 * gates; 检索头识别: only the gates are trained). With dout [B, T, Hq, D] bf16
 * the gradient of the distillation loss with respect to the gate-blended
 * output, writes
 *   grad_alpha[kv] = sum over the batch, the tokens, the query heads of KV head
 *                    kv and the channels of dout * (full - streaming)
 *                    + l1_weight * sign(alpha[kv])   (sign(0) taken as 0).
 * q/k/v and the size limit as for duo_mixed_forward; alpha and grad_alpha
 * [Hkv] fp32 on the device (alpha enters only through the L1 term). The
 * workspace (device, at least duo_mixed_alpha_grad_workspace bytes) is
 * overwritten; the sum over it runs in a fixed order, so the result is
 * reproducible. A missing, misaligned or short workspace returns
 * DUO_ERR_INVALID_ARG / DUO_ERR_LAYOUT; other errors as for
 * duo_mixed_forward. */
duo_status duo_mixed_alpha_grad(const duo_layer_desc* desc, const void* q, const void* k,
                                const void* v, const void* dout, const float* alpha,
                                float l1_weight, int32_t seq_len, float* grad_alpha,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Host-only: stable permutation that makes retrieval heads contiguous
 * (xllm-io review, section 三 模型部署优化: projection weights reordered so
 * that retrieval and streaming heads form contiguous blocks; section 三 推理流程:
 * the heads are split and concatenated along the head axis).
 * mask[h] != 0 marks KV head h as a retrieval head. perm_out[i] receives the
 * original KV head placed at position i (retrieval heads ascending, then
 * streaming heads ascending); *n_retrieval_out the number of retrieval
 * heads. */
duo_status duo_head_permutation(const uint8_t* mask, int32_t n_kv_heads, int32_t* perm_out,
                                int32_t* n_retrieval_out);

/* duo_mixed_alpha_grad with the block-sparse Lambda mask of
 * duo_mixed_forward_block (lambda_block 0 or 64). */
duo_status duo_mixed_alpha_grad_block(const duo_layer_desc* desc, const void* q, const void* k,
                                      const void* v, const void* dout, const float* alpha,
                                      float l1_weight, int32_t seq_len, int32_t lambda_block,
                                      float* grad_alpha, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* Partial-sum slots of duo_mixed_alpha_grad_noalloc: one per attention block
 * of the flash kernel, B * Hkv * ceil(seq_len / 256) for G = 1,
 * B * Hkv * (G / 2) * ceil(seq_len / 128) for G = 2, and
 * B * Hkv * (G / 4) * ceil(seq_len / 64) for G = 4 or 8 (what
 * duo_mixed_alpha_grad_workspace reports, in floats). */
#define DUO_GRAD_SCRATCH_PARTIALS 65536

/* duo_mixed_alpha_grad_block without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops
 * that forbid hipMalloc). The per-block partial sums go to a file-scope
 * device array of DUO_GRAD_SCRATCH_PARTIALS floats (256 KiB) that each device
 * the library runs on holds until the process ends; its address is looked up
 * on the first call on a device. A launch needing more partial slots returns
 * DUO_ERR_CAPACITY (use duo_mixed_alpha_grad_block with a workspace). Calls
 * on one device share that array: calls that overlap on one device (other
 * streams, other threads) race and must be ordered by the caller. Nothing
 * is allocated; other arguments and errors as for duo_mixed_alpha_grad_block. */
duo_status duo_mixed_alpha_grad_noalloc(const duo_layer_desc* desc, const void* q, const void* k,
                                        const void* v, const void* dout, const float* alpha,
                                        float l1_weight, int32_t seq_len, int32_t lambda_block,
                                        float* grad_alpha, hipStream_t stream);

/* Host-only: retrieval mask from trained gates (xllm-io review, section 三
 * 检索头识别, step 3: alpha is binarized as 1[alpha >= tau]; paperlayer
 * summary, section 2, Binarizing Attention Implementations: tau is the
 * sparsity quantile of the gates). Of the n gates, k = floor(sparsity * n)
 * (in double precision) become streaming heads: tau is the (k+1)-th smallest
 * gate and mask_out[i] = (alpha[i] >= tau), so gates tied with tau stay
 * retrieval heads; k = n marks every head streaming. sparsity must lie in
 * [0, 1]; a NaN gate, n < 1 or a null pointer returns DUO_ERR_INVALID_ARG.
 * mask_out[n] (1 = retrieval) is the caller's. */
duo_status duo_binarize_gates(const float* alpha, int32_t n, double sparsity, uint8_t* mask_out);

/* Host-only: moves whole head blocks of a row-major matrix so that block i of
 * `out` is block perm[i] of `in`, a block being rows_per_head rows of
 * row_bytes bytes. Applied to the query/key/value projection weights (output
 * rows) with the permutation of duo_head_permutation (a KV head's query heads
 * moving together), it makes the retrieval heads contiguous, as the caches
 * here expect (xllm-io review, section 三 模型部署优化). in and out are the
 * caller's host buffers and must not overlap (DUO_ERR_LAYOUT); a perm that is
 * not a permutation of [0, n_heads) returns DUO_ERR_INVALID_ARG. */
duo_status duo_reorder_head_rows(const void* in, void* out, const int32_t* perm, int32_t n_heads,
                                 int64_t rows_per_head, int64_t row_bytes);

/* Host-only: ring slot of token position p (the rule stated above), or -1
 * for invalid arguments. The streaming cache holds the sinks and the most
 * recent tokens (xllm-io review, section 三 推理流程, 解码阶段; paperlayer
 * summary of arXiv 2410.10819v1, section 2); the ring that holds them is
 * this library's layout. */
int32_t duo_ring_slot(int64_t position, int32_t sink, int32_t recent);

/* Static text for a status code. */
const char* duo_status_string(duo_status status);

#ifdef __cplusplus
}
#endif
#endif /* DUO_H_ */
