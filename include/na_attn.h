/*
 * na_attn.h — C ABI of the fused causal multi-head self-attention library
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  nanochat runs every transformer block's attention as
 * flash_attn_func(q, k, v, causal=True, window_size=...) on (B, T, H, D)
 * tensors, FlashAttention-3 on Hopper in bfloat16 with PyTorch SDPA as the
 * fallback elsewhere (apidog blog "ChatGPTを50ドルで独自にトレーニングする方法",
 * section 5 "Flash Attention integration"; the architecture list and the
 * (B, T, n_kv_head, head_dim) view are in section 1 "GPT model").  Chat
 * inference attends one new token per sequence against a prefilled KV cache
 * through flash_attn_with_kvcache (same blog, section 6 "inference engine").
 * Shapes: head dim 128, d20 = 1280 channels = 10 heads (aisight.pl article
 * "Karpathy udostępnia nanochat ...", section "Model i założenia skalowania").
 *
 * Readings fixed by this library (the pages do not write them out):
 *   - scores z_ij = s <q_i, k_j> with s = 1/sqrt(D); softmax over keys;
 *   - causal: key j is visible to query i iff j <= i (T_q = T_k, top left);
 *   - n_kv_head = n_head; full causal window (the *_window entry points
 *     below take a sliding window, the *_gqa ones fewer key/value heads);
 *   - KV caches: na_attn_decode reads a cache that already holds the new
 *     token; na_attn_prefill and na_attn_decode_append write the new rows
 *     first (bottom-right causal alignment for a chunk);
 *   - the prologue (QK norm, rotary embedding, value-embedding gate) has
 *     entry points of its own and is folded into the prefill, the decode
 *     step and, optionally, the backward (na_attn_*_rope, *_append);
 *   - lse_i = ln sum_j exp(z_ij) over visible keys (natural log, fp32);
 *   - bf16 inputs are rounded values; all accumulation is fp32; fp32 -> bf16
 *     conversions round to nearest even.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates device memory; scratch space (delta, the decode
 *     workspace) is passed in.  Inputs are only read (the caches of the
 *     appending calls are read and written); outputs are fully overwritten
 *     (no need to zero them).
 *   - bf16 tensors are stored as 16-bit bfloat16.  Layout of q, k, v, o, dout,
 *     dq, dk, dv: (B, T, H, D) contiguous, element ((b*T + t)*H + h)*D + d.
 *     lse and delta: fp32 (B, H, T) contiguous, element (b*H + h)*T + t.
 *   - D must be 128 (else NA_ERR_UNSUPPORTED).  B, T, H >= 1.  Every pointer
 *     must be 16-byte aligned.  An output may not be the same pointer as an
 *     input (NA_ERR_INVALID_ARG).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work and return without synchronising.  Arguments are checked on
 *     the host before any HIP call; on a check failure nothing is enqueued and
 *     the status says why (na_last_error() gives a message).  A launch failure
 *     returns NA_ERR_HIP.  Device faults surface at the caller's next sync.
 *   - Results are bitwise deterministic (no atomics).  Calls are re-entrant.
 */
#ifndef NA_ATTN_H
#define NA_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int na_status;
#define NA_OK 0
#define NA_ERR_INVALID_ARG 1
#define NA_ERR_UNSUPPORTED 2
#define NA_ERR_HIP 3

/*
 * Forward: o = softmax(s q k^T + causal mask) v and lse, per (b, h).
 * q, k, v: bf16 (B, T, H, D) inputs.  o: bf16 (B, T, H, D) output.
 * lse: fp32 (B, H, T) output (needed by na_attn_bwd).
 */
na_status na_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int T, int H, int D, void* stream);

/*
 * Backward of the forward above for the loss L with dL/do = dout and no
 * gradient through lse:
 *   delta_i = sum_d dout_id o_id          (written to `delta`)
 *   P = exp(s q k^T - lse) (masked), dP = dout v^T, dS = P * (dP - delta)
 *   dv = P^T dout,  dq = s dS k,  dk = s dS^T q.
 * q, k, v, o, dout: bf16 (B, T, H, D) inputs; o and lse are the forward's
 * outputs.  dq, dk, dv: bf16 (B, T, H, D) outputs.  delta: fp32 (B, H, T)
 * caller-provided scratch, holds delta on return.
 * workspace: optional device scratch for dS, at least
 * na_attn_bwd_workspace_bytes(B, T, H, D) bytes (NA_ERR_INVALID_ARG if
 * smaller).  With it, the dk/dv kernel stores dS (bf16) once and dq is a GEMM
 * over it; with workspace == NULL (workspace_bytes ignored) the dq pass
 * recomputes S and dP instead.  Both give the same result up to rounding.
 * Enqueues three kernels: delta, dk/dv (one workgroup per key tile), dq (one
 * per query tile).  The workspace path needs T <= 1048576.
 */
na_status na_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      float* delta, void* workspace, size_t workspace_bytes, int B, int T,
                      int H, int D, void* stream);

/* Bytes of dS workspace for na_attn_bwd (0 if the sizes are invalid): B*H
 * lower-triangular sets of 32 x 32 bf16 blocks, about B*H*T*T bytes. */
size_t na_attn_bwd_workspace_bytes(int B, int T, int H, int D);

/*
 * Decode: one new query per sequence against a padded KV cache.
 * q: bf16 (B, H, D).  k_cache, v_cache: bf16 (B, T_cap, H, D); only rows
 * t < seqlens[b] are read.  seqlens: DEVICE int32[B]; values are clamped to
 * [0, T_cap] on the device (not checked on the host); the query sits at
 * position seqlens[b]-1 and sees keys 0..seqlens[b]-1.  o: bf16 (B, H, D)
 * output; lse: fp32 (B, H) output, or NULL.  A sequence of length 0 gives
 * o = 0 and lse = -inf.  workspace: device scratch of at least
 * na_attn_decode_workspace_bytes(B, H, D, T_cap) bytes (NA_ERR_INVALID_ARG if
 * smaller).  H <= 32 (else NA_ERR_UNSUPPORTED), B <= 65535.  Enqueues two
 * kernels per batch of up to 4096 sequences: split-KV partials over equal
 * ranges of the visible keys, then their combine (the batches reuse the
 * workspace in stream order).
 */
na_status na_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                         const int* seqlens, void* o, float* lse, int B, int H, int D,
                         int T_cap, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of decode workspace needed for these sizes (0 if the sizes are invalid). */
size_t na_attn_decode_workspace_bytes(int B, int H, int D, int T_cap);

/*
 * na_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory: code being captured into a HIP graph, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments (minus workspace),
 * layouts, results and errors as na_attn_decode, and the same kernels; the
 * split-KV partials go to a fixed scratch array of 16 MiB that the library
 * holds in each device's memory until the process ends.  Sizes whose
 * na_attn_decode_workspace_bytes exceed 16 MiB are rejected with
 * NA_ERR_INVALID_ARG before anything is enqueued (the d20 decode shape, B = 64,
 * H = 10, T_cap = 2048, needs 11.0 MB).  Allocates nothing: the first call on
 * a device looks up the scratch's device address (hipGetSymbolAddress) and
 * caches it.  All calls on one device share the scratch: calls that may
 * overlap on one device (different streams without ordering) race and must
 * be serialised by the caller.  Nothing in the scratch needs clearing between
 * calls.
 */
na_status na_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                 const int* seqlens, void* o, float* lse, int B, int H, int D,
                                 int T_cap, void* stream);

/*
 * fp32 twins of the forward and backward (fp32 storage and arithmetic
 * throughout, no bf16 rounding anywhere); same layouts, same conventions.
 * For correctness at fp32 tolerances, not speed.
 */
na_status na_attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int B, int T, int H, int D, void* stream);
na_status na_attn_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                          const float* dout, const float* lse, float* dq, float* dk, float* dv,
                          float* delta, int B, int T, int H, int D, void* stream);

/*
 * Per-kernel timing twins of na_attn_bwd and na_attn_decode: identical work
 * and results, plus hipEventRecord(events[i], stream) right before kernel i
 * and of events[n] after the last kernel, so a caller can time each kernel
 * with HIP events on the stream it runs on.  `events` points to caller-created
 * hipEvent_t handles: 4 for the backward (delta, dk/dv, dq), 3 for the decode
 * (split, combine).  NULL events behaves like the plain entry point.
 */
na_status na_attn_bwd_timed(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, void* dq, void* dk, void* dv,
                            float* delta, void* workspace, size_t workspace_bytes, int B,
                            int T, int H, int D, void* stream, void* const* events);
na_status na_attn_decode_timed(const void* q, const void* k_cache, const void* v_cache,
                               const int* seqlens, void* o, float* lse, int B, int H, int D,
                               int T_cap, void* workspace, size_t workspace_bytes, void* stream,
                               void* const* events);

/*
 * Sliding-window (banded causal) variants.  nanochat alternates short- and
 * long-window layers (the "SSSL" pattern of the blog's section 1 "GPT model")
 * through flash_attn_func's window_size argument (section 5).  The pages give
 * neither the window length nor the argument's convention; here, as in
 * flash-attention's (left, right) = (window, 0) band under a causal mask, key j
 * is visible to query i iff i - window <= j <= i (the query and the `window`
 * keys before it).  Decode: the query sits at row L - 1 of a sequence of
 * length L and sees keys max(0, L - 1 - window) .. L - 1.  window < 0, or a
 * window that reaches key 0 from every row (window >= T - 1, resp.
 * T_cap - 1), is exactly the plain entry point.  The windowed backward runs
 * with or without the dS workspace, as the plain one (without it the dq pass
 * recomputes S and dP over the band).  Arguments,
 * layouts and errors otherwise as for the plain calls; `events` as for the
 * _timed entry points (NULL allowed).
 */
na_status na_attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int T, int H, int D, int window, void* stream);
na_status na_attn_bwd_window(const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             float* delta, void* workspace, size_t workspace_bytes, int B,
                             int T, int H, int D, int window, void* stream,
                             void* const* events);
na_status na_attn_decode_window(const void* q, const void* k_cache, const void* v_cache,
                                const int* seqlens, void* o, float* lse, int B, int H, int D,
                                int T_cap, int window, void* workspace, size_t workspace_bytes,
                                void* stream, void* const* events);

/*
 * Grouped-query attention (fewer key/value heads than query heads, the
 * architecture list of the blog's section 1 "GPT model"): k, v, dk, dv (and
 * the decode caches) have H_kv heads, (B, T, H_kv, D) contiguous; q, o, dout,
 * dq have H heads; H must be a multiple of H_kv (else NA_ERR_INVALID_ARG), and
 * query head h reads key/value head h / (H / H_kv).  dk and dv are the sums
 * over the query heads that read each key/value head.  lse, delta and the
 * workspaces are per query head, sized as for the plain calls with H.
 * H_kv == H is plain multi-head attention; `window` as for the *_window
 * entry points (< 0: none).  bf16 only.
 */
na_status na_attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int T, int H, int H_kv, int D, int window, void* stream);
na_status na_attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv,
                          float* delta, void* workspace, size_t workspace_bytes, int B, int T,
                          int H, int H_kv, int D, int window, void* stream,
                          void* const* events);
na_status na_attn_decode_gqa(const void* q, const void* k_cache, const void* v_cache,
                             const int* seqlens, void* o, float* lse, int B, int H, int H_kv,
                             int D, int T_cap, int window, void* workspace,
                             size_t workspace_bytes, void* stream, void* const* events);

/*
 * Prefill over a KV cache (the inference engine's prefilled prompt cache,
 * flash_attn_with_kvcache, blog section 6): for each sequence b whose caches
 * hold L = cache_lens[b] rows, the T_q new key/value rows k_new[b], v_new[b]
 * are written to cache rows L .. L + T_q - 1, then query row r of q[b] (at
 * position L + r) attends over cache rows 0 .. L + r (with a window, rows
 * L + r - window .. L + r).  The pages do not spell out the alignment; this is
 * flash_attn_with_kvcache's bottom-right causal convention, which reduces to
 * the decode call for T_q = 1 and to the training forward for L = 0.
 * q: bf16 (B, T_q, H, D); k_new, v_new: bf16 (B, T_q, H_kv, D); k_cache,
 * v_cache: bf16 (B, T_cap, H_kv, D), read and written (rows other than
 * L .. L + T_q - 1 are left as they are); cache_lens: DEVICE int32[B], clamped
 * to [0, T_cap - T_q] on the device and not updated (the caller adds T_q).
 * o: bf16 (B, T_q, H, D) output; lse: fp32 (B, H, T_q) output, or NULL.
 * H a multiple of H_kv; T_cap >= T_q.  Enqueues two kernels: the append, then
 * the attention.  bf16 only.
 */
na_status na_attn_prefill(const void* q, const void* k_new, const void* v_new, void* k_cache,
                          void* v_cache, const int* cache_lens, void* o, float* lse, int B,
                          int T_q, int H, int H_kv, int D, int T_cap, int window,
                          void* stream);

/*
 * Attention prologue: QK normalisation and rotary position embedding of the
 * query and key heads, the two steps nanochat applies to q and k before
 * attention (blog section 1 "GPT model", architecture features; the blog gives
 * no formula).  Readings: for each head row x of D elements,
 *   z = x / sqrt(mean(x^2) + eps)                  (RMS norm, no learned scale)
 *   y_i      = z_i cos(th_{p,i}) - z_{i+D/2} sin(th_{p,i})
 *   y_{i+D/2} = z_i sin(th_{p,i}) + z_{i+D/2} cos(th_{p,i}),  i < D/2,
 * at position p = t + clamp(pos_offset[b], 0, T_tab - T) (p = t when
 * pos_offset is NULL).  The angles come in as tables: cos_tab, sin_tab fp32
 * (T_tab, D/2) contiguous, element p*(D/2) + i (the usual choice is
 * th_{p,i} = p * 10000^(-2i/D)); the clamp matches na_attn_prefill's, so a
 * prefill chunk is rotated at its cache positions by passing cache_lens.
 * q: bf16 (B, T, H, D); k: bf16 (B, T, H_kv, D); q_out, k_out: bf16 outputs of
 * the same shapes.  H, H_kv >= 1; T_tab >= T; eps >= 0 and finite.  One
 * kernel; fp32 arithmetic, outputs rounded to nearest even.
 */
na_status na_qk_norm_rope_fwd(const void* q, const void* k, void* q_out, void* k_out,
                              const float* cos_tab, const float* sin_tab, const int* pos_offset,
                              int B, int T, int H, int H_kv, int D, int T_tab, float eps,
                              void* stream);

/*
 * Training forward with the QK prologue folded in (blog section 1 "GPT model":
 * QK norm and rotary embedding ahead of attention; section 5: the attention
 * call): the readings of na_qk_norm_rope_fwd at positions p = t, then the
 * causal attention of na_attn_fwd_gqa (window as there).  q_raw: bf16
 * (B, T, H, D) raw query heads; k_raw: bf16 (B, T, H_kv, D) raw key heads;
 * v: bf16 (B, T, H_kv, D) (the value gate's output where the layer has one).
 * Outputs: q_rot, k_rot, bf16 of the shapes of q_raw, k_raw, the rotated heads
 * (what na_qk_norm_rope_fwd writes as q_out, k_out, up to the rounding of the
 * row's mean square: the operands the backward takes as q, k, e.g. in
 * na_attn_bwd_rope); o, lse as in na_attn_fwd_gqa.  cos_tab, sin_tab: fp32
 * (T_tab, D/2), T_tab >= T; eps >= 0 and finite.  Enqueues two kernels: the
 * key rows' prologue, then the forward, which normalises and rotates each
 * query row as it loads it and writes it to q_rot, so the rotated queries
 * are not read back.  All buffers distinct.
 */
na_status na_attn_fwd_rope(const void* q_raw, const void* k_raw, const void* v,
                           const float* cos_tab, const float* sin_tab, int T_tab, float eps,
                           void* q_rot, void* k_rot, void* o, float* lse, int B, int T, int H,
                           int H_kv, int D, int window, void* stream);

/*
 * Backward of na_qk_norm_rope_fwd: given q, k (the forward's inputs) and
 * dq_rot, dk_rot (the gradients of q_out, k_out, e.g. what na_attn_bwd
 * returns), writes dq, dk (the gradients of q, k):
 *   dz = R^T dy (the rotation by -th),  dx = r (dz - z mean(dz z)),
 *   r = 1 / sqrt(mean(x^2) + eps), recomputed from x.
 * Shapes, tables and checks as in the forward; dq, dk are bf16 outputs.
 */
na_status na_qk_norm_rope_bwd(const void* q, const void* k, const void* dq_rot,
                              const void* dk_rot, void* dq, void* dk, const float* cos_tab,
                              const float* sin_tab, const int* pos_offset, int B, int T, int H,
                              int H_kv, int D, int T_tab, float eps, void* stream);

/*
 * Value-embedding gate (ResFormer value residual; blog section 1 "GPT model",
 * value embeddings): on the layers that carry a value embedding, each
 * key/value head's v is mixed with the embedding ve through a per-head gate
 * that depends on the input,
 *   v_out = v + 3 sigmoid(gate) ve,
 * where gate (B, T, H_kv) holds the logits of the small ve_gate projection
 * (an ordinary matrix product upstream, not part of this call).
 * v, ve, v_out: bf16 (B, T, H_kv, D); gate: bf16 (B, T, H_kv).  One kernel,
 * fp32 arithmetic.
 */
na_status na_value_gate_fwd(const void* v, const void* ve, const void* gate, void* v_out, int B,
                            int T, int H_kv, int D, void* stream);

/*
 * Backward of na_value_gate_fwd given dv_out, the gradient of v_out (e.g. the
 * dv that na_attn_bwd returns): the gradient of v is dv_out itself (nothing is
 * written for it); dve = 3 sigmoid(gate) dv_out (bf16 (B, T, H_kv, D)) and
 * dgate = 3 sigmoid(gate) (1 - sigmoid(gate)) sum_d ve dv_out (bf16
 * (B, T, H_kv)).  One kernel.
 */
na_status na_value_gate_bwd(const void* ve, const void* gate, const void* dv_out, void* dve,
                            void* dgate, int B, int T, int H_kv, int D, void* stream);

/*
 * Backward with the prologue's backward folded in (the training step with QK
 * norm and rotary embedding: na_qk_norm_rope_fwd made q, k from q_raw, k_raw,
 * and na_attn_fwd_gqa ran on q, k, v).  Computes what na_attn_bwd_gqa
 * followed by na_qk_norm_rope_bwd computes, in one pass: dv as in
 * na_attn_bwd_gqa, and dq, dk as the gradients of q_raw and k_raw (each
 * row's dz = R^T g, dx = r (dz - z mean(dz z)) applied in the epilogues that
 * write dq and dk, with positions t, tables fp32 (T_tab >= T, D/2)).
 * q, k: the rotated heads (the forward's inputs); q_raw, k_raw: the
 * prologue's inputs, same layouts.  The dS workspace is required.
 * ve, gate, dve, dgate: all NULL, or all given when v is the value-embedding
 * gate's output v' = v + 3 sigmoid(gate) ve (na_value_gate_fwd; blog
 * section 1, value embeddings): then the kernel that writes dv (= dv') also
 * writes dve and dgate, exactly what na_value_gate_bwd(ve, gate, dv) writes
 * (ve, dve bf16 (B, T, H_kv, D); gate, dgate bf16 (B, T, H_kv)).  Other
 * arguments as in na_attn_bwd_gqa.
 */
na_status na_attn_bwd_rope(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, const void* q_raw,
                           const void* k_raw, const float* cos_tab, const float* sin_tab,
                           int T_tab, float eps, const void* ve, const void* gate, void* dq,
                           void* dk, void* dv, void* dve, void* dgate, float* delta,
                           void* workspace, size_t workspace_bytes, int B, int T, int H,
                           int H_kv, int D, int window, void* stream);

/*
 * Prefill with the prologue folded in: as na_attn_prefill, but q and k_new
 * hold the raw query and key heads, and each head row is RMS-normalised and
 * rotated (the readings of na_qk_norm_rope_fwd) at its cache position on the
 * way: key row t of sequence b at position L + t as it is appended (the cache
 * receives the rotated bf16 row), query row r at position L + r as the
 * attention loads it, with L = cache_lens[b] clamped to [0, T_cap - T_q].
 * Equal, up to rounding, to na_qk_norm_rope_fwd on q and k_new with
 * pos_offset = cache_lens followed by na_attn_prefill, without the round trip
 * of the rotated q and k_new through memory.  cos_tab, sin_tab: fp32
 * (T_tab, D/2), T_tab >= T_cap; eps >= 0 and finite.
 * ve, gate: the value-embedding gate (blog section 1, value embeddings), both
 * or neither: with them each value row is appended as
 * v_new + 3 sigmoid(gate) ve (ve bf16 (B, T_q, H_kv, D), gate bf16 logits
 * (B, T_q, H_kv), as in na_value_gate_fwd); without them (NULL) v_new is
 * appended as is.  Other arguments, checks and outputs as in
 * na_attn_prefill.
 */
na_status na_attn_prefill_rope(const void* q, const void* k_new, const void* v_new,
                               void* k_cache, void* v_cache, const int* cache_lens,
                               const float* cos_tab, const float* sin_tab, int T_tab, float eps,
                               const void* ve, const void* gate, void* o, float* lse, int B,
                               int T_q, int H, int H_kv, int D, int T_cap, int window,
                               void* stream);

/*
 * Decode step with the append (the inference engine's per-token call of
 * flash_attn_with_kvcache with the new key and value, blog section 6): for
 * each sequence b, the new token's key/value rows k_new[b], v_new[b] are
 * written to cache row L = seqlens[b] (rows already cached; clamped to
 * [0, T_cap - 1] on the device, not updated: the caller adds 1), then the
 * query attends over rows 0 .. L (with a window, L - window .. L) exactly as
 * na_attn_decode_gqa over L + 1 rows.
 * Optional prologue, as in na_attn_prefill_rope: with cos_tab, sin_tab (fp32
 * (T_tab, D/2), T_tab >= T_cap; both or neither) q and k_new are raw heads,
 * RMS-normalised (eps) and rotated at position L (k_new in the append, q as
 * the decode loads it); with ve, gate (bf16 (B, H_kv, D) and (B, H_kv); both
 * or neither) the value row is appended as v_new + 3 sigmoid(gate) ve.
 * q: bf16 (B, H, D); k_new, v_new: bf16 (B, H_kv, D); caches bf16
 * (B, T_cap, H_kv, D), read and written (only row L changes).  o, lse,
 * workspace and the limits as in na_attn_decode.  Enqueues three kernels:
 * the append, the split and the combine.
 */
na_status na_attn_decode_append(const void* q, const void* k_new, const void* v_new,
                                void* k_cache, void* v_cache, const int* seqlens,
                                const float* cos_tab, const float* sin_tab, int T_tab, float eps,
                                const void* ve, const void* gate, void* o, float* lse, int B,
                                int H, int H_kv, int D, int T_cap, int window, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* na_status_string(na_status s);

/* Message for the last failing call on this thread ("" if none). */
const char* na_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* NA_ATTN_H */
