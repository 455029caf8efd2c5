/*
 * fa.h -- C ABI of the exact tiled attention forward pass for AMD MI355X
 * (gfx950 / CDNA4).
 *
 * The operation (per batch b and head h), as defined on the pages
 * "Build a FlashAttention Kernel from Scratch with Python and NumPy"
 * (Steps 3-5), "Building a FlashAttention-2 Forward Kernel in Pure NumPy"
 * (Architecture Overview, Steps 2-4) and "Python Attention Mechanisms
 * Explained" (The Core Idea; Causal Masking):
 *
 *     s_ij   = (q_i . k_j) / sqrt(D)          for kept keys j
 *     O_i    = sum_j exp(s_ij) v_j / sum_j exp(s_ij)
 *     LSE_i  = ln sum_j exp(s_ij)
 *
 * computed tile by tile with an online softmax (running row max and running
 * exp-sum, rescaled as new key tiles arrive) so that the Nq x Nk score
 * matrix never exists in memory.  Keys kept: all j < Nk, or, with
 * causal != 0, j <= i (diagonal kept, indices aligned at the top-left when
 * Nq != Nk).  Accumulation is fp32 for every dtype; O is rounded to the
 * input dtype with round-to-nearest-even; LSE is fp32 (natural log).
 *
 * Ownership: the caller allocates and owns every buffer.  The library keeps
 * no pointer after a call returns, allocates nothing, copies nothing and
 * does not synchronise; work is enqueued on `stream` and completes
 * asynchronously.  Calls are re-entrant and thread-safe (no global mutable
 * state), except that fa_fwd_splitkv_static calls share one device array per
 * device (see there).  Every element of o and lse is written.
 *
 * Errors: arguments are validated before any work is enqueued; a status
 * other than FA_OK and FA_ERR_HIP means nothing was enqueued.  FA_ERR_HIP
 * reports that the runtime refused a launch of this call (or that no device
 * is current); it comes from the launches' own status, so an error that the
 * caller's earlier HIP work left pending is neither reported nor cleared.
 * Faults during execution surface at the caller's next synchronisation on
 * `stream`.  NaN or Inf inputs are not checked and propagate to the rows
 * they touch.
 *
 * Workgroup shapes (and fa_fwd_splitkv's automatic range count) are chosen
 * against the compute-unit count of the current device, read on every call.
 */
#ifndef FA_H
#define FA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_DTYPE_FP32 = 0, /* IEEE binary32 */
  FA_DTYPE_FP16 = 1, /* IEEE binary16 */
  FA_DTYPE_BF16 = 2  /* bfloat16 */
} fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,     /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,    /* negative size, Nk < 1 with rows to compute, or too large
                          ((N + 256) * D * element size must stay below 2^31 for
                          N = Nq and N = Nk: one head is addressed with 32-bit
                          offsets) */
  FA_ERR_HEAD_DIM = 3, /* D not in {32, 64, 128, 256}; D = 256 with FA_DTYPE_FP32 */
  FA_ERR_DTYPE = 4,    /* unknown dtype code */
  FA_ERR_ALIGN = 5,    /* q, k, v, o not 16-byte aligned, or lse not 4-byte aligned */
  FA_ERR_ALIAS = 6,    /* o or lse overlaps an input, or o overlaps lse */
  FA_ERR_HIP = 7,      /* the HIP runtime refused a launch of this call, or no
                          device is current */
  FA_ERR_SCALE = 8,    /* softmax_scale neither FA_DEFAULT_SCALE nor a finite
                          number > 0 (or so small or large that softmax_scale
                          * log2(e) is not a normal float) */
  FA_ERR_WORKSPACE = 9, /* workspace_bytes below the matching *_workspace_size() */
  FA_ERR_SCRATCH = 10    /* fa_fwd_splitkv_static: the call's partials need more
                            than FA_STATIC_SCRATCH_BYTES */
} fa_status;

/*
 * The softmax_scale value that selects the default scale 1/sqrt(D) in every
 * entry point that takes a scale (every page divides the scores by the
 * square root of the head dimension).
 */
#define FA_DEFAULT_SCALE 0.0

/*
 * fa_fwd -- exact attention forward.
 *
 *   q    device pointer, [B, H, Nq, D] contiguous row-major, `dtype`
 *   k    device pointer, [B, H, Nk, D] contiguous row-major, `dtype`
 *   v    device pointer, [B, H, Nk, D] contiguous row-major, `dtype`
 *   o    device pointer, [B, H, Nq, D] contiguous row-major, `dtype` (output)
 *   lse  device pointer, [B, H, Nq] contiguous fp32 (output, natural log)
 *   B, H, Nq, Nk, D   sizes; D in {32, 64, 128, 256} (256: fp16 and bf16 only).  B*H*Nq == 0 is a valid no-op
 *        (pointers may then be NULL); otherwise Nk >= 1.
 *   causal  0: every key is kept; non-zero: key j kept for query i iff j <= i
 *   dtype   an fa_dtype code
 *   stream  a hipStream_t, or NULL for the null stream
 *
 * All pointers refer to memory of the current HIP device.  Scale is fixed at
 * 1/sqrt(D) (every page divides by the square root of the head dimension).
 * Returns an fa_status code.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
           int causal, int dtype, void* stream);

/*
 * fa_fwd_scaled -- fa_fwd with an explicit softmax scale: s_ij =
 * softmax_scale * (q_i . k_j).  The pages call the library kernel with a
 * softmax_scale argument ("Flash Attention vs Standard Attention",
 * Implementation), set there to 1/sqrt(D); any finite softmax_scale > 0 is
 * accepted (the kernels take the row max of the raw dot products, which
 * commutes with a positive scale), and FA_DEFAULT_SCALE selects 1/sqrt(D).
 * Scores whose scaled value overflows fp32 behave like Inf inputs.  Every other argument, the layouts, the
 * ownership and the errors are those of fa_fwd; an invalid softmax_scale
 * returns FA_ERR_SCALE before any HIP call.  fa_fwd(...) is
 * fa_fwd_scaled(..., FA_DEFAULT_SCALE, ...), i.e. with 1/sqrt(D).
 */
int fa_fwd_scaled(const void* q, const void* k, const void* v, void* o, float* lse,
                  int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                  double softmax_scale, int causal, int dtype, void* stream);

/*
 * fa_fwd_splitkv_workspace_size -- bytes of device workspace fa_fwd_splitkv
 * needs for these sizes and num_splits (0 = automatic, as fa_fwd_splitkv
 * chooses): (D + 1) fp32 values per query row and key range, or 0 when the
 * call runs as one range.  -1 for negative or overflowing sizes or
 * num_splits outside [0, 1024].  The automatic count depends on the current
 * device's compute units: ask with the device current that the call will
 * run on (with no device, the count is planned for 256 compute units).
 */
int64_t fa_fwd_splitkv_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                                      int64_t num_splits);

/*
 * fa_fwd_splitkv -- the same result as fa_fwd_scaled, computed with the keys
 * of every head split into ranges that separate workgroups process in
 * parallel: the shape of decoding with a KV cache ("Python Attention
 * Mechanisms Explained", Causal Masking and Incremental Decoding: a few new
 * query rows against many cached keys), where one workgroup per head and
 * query tile would leave most of the GPU idle.  Each range writes an exact
 * partial (O_s, LSE_s) in fp32 to the workspace; a second kernel combines
 * them with the associative update that folds partial results into one
 * output row ("Building a FlashAttention-2 Forward Kernel in Pure NumPy",
 * Architecture Overview):
 *
 *     LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s.
 *
 *   num_splits  number of key ranges, 0 for automatic (enough workgroups to
 *               fill the current device's compute units, at least 256 keys
 *               a range); at most 1024.  The range length is rounded up to
 *               whole 64-key tiles, so fewer ranges may result; with one
 *               range this is fa_fwd_scaled.
 *   workspace   device memory of fa_fwd_splitkv_workspace_size(...) bytes
 *               (may be NULL when that is 0), 16-byte aligned, owned by the
 *               caller; scratch after the call.
 *
 * Every other argument, layout and error is that of fa_fwd_scaled (every
 * dtype; D = 256 for fp16 and bf16 only), plus FA_ERR_WORKSPACE for a short
 * workspace and FA_ERR_ALIAS if it overlaps an input or output.
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   void* workspace, int64_t workspace_bytes, int64_t B, int64_t H, int64_t Nq,
                   int64_t Nk, int64_t D, double softmax_scale, int64_t num_splits, int causal,
                   int dtype, void* stream);

/* Size of the device scratch that fa_fwd_splitkv_static uses: 32 MiB. */
#define FA_STATIC_SCRATCH_BYTES (32 * 1024 * 1024)

/*
 * fa_fwd_splitkv_static -- fa_fwd_splitkv for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same key ranges, kernels and result,
 * but the fp32 partials go to a scratch array that the library holds in
 * device memory (FA_STATIC_SCRATCH_BYTES on every device it runs on, kept
 * until the process ends) instead of a caller workspace.  The call allocates
 * nothing; the caller still passes every input and output.
 *
 * Every argument, layout and error is that of fa_fwd_splitkv without its
 * workspace arguments, plus FA_ERR_SCRATCH (before anything is enqueued)
 * when the call's partials, fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, D,
 * num_splits) bytes, exceed FA_STATIC_SCRATCH_BYTES: at D = 128 the scratch
 * holds 65027 (query row, key range) partials, e.g. 32 heads x 16 rows x 64
 * ranges.  A call that runs as one range uses no scratch.
 *
 * All calls on one device share its scratch array: calls that overlap in
 * time on one device (on different streams, or from different host threads
 * without ordering) race and may return wrong results; calls on one stream
 * run in order.  Each call writes every partial it reads, so nothing has to
 * be cleared between calls.
 */
int fa_fwd_splitkv_static(const void* q, const void* k, const void* v, void* o, float* lse,
                          int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                          double softmax_scale, int64_t num_splits, int causal, int dtype,
                          void* stream);

/*
 * fa_fwd_varlen -- fa_fwd_scaled over a batch of B packed sequences of
 * different lengths, with no padding: the variable-length batches the pages
 * describe ("Flash Attention vs Standard Attention", Frequently Asked
 * Questions: un-padded sequences processed without padding to the longest
 * one; "Python Attention Mechanisms Explained", Practical Tips for Python
 * Developers: padded positions are skipped).  Sequence b has the query rows [cu_seqlens_q[b],
 * cu_seqlens_q[b+1]) and the key rows [cu_seqlens_k[b], cu_seqlens_k[b+1]);
 * it attends to its own keys only, with the causal mask (if any) aligned at
 * its own first row and key.
 *
 *   q, o  device, [H, total_q, D] contiguous, `dtype` (head-major packing:
 *         each (head, sequence) is one contiguous block of rows)
 *   k, v  device, [H, total_k, D] contiguous, `dtype`
 *   lse   device, [H, total_q] fp32 (output, natural log)
 *   cu_seqlens_q, cu_seqlens_k   device int32 arrays of B + 1 offsets,
 *         non-decreasing from 0 to total_q / total_k.  They are read on the
 *         device only (no copy, no synchronisation); offsets outside
 *         [0, total] are clamped there, so bad offsets give wrong rows but
 *         no access outside the buffers.
 *   max_seqlen_q  at least the longest sequence's query count (it sizes the
 *         grid; query rows past it are not written)
 *   dtype  any fa_dtype (D = 256: fp16 and bf16 only, FA_ERR_HEAD_DIM
 *         otherwise).
 *
 * A sequence with queries but no keys gets O = 0 and LSE = -inf (the empty
 * sum).  B*H == 0, total_q == 0 or max_seqlen_q == 0 is a no-op.  Other
 * errors as fa_fwd_scaled; FA_ERR_SHAPE also for max_seqlen_q > total_q.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int64_t B, int64_t H,
                  int64_t total_q, int64_t total_k, int64_t max_seqlen_q, int64_t D,
                  double softmax_scale, int causal, int dtype, void* stream);

/*
 * fa_bwd_workspace_size -- bytes of device workspace fa_bwd needs: two fp32
 * values per query row (8 * B * H * Nq); -1 if that overflows or a size is
 * negative.  After a call the workspace holds, per query row r (rows in the
 * order of lse), LSE_r log2(e) at float index r and delta_r = sum_d dO_rd O_rd
 * (from the stored values, in fp32) at index rows + r: the statistics of the
 * softmax gradient ("Building a FlashAttention-2 Forward Kernel in Pure
 * NumPy", Extending It), which the gradient kernels read.
 */
int64_t fa_bwd_workspace_size(int64_t B, int64_t H, int64_t Nq);

/*
 * fa_bwd -- exact attention backward: the gradients of sum(dout * O) with
 * respect to q, k and v, where O = attention(q, k, v) as fa_fwd_scaled
 * defines it.  "Building a FlashAttention-2 Forward Kernel in Pure NumPy"
 * (Extending It) names this step: the forward's softmax statistics are kept
 * and every score tile is recomputed while the gradients stream tile by
 * tile.  Here the statistic is lse, so P = exp(s - LSE) exactly, and
 *
 *     dV = P^T dO,  dS = P * (dO V^T - delta),  delta_i = dO_i . O_i,
 *     dQ = scale * dS K,  dK = scale * dS^T Q.
 *
 *   q, k, v   the forward's inputs (device, layouts as fa_fwd)
 *   o, lse    the forward's outputs for these inputs and this scale, exactly
 *             as fa_fwd / fa_fwd_scaled wrote them
 *   dout      device pointer, [B, H, Nq, D], `dtype`: the gradient of O
 *   dq        device pointer, [B, H, Nq, D], `dtype` (output)
 *   dk, dv    device pointers, [B, H, Nk, D], `dtype` (outputs)
 *   workspace device memory of at least fa_bwd_workspace_size(B, H, Nq)
 *             bytes, 16-byte aligned, owned by the caller; its contents on
 *             entry do not matter and are scratch after the call
 *   softmax_scale  the forward's scale: finite and > 0, or FA_DEFAULT_SCALE
 *             for 1/sqrt(D) (fa_fwd's)
 *   causal, dtype, stream   as fa_fwd
 *   B, H, Nq, Nk, D   sizes as fa_fwd; D in {32, 64, 128, 256} (256: fp16
 *             and bf16 only)
 *
 * Accumulation is fp32.  16-bit dtypes: P and dS enter the products rounded
 * to `dtype`, and dq, dk, dv are rounded to it (nearest even); fp32: no
 * rounding between the products.
 * B*H == 0, or Nq == Nk == 0, is a no-op; Nq == 0 < Nk writes dK = dV = 0;
 * Nk == 0 < Nq is FA_ERR_SHAPE.  Keys that no query sees (causal, Nk > Nq)
 * get dK = dV = 0.  Pointers must be non-NULL and 16-byte aligned (lse
 * 4-byte aligned) unless the call is a no-op; when Nq == 0 the query-side
 * buffers (q, o, lse, dout, dq, workspace) are empty and may be NULL.  No
 * output or the workspace may
 * overlap an input or another output (FA_ERR_ALIAS).  Validation happens
 * before any HIP call; the library allocates nothing and keeps no pointer.
 * The result is deterministic (no atomics).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, void* workspace,
           int64_t workspace_bytes, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
           double softmax_scale, int causal, int dtype, void* stream);

/*
 * fa_bwd_varlen -- fa_bwd over packed variable-length sequences: the
 * gradients of sum(dout * O) where O = fa_fwd_varlen(q, k, v, ...) with the
 * same offsets, scale and mask ("Frequently Asked Questions" and "Practical
 * Tips for Python Developers" name packed variable-length batches; each
 * sequence is an independent attention problem, so its gradients are fa_bwd's
 * on its own rows).
 *
 *   q, o, dout, dq   device, [H, total_q, D] contiguous, `dtype`
 *   k, v, dk, dv     device, [H, total_k, D] contiguous, `dtype`
 *   lse              device, [H, total_q] fp32: fa_fwd_varlen's output
 *   cu_seqlens_q, cu_seqlens_k   device int32 [B + 1] offsets, as
 *         fa_fwd_varlen (clamped into [0, total] on the device)
 *   workspace   device memory of at least fa_bwd_workspace_size(1, H,
 *         total_q) bytes, 16-byte aligned, owned by the caller; scratch
 *         after the call
 *   max_seqlen_q, max_seqlen_k   at least the longest sequence's query /
 *         key count (they size the grids; rows past them are not written)
 *   D in {32, 64, 128, 256} (256: fp16 and bf16 only); any fa_dtype
 *
 * A sequence with queries but no keys gets dq = 0; keys of a sequence
 * without queries (or that no query sees under the causal mask) get
 * dk = dv = 0.  Rows outside every sequence are not written.  The buffers of
 * an empty side (total_q == 0: q, o, lse, dout, dq, workspace; total_k == 0:
 * k, v, dk, dv) may be NULL.  Errors as fa_bwd; the offsets arrays are inputs
 * for FA_ERR_ALIAS.  Deterministic (no atomics); the library allocates
 * nothing and keeps no pointer.
 */
int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dout, void* dq, void* dk, void* dv, const int32_t* cu_seqlens_q,
                  const int32_t* cu_seqlens_k, void* workspace, int64_t workspace_bytes, int64_t B,
                  int64_t H, int64_t total_q, int64_t total_k, int64_t max_seqlen_q, int64_t max_seqlen_k,
                  int64_t D, double softmax_scale, int causal, int dtype, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
