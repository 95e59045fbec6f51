/*
 * kdtopk.h -- C ABI of the fused chunked top-K KL distillation loss on AMD
 * MI355X (gfx950).
 *
 * The operation is the loss described in "Distilling an LLM on One GPU:
 * Offline Top-K Logits and a Fused Chunked KL Loss" (section "The two
 * changes") and in "New distillation trick cuts training memory below
 * single-GPU limit for large language models": the student
 * hidden states H[N,D] are projected through the LM head W[V,D] one chunk of
 * positions at a time, each chunk's logits are folded into a running KL loss
 * against an offline teacher cache (top-K token ids and logits per position)
 * and discarded, and the backward pass recomputes each chunk's logits instead
 * of storing them.  No [N,V] logits grid is ever written to device memory.
 *
 * Definitions (fp32 arithmetic on bf16 inputs, fp32 accumulation):
 *   z[n,v]   = (H[n,:] . W[v,:]) / T                       student logits
 *   lse[n]   = log sum_v exp(z[n,v])                        full vocabulary
 *   p[n,k]   = softmax_k(topk_logit[n,:] / T)               teacher, renormalised over K
 *   KL_n     = sum_k p[n,k] (log p[n,k] - z[n,idx[n,k]] + lse[n])   (0 log 0 = 0)
 *   loss     = (1/N) sum_n KL_n
 *   G[n,v]   = g/(N T) (exp(z[n,v] - lse[n]) - sum_{k: idx[n,k]=v} p[n,k]),  g = *grad_loss or 1
 *   dH       = G W          (overwritten, bf16)
 *   dW      += G^T H        (accumulated, fp32)
 *
 * Conventions shared by every entry point:
 *   - All tensors are dense row-major.  bf16 tensors are passed as uint16_t
 *     bit patterns.  Every data pointer is a DEVICE pointer owned by the
 *     caller; the library never allocates, frees or retains device memory.
 *   - H, W, dH and dW must be 16-byte aligned; idx, topk_logit, lse, row_kl
 *     and loss 4-byte aligned.  D must be a multiple of 8.
 *   - Limits: 1 <= K <= min(V, KD_MAX_K); 1 <= V <= KD_MAX_V; N >= 0;
 *     chunk >= 1 (a chunk larger than N is clamped to N; the last chunk may be
 *     ragged); T finite and > 0.  The GEMMs read their bf16 operands with
 *     32-bit byte offsets, so V * D and (clamped chunk) * D must stay below
 *     2^31 - 64 elements; N < 2^31, N * K < 2^31 and D <= 2^20.  Outside these
 *     the calls return KD_ERR_UNSUPPORTED (and the size queries 0).  Any
 *     chunk within them is accepted: the gradient GEMMs of a group of chunks
 *     are split into row blocks whose G rows stay within 32-bit offsets.
 *   - Calls only enqueue work on hip_stream (a hipStream_t, NULL = the null
 *     stream) and return; nothing synchronises the host.  Outputs are valid
 *     when the stream reaches the end of the call.  Asynchronous device
 *     faults surface at the caller's next synchronisation.
 *   - Arguments are checked on the host before any HIP call; an invalid
 *     argument returns a status and enqueues nothing.  KD_ERR_HIP reports a
 *     failed launch; outputs are then unspecified.
 *   - Token ids outside [0, V) give unspecified (but memory-safe) results;
 *     kd_topk_kl_validate detects them.  Duplicate ids within a row act as
 *     one entry holding the summed probability.
 *   - A teacher logit of -inf gives its entry p = 0 (a masked token).  A row
 *     whose K teacher logits are all -inf has no teacher distribution; its
 *     results are unspecified.
 *   - Calls on different streams need distinct workspaces; forward and
 *     backward may share one workspace when issued in order on one stream.
 *   - Results are deterministic: the same inputs give bit-identical outputs
 *     (rows with duplicate ids excepted).
 *
 * Debug aids (off the hot path):
 *   - KD_VALIDATE=1 in the environment (read at every call) makes each entry
 *     point that reads the top-K cache check its ids first, on its stream,
 *     and wait for the answer: an id outside [0, V) returns
 *     KD_ERR_INVALID_IDS before any other work.  Such calls synchronise the
 *     host with the stream and cannot be captured into a HIP graph.
 *   - libkdtopk_debug.so, built beside libkdtopk.so with the same exports,
 *     checks the indices of the cache-entry scatters and gathers on the
 *     device (bucketing, the forward's gather, the backward's scatter)
 *     against the extents they address.  A failed check skips that access;
 *     the top-K forward and backward then wait for their stream at the end
 *     and return KD_ERR_DEBUG_CHECK.  Arithmetic is that of libkdtopk.so.
 */
#ifndef KDTOPK_H
#define KDTOPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KD_MAX_K 256
#define KD_MAX_V (1 << 20)

typedef enum kd_status {
  KD_OK = 0,
  KD_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, bad T */
  KD_ERR_UNSUPPORTED = 2, /* valid but outside this library's limits */
  KD_ERR_WORKSPACE = 3,   /* workspace smaller than kd_topk_kl_workspace_size */
  KD_ERR_HIP = 4,         /* a HIP runtime call or launch failed */
  KD_ERR_INVALID_IDS = 5, /* KD_VALIDATE=1 only: a cached id lies outside [0, V) */
  KD_ERR_DEBUG_CHECK = 6  /* debug library only: a device-side bounds check failed */
} kd_status;

/*
 * Bytes of device workspace that kd_topk_kl_forward and kd_topk_kl_backward
 * need for this problem (one size serves both).  Depends only on the
 * arguments, never on the device.  Returns 0 for arguments that the entry
 * points would reject.  The workspace holds the teacher probabilities and
 * id buckets of one group of consecutive chunks (the fewest whole chunks
 * that hold 8192 positions, at most 8 chunks and at most N positions), the
 * forward's per-vocab-tile softmax partials of one chunk and, for the
 * backward, the bf16 gradient rows G of one group with fp32 split partials
 * for dH when a block of rows is too small to fill the device.  The size is
 * O(R * V + R * K) bytes plus 4 N bytes, where R is the
 * group's rows (at most max(chunk, 8192) rounded to whole chunks): bounded
 * in N, never O(N * V).
 */
size_t kd_topk_kl_workspace_size(int64_t N, int64_t D, int64_t V, int32_t K,
                                 int64_t chunk);

/*
 * Forward pass ("Distilling an LLM on One GPU", section "The two changes":
 * each chunk of positions is projected to logits, added into the running
 * loss and dropped before the next chunk).
 *
 *   H          bf16 [N, D]   student hidden states (read)
 *   W          bf16 [V, D]   LM-head weight, nn.Linear layout (read)
 *   topk_idx   int32 [N, K]  cached teacher token ids (read)
 *   topk_logit fp32 [N, K]   cached teacher logits, any per-row offset (read)
 *   T          temperature applied to student and teacher
 *   chunk      positions per chunk
 *   loss       fp32 [1]      written: mean_n KL_n (0 when N == 0)
 *   lse        fp32 [N]      written: student log-normaliser, needed by backward
 *   row_kl     fp32 [N]      written when not NULL: KL_n per position
 *   workspace  device scratch of workspace_bytes >= kd_topk_kl_workspace_size
 */
kd_status kd_topk_kl_forward(const uint16_t* H, const uint16_t* W,
                             const int32_t* topk_idx, const float* topk_logit,
                             int64_t N, int64_t D, int64_t V, int32_t K, float T,
                             int64_t chunk, float* loss, float* lse, float* row_kl,
                             void* workspace, size_t workspace_bytes,
                             void* hip_stream);

/*
 * Allocation-free forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, results and errors as kd_topk_kl_forward
 * without the workspace: its scratch is a 64 MiB array the library holds in
 * device memory on each GPU it runs on, until the process ends.  Nothing is
 * allocated or freed by the call.
 *   - Problems whose forward workspace region exceeds 64 MiB return
 *     KD_ERR_WORKSPACE before any HIP call.  The region is O(chunk * V / 256
 *     + R * K + N) bytes (R: rows of a group of chunks, see
 *     kd_topk_kl_workspace_size): 25 MiB at N = 262144, V = 131072,
 *     chunk = 4096 and 42 MiB at chunk 8192; chunk 16384 at V = 131072
 *     (83 MiB) does not fit.
 *   - Every call on one GPU uses that GPU's single array: calls that overlap
 *     on one GPU (other streams, other host threads) race and give undefined
 *     results.  Calls on different GPUs are independent.
 *   - The first call on a device looks the array up (hipGetSymbolAddress);
 *     that call's HIP errors return KD_ERR_HIP.
 */
kd_status kd_topk_kl_forward_noalloc(const uint16_t* H, const uint16_t* W,
                                     const int32_t* topk_idx, const float* topk_logit,
                                     int64_t N, int64_t D, int64_t V, int32_t K, float T,
                                     int64_t chunk, float* loss, float* lse, float* row_kl,
                                     void* hip_stream);

/*
 * Backward pass (same section: the backward recomputes every chunk's
 * logits instead of keeping them, so the projection runs twice).
 *
 *   H, W, topk_idx, topk_logit, N, D, V, K, T, chunk   as in the forward
 *   lse        fp32 [N]  from the forward on the same inputs (read)
 *   grad_loss  fp32 [1]  device scalar dLoss_out/dloss, or NULL for 1
 *   dH         bf16 [N, D]  overwritten with G W
 *   dW         fp32 [V, D]  accumulated: dW += G^T H (zero it for a fresh gradient).
 *              Device memory from hipMalloc: the accumulation uses fp32
 *              atomic adds in L2, one per element per dW GEMM, so the result
 *              equals a plain read-modify-write and is deterministic.  Calls
 *              that accumulate into the same dW must be ordered (one stream).
 *   workspace  as in the forward
 */
kd_status kd_topk_kl_backward(const uint16_t* H, const uint16_t* W,
                              const int32_t* topk_idx, const float* topk_logit,
                              const float* lse, const float* grad_loss,
                              int64_t N, int64_t D, int64_t V, int32_t K, float T,
                              int64_t chunk, uint16_t* dH, float* dW,
                              void* workspace, size_t workspace_bytes,
                              void* hip_stream);

/*
 * Loss extensions (the pages report ablations over loss terms and a cost of
 * packing sequences with an all-ones mask: "The $250GB Memory Spike That
 * Killed Distillation Projects Is Now Optional", section "What a Single H200
 * GPU Can Now Do That Once Required Four Nodes").  With z, lse, p and KL_n as
 * above:
 *
 *   CE_n   = lse_n - z[n, y_n]  for a label 0 <= y_n < V, else 0
 *   l_n    = s (kd_weight KL_n + ce_weight CE_n),  s = T^2 with KD_SCALE_T2, else 1
 *   loss   = sum_n w_n l_n / sum_n w_n   (w_n = 1 without row_weight; 0 if the
 *                                         weights sum to 0)
 *   G[n,v] = g s (w_n / sum w) / T ((kd_weight + ce_weight [label]) softmax(z_n)_v
 *            - kd_weight sum_{k: idx=v} p[n,k] - ce_weight [v = y_n])
 *
 *   row_weight  fp32 [N] or NULL (a 0/1 mask, or any finite weights)
 *   labels      int32 [N] or NULL (no cross-entropy term); y_n outside [0, V)
 *               means no label for that position
 *   flags       0 or KD_SCALE_T2
 *   row_loss    fp32 [N] out or NULL: l_n
 * Everything else as in kd_topk_kl_forward / kd_topk_kl_backward (same
 * workspace size).  The plain entry points are the case row_weight = labels =
 * NULL, kd_weight = 1, flags = 0.
 */
enum { KD_SCALE_T2 = 1 };
kd_status kd_topk_kl_forward_ex(const uint16_t* H, const uint16_t* W, const int32_t* topk_idx,
                                const float* topk_logit, int64_t N, int64_t D, int64_t V, int32_t K,
                                float T, int64_t chunk, const float* row_weight, const int32_t* labels,
                                float kd_weight, float ce_weight, int32_t flags, float* loss, float* lse,
                                float* row_loss, void* workspace, size_t workspace_bytes, void* hip_stream);
kd_status kd_topk_kl_backward_ex(const uint16_t* H, const uint16_t* W, const int32_t* topk_idx,
                                 const float* topk_logit, const float* lse, const float* grad_loss,
                                 int64_t N, int64_t D, int64_t V, int32_t K, float T, int64_t chunk,
                                 const float* row_weight, const int32_t* labels, float kd_weight,
                                 float ce_weight, int32_t flags, uint16_t* dH, float* dW, void* workspace,
                                 size_t workspace_bytes, void* hip_stream);

/*
 * Kept-gradient comparator (the "forward-chunked" variant the pages compare
 * against: it keeps what the backward needs instead of recomputing it; "The
 * $250GB Memory Spike That Killed Distillation Projects Is Now Optional",
 * section "What a Single H200 GPU Can Now Do"; "Distilling an LLM on One
 * GPU", section "What this changes in practice").  Same loss and gradients
 * as the entry points above, 6 N D V flops instead of 8, memory O(N V):
 *
 *   kd_topk_kl_forward_keep    as kd_topk_kl_forward (same outputs), and it
 *                              also leaves G / g for all N positions (bf16)
 *                              in the workspace;
 *   kd_topk_kl_backward_keep   dH = g G W (overwritten) and dW += g G^T H from
 *                              that workspace; g = *grad_loss or 1.
 *
 * The workspace (kd_topk_kl_keep_workspace_size bytes, 256-byte aligned,
 * caller-owned) must be the one the forward filled, with the same sizes; it is
 * N * V * 2 bytes plus a chunk's fp32 logits and the forward's buffers.
 */
size_t kd_topk_kl_keep_workspace_size(int64_t N, int64_t D, int64_t V, int32_t K, int64_t chunk);
kd_status kd_topk_kl_forward_keep(const uint16_t* H, const uint16_t* W, const int32_t* topk_idx,
                                  const float* topk_logit, int64_t N, int64_t D, int64_t V, int32_t K,
                                  float T, int64_t chunk, float* loss, float* lse, float* row_kl,
                                  void* workspace, size_t workspace_bytes, void* hip_stream);
kd_status kd_topk_kl_backward_keep(const uint16_t* H, const uint16_t* W, const float* grad_loss,
                                   int64_t N, int64_t D, int64_t V, int32_t K, float T, int64_t chunk,
                                   uint16_t* dH, float* dW, void* workspace, size_t workspace_bytes,
                                   void* hip_stream);

/*
 * Kept-logits comparator: the pages' next-best variant, which chunks the
 * forward but keeps each chunk's logits for the backward instead of
 * recomputing them ("Distilling an LLM on One GPU", section "The two
 * changes": it reaches 134.2 GiB at 256K tokens against 11.6 GiB for the
 * fully chunked loss; "Breaking the Memory Barrier", section "Supporting
 * Context and Metrics").  Same loss and gradients as kd_topk_kl_forward /
 * kd_topk_kl_backward, 6 N D V flops instead of 8, memory O(N V):
 *
 *   kd_topk_kl_forward_keep_logits   as kd_topk_kl_forward, and it also
 *                                    leaves z = (H W^T)/T for all N positions
 *                                    (fp32 [N, Vp], Vp = V rounded up to 256)
 *                                    in the workspace;
 *   kd_topk_kl_backward_keep_logits  as kd_topk_kl_backward, forming each
 *                                    chunk's G from the kept logits (which it
 *                                    overwrites: one backward per forward).
 *
 * The workspace (kd_topk_kl_keep_logits_workspace_size bytes, 256-byte
 * aligned, caller-owned) must be the one the forward filled, with the same
 * sizes: kd_topk_kl_workspace_size plus N * Vp * 4 bytes.
 */
size_t kd_topk_kl_keep_logits_workspace_size(int64_t N, int64_t D, int64_t V, int32_t K, int64_t chunk);
kd_status kd_topk_kl_forward_keep_logits(const uint16_t* H, const uint16_t* W, const int32_t* topk_idx,
                                         const float* topk_logit, int64_t N, int64_t D, int64_t V, int32_t K,
                                         float T, int64_t chunk, float* loss, float* lse, float* row_kl,
                                         void* workspace, size_t workspace_bytes, void* hip_stream);
kd_status kd_topk_kl_backward_keep_logits(const uint16_t* H, const uint16_t* W, const int32_t* topk_idx,
                                          const float* topk_logit, const float* lse, const float* grad_loss,
                                          int64_t N, int64_t D, int64_t V, int32_t K, float T, int64_t chunk,
                                          uint16_t* dH, float* dW, void* workspace, size_t workspace_bytes,
                                          void* hip_stream);

/*
 * Dense-teacher (online) mode: the same fused loss with the teacher's full-
 * vocabulary logits streamed chunk by chunk instead of a top-K cache, i.e.
 * KL(softmax(t/T) || softmax(z/T)) over all V entries (the online
 * distillation setup the cache replaces: "Distilling an LLM on One GPU",
 * section "Why distillation recovery is expensive"; "Breaking the Memory
 * Barrier", section "Detailed Chronology and Technical Evolution").
 *
 *   teacher_logits  [N, V], t_dtype KD_DTYPE_F32 (16-byte aligned) or
 *                   KD_DTYPE_BF16 (8-byte aligned); V % 4 == 0
 *   lse, lse_t      fp32 [N] out (forward) / in (backward): student and
 *                   teacher log-normalisers at temperature T
 *   loss, row_kl, dH, dW, grad_loss, workspace   as in the top-K entry points
 *                   (workspace: kd_dense_kl_workspace_size bytes)
 *
 *   KL_n = sum_v p (a - z/T) - lse_t + lse,  a = t/T,  p = softmax(a);
 *   G = g/(N T) (softmax(z/T) - softmax(t/T)).
 * A row whose teacher logits are all -inf is outside the contract.  The
 * teacher logits are read once in the forward and once in the backward.
 */
size_t kd_dense_kl_workspace_size(int64_t N, int64_t D, int64_t V, int64_t chunk);
kd_status kd_dense_kl_forward(const uint16_t* H, const uint16_t* W, const void* teacher_logits,
                              int32_t t_dtype, int64_t N, int64_t D, int64_t V, float T, int64_t chunk,
                              float* loss, float* lse, float* lse_t, float* row_kl, void* workspace,
                              size_t workspace_bytes, void* hip_stream);
kd_status kd_dense_kl_backward(const uint16_t* H, const uint16_t* W, const void* teacher_logits,
                               int32_t t_dtype, const float* lse, const float* lse_t,
                               const float* grad_loss, int64_t N, int64_t D, int64_t V, float T,
                               int64_t chunk, uint16_t* dH, float* dW, void* workspace,
                               size_t workspace_bytes, void* hip_stream);

/*
 * Debug aid, not on the hot path: checks the teacher cache's ids.
 * d_flags (device int32 [1]) is overwritten with bit 0 set if some id lies
 * outside [0, V) and bit 1 set if some row holds an id twice.
 */
kd_status kd_topk_kl_validate(const int32_t* topk_idx, int64_t N, int32_t K,
                              int64_t V, int32_t* d_flags, void* hip_stream);

/*
 * Teacher top-K cache writer (the offline step before the loss: the teacher
 * runs once and its K largest logits per position are kept; "Distilling an
 * LLM on One GPU", section "The two changes"; "The $250GB Memory Spike That
 * Killed Distillation Projects Is Now Optional", section "Offline Top-K").
 *
 *   logits      [N, V] teacher logits, dtype KD_DTYPE_F32 (float) or
 *               KD_DTYPE_BF16 (uint16_t bf16 bit patterns), row-major
 *   topk_idx    int32 [N, K] out: token ids, best first
 *   topk_logit  fp32  [N, K] out: their logits (bf16 widened exactly; -0.0 is
 *               written as +0.0)
 *
 * Order: larger logit first; equal logits (-0.0 equals +0.0) by lower id, so
 * the result is unique.  NaN logits are outside the contract (memory-safe,
 * result unspecified).  1 <= K <= min(V, KD_MAX_K); V <= 2^31 - 1.  One pass
 * over the logits; no workspace.  Alignment: 4 bytes (fp32) or 2 bytes (bf16);
 * rows whose byte length is a multiple of 16 with a 16-byte aligned base are
 * read with 16-byte loads.  Output rows are written in full.
 */
enum { KD_DTYPE_F32 = 0, KD_DTYPE_BF16 = 1 };
kd_status kd_topk_select(const void* logits, int32_t dtype, int64_t N, int64_t V, int32_t K,
                         int32_t* topk_idx, float* topk_logit, void* hip_stream);

/* Static, human-readable name of a status code. */
const char* kd_status_string(kd_status s);

/*
 * Name of the HIP error (hipGetErrorName) behind the most recent KD_ERR_HIP
 * returned on the calling thread, or "" if there was none.  Static storage;
 * the caller does not free it.
 */
const char* kd_last_hip_error(void);

/*
 * Measurement aids.  kd_profile_enable(mask) makes every later launch of each
 * kernel class i with bit i set in mask (classes KD_KERNEL_*) bracketed by
 * HIP events recorded on the stream it is launched on; mask 0 turns this off.
 * kd_profile_read waits for the recorded events of one class, returns their
 * summed milliseconds and the number of launches since the last read, and
 * clears them.
 */
enum {
  KD_KERNEL_TEACHER = 0,    /* teacher probabilities of a chunk */
  KD_KERNEL_LOGITS_FWD = 1, /* forward logits tile + online softmax / gather epilogue */
  KD_KERNEL_COMBINE = 2,    /* merge of vocab-tile partials into lse and KL per row */
  KD_KERNEL_FINALIZE = 3,   /* mean over positions */
  KD_KERNEL_LOGITS_BWD = 4, /* recomputed logits tile + gradient epilogue */
  KD_KERNEL_DH = 5,         /* dH = G W */
  KD_KERNEL_DH_REDUCE = 6,  /* sum of the dH split partials */
  KD_KERNEL_DW = 7,         /* dW += G^T H */
  KD_KERNEL_BUCKET = 8,     /* cache entries bucketed by tile */
  KD_KERNEL_TOPK_SELECT = 9, /* teacher top-K cache writer */
  KD_KERNEL_KEEP_GRAD = 10, /* kept-gradient mode: G of a chunk from its kept logits */
  KD_KERNEL_COUNT = 11
};
kd_status kd_profile_enable(uint32_t kernel_mask);
kd_status kd_profile_read(int32_t kernel_id, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* KDTOPK_H */
