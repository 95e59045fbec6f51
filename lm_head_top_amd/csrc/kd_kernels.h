// Launchers of the gfx950 kernels of the fused chunked top-K KL loss.
// Each launcher enqueues one kernel on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kd_plan.h"

namespace kd {

// Per-chunk teacher side: p = softmax_K(t/T) and h = sum p log p per position.
struct TeacherArgs {
  const float* t;       // [rows, K], offset to the chunk's first row
  int rows, K;
  float invT;
  float* p;             // [c_pad, K]
  float* h;             // [c_pad]
};

// Per-chunk cache entries bucketed by (position tile, vocab tile).
// Buckets the cached ids of a run of consecutive chunks (chunk rows each, the
// last one possibly shorter): block (pt, j) takes position tile pt of chunk j.
struct BucketArgs {
  const int32_t* idx;   // [rows, K], offset to the first chunk's first row
  int rows, K, V, nvt;  // rows: of all the chunks
  int chunk;            // rows per chunk
  int KE;               // entries per row: K, or K + 1 with labels
  const int32_t* labels;  // [rows] hard labels (offset to the first chunk), or null
  int32_t* boff;        // chunk j: [npt, nvt + 1] at j * boff_stride
  uint32_t* ent;        // chunk j: [npt, kTile * KE] at j * ent_stride
  int64_t boff_stride, ent_stride;
};

// The chunk's logits tile kernel: z^T = W H_c^T / T over one (vocab tile,
// position tile), with the forward or the backward epilogue.
struct LogitsArgs {
  const uint16_t* W;    // [V, D]
  const uint16_t* Hc;   // [rows, D], offset to the chunk
  int rows, D, V, K, nvt, npt;
  int64_t c_pad, Vp;
  float invT;
  const int32_t* boff;
  const uint32_t* ent;
  int KE;               // cache entries per row (K, or K + 1 with the label last)
  // dense teacher (full-vocabulary teacher logits instead of the top-K cache)
  const void* tlog;     // [rows, V] teacher logits of the chunk (fp32 or bf16), or null
  int t_dtype;          // 0 fp32, 1 bf16
  float* tm;            // [nvt, c_pad] tile max of t / T
  float* ts0;           // [nvt, c_pad] tile sum exp(a - max)
  float* ts1;           // [nvt, c_pad] tile sum exp(a - max) (a - z)
  const float* lse_t;   // [rows] teacher log-normaliser (backward)
  // forward outputs
  float* zkeep;         // [rows, Vp] fp32 z kept for the kept-gradient mode, or null
  float* pm;            // [nvt, c_pad] tile max of z
  float* ps;            // [nvt, c_pad] tile sum exp(z - max)
  float* zsel;          // [c_pad, K]   z at the cached ids
  // backward inputs / outputs
  const float* lse;     // [rows] offset to the chunk
  const float* p;       // [c_pad, K]
  const float* grad_loss;  // device scalar or null
  float g_scale;        // s / (N T) without row weights, s / T with them (s = T^2 or 1)
  // loss extensions (defaults: no weights, no labels, alpha 1, beta 0)
  const float* row_w;     // [rows] per-position weights, offset to the chunk, or null
  const float* inv_wsum;  // device scalar 1 / sum of all weights (with row_w)
  const int32_t* labels;  // [rows] hard labels, offset to the chunk, or null
  float alpha, beta;      // weights of the KL and the cross-entropy terms
  uint16_t* G;          // [rows, Vp] bf16, offset to the chunk's first row (zero past V)
};

struct DenseCombineArgs {
  const float* pm;
  const float* ps;
  const float* tm;
  const float* ts0;
  const float* ts1;
  int rows, nvt;
  int64_t c_pad;
  float* lse;      // [rows], offset to the chunk
  float* lse_t;    // [rows], offset to the chunk
  float* rowkl;    // [rows], offset to the chunk
};

struct CombineArgs {
  const float* pm;
  const float* ps;
  const float* zsel;    // [c_pad, KE]
  const float* p;
  const float* h;
  int rows, K, nvt;
  int KE, V;
  const int32_t* labels;  // [rows] offset to the chunk, or null
  float alpha, beta, scale;
  int64_t c_pad;
  float* lse;      // [rows], offset to the chunk
  float* rowkl;    // [rows], offset to the chunk
};

struct DhArgs {
  const uint16_t* G;   // [rows, Vp], offset to the block's first row
  const uint16_t* W;   // [V, D]
  int rows, D, V;
  int64_t Vp;
  int split;           // number of K splits
  int ktiles_per_split;
  float* part;         // [split, c_pad, D] (split > 1)
  uint16_t* dH;        // [rows, D] offset to the block (split == 1)
  int64_t c_pad;       // row stride of `part` per split (the block's rows, padded)
  const float* scale;  // device scalar multiplying the result, or null
};

// dW += G^T H over a group of consecutive chunks (their G rows are stored
// one after another, like their H rows).
struct DwArgs {
  const uint16_t* G;   // [rows, Vp], the group's first position
  const uint16_t* H;   // [rows, D], the group's first position
  int rows;            // positions in the group
  int D, V;
  int64_t Vp;
  float* dW;           // [V, D]
  const float* scale;  // device scalar multiplying G^T H, or null
};

int gemm_bk();  // K depth of one GEMM pipeline stage
hipError_t launch_teacher(const TeacherArgs& a, hipStream_t s);
hipError_t launch_bucket(const BucketArgs& a, int npt, int nchunks, hipStream_t s);
hipError_t launch_logits_fwd(const LogitsArgs& a, hipStream_t s);
hipError_t launch_logits_bwd(const LogitsArgs& a, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_finalize(const float* rowl, const float* w, int64_t N, float* loss, float* inv_wsum,
                           hipStream_t s);
hipError_t launch_dense_combine(const DenseCombineArgs& a, hipStream_t s);
hipError_t launch_dh(const DhArgs& a, hipStream_t s);
hipError_t launch_dh_reduce(const float* part, int split, int rows, int D, int64_t c_pad,
                            uint16_t* dH, hipStream_t s);
hipError_t launch_dw(const DwArgs& a, hipStream_t s);
// Kept-gradient mode: G_c = bf16(gs (exp(z - lse) - p scattered at the ids))
// from the chunk's kept fp32 logits z [rows, Vp] (overwritten).
hipError_t launch_keep_grad(float* z, const float* lse, const int32_t* idx, const float* p, int rows, int K,
                            int V, int64_t Vp, float gs, uint16_t* G, hipStream_t s);
hipError_t launch_validate(const int32_t* idx, int64_t N, int K, int64_t V, int32_t* flags,
                           hipStream_t s);
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s);
// Debug builds: waits for s, then returns (and clears) the bits of the
// device-side bounds checks that failed since the last call.  Other builds
// return 0 at once.
hipError_t debug_fault_take(unsigned* bits, hipStream_t s);

// Teacher top-K cache writer: one workgroup per row of logits [N, V] (dtype 0
// fp32, 1 bf16; vec: 16-byte loads allowed).
hipError_t launch_topk_select(const void* logits, int dtype, bool vec, int64_t N, int64_t V, int K,
                              int32_t* idx, float* val, hipStream_t s);

}  // namespace kd
