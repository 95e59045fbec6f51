// Host-side problem plan: argument checks, tiling constants and the
// workspace layout of the fused chunked top-K KL loss.  Pure C++ (no HIP), so
// the checks can be exercised on a machine without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "kdtopk.h"

namespace kd {

// Tile sizes shared by the plan and the kernels.
constexpr int kTile = 256;          // vocab rows / positions / D columns per GEMM tile
constexpr int kMaxVocabTiles = KD_MAX_V / kTile;
constexpr int kMaxDhSplit = 8;      // split-K factor ceiling for dH = G W
constexpr int kRefCUs = 256;        // CU count the dH split is sized for (fixed, so plans are device independent)

struct Plan {
  int64_t N = 0, D = 0, V = 0, chunk = 0;
  int32_t K = 0;
  float T = 1.f;
  int64_t c_pad = 0;   // chunk rounded up to kTile
  int64_t nvt = 0;     // vocab tiles
  int64_t Vp = 0;      // V rounded up to kTile (row stride of G)
  int64_t npt = 0;     // position tiles per chunk
  int dh_split = 1;    // split-K factor of a dH GEMM over one chunk (the kept-gradient comparator)
  int dw_group = 1;    // consecutive chunks whose G rows feed one dW GEMM (K = dw_group * chunk)
  int64_t gemm_rows = 0; // most rows of G (and H) one dH or dW GEMM may take: its operands are
                         // addressed with 32-bit buffer offsets (rows * Vp and rows * D below 2^31
                         // elements); a group's GEMMs are split into row blocks of at most this
  int64_t grp_pad = 0; // rows of one dH GEMM over a group: min(group rows, kDhRows, gemm_rows), rounded up to kTile
  int grp_split = 1;   // split-K factor of such a dH GEMM
  // The teacher probabilities and the id buckets are formed for a group of
  // dw_group chunks at once: chunk j of a group has its p and h rows at
  // j * chunk and its bucket offsets and entries at j * boff_stride and
  // j * ent_stride (elements).
  int64_t boff_stride = 0;  // npt * (nvt + 1)
  int64_t ent_stride = 0;   // npt * kTile * (K + 1)
  // workspace byte offsets
  size_t off_p = 0, off_h = 0, off_boff = 0, off_ent = 0, off_scalar = 0;  // shared by fwd and bwd
  size_t off_pm = 0, off_ps = 0, off_zsel = 0, off_rowkl = 0;  // forward only
  size_t off_g = 0, off_dhp = 0;  // backward only (aliases forward); dhp: [grp_split, grp_pad, D]
  size_t fwd_bytes = 0;  // the part of the workspace the forward uses (shared and forward-only regions)
  size_t bytes = 0;
};

// Kept-gradient mode (the comparator that keeps G for the backward instead of
// recomputing it): the forward region of the plan, the chunk's fp32 logits,
// G for all N positions (bf16 [N, Vp]) and the dH split partials.
struct KeepPlan {
  Plan base;
  size_t off_z = 0, off_gall = 0, off_dhp = 0, bytes = 0;
  int64_t dw_rows = 0;  // positions per dW GEMM (32-bit buffer offsets into G and H)
};

kd_status make_keep_plan(int64_t N, int64_t D, int64_t V, int32_t K, float T, int64_t chunk,
                         KeepPlan* plan);

// Kept-logits mode (the comparator that keeps every chunk's fp32 logits from
// the forward for the backward, which then skips the recompute GEMM): the
// plan of the top-K path plus z for all N positions, fp32 [N, Vp].
struct KeepLogitsPlan {
  Plan base;
  size_t off_z = 0, bytes = 0;
};

kd_status make_keep_logits_plan(int64_t N, int64_t D, int64_t V, int32_t K, float T, int64_t chunk,
                                KeepLogitsPlan* plan);

// Dense-teacher mode (full-vocabulary teacher logits streamed per chunk
// instead of a top-K cache): the plan of the top-K path with K = 1 (its cache
// buffers go unused) plus the teacher's per-tile partials.
struct DensePlan {
  Plan base;
  size_t off_tm = 0, off_ts0 = 0, off_ts1 = 0, bytes = 0;
};

kd_status make_dense_plan(int64_t N, int64_t D, int64_t V, float T, int64_t chunk, DensePlan* plan);

// Fills `plan` from the problem sizes.  Returns KD_OK or the reason the sizes
// are rejected.  Does not look at pointers.
kd_status make_plan(int64_t N, int64_t D, int64_t V, int32_t K, float T, int64_t chunk,
                    Plan* plan);

// Split-K factor of a dH GEMM (G W) over `c` rows and hidden size D.
int dh_split_for(int64_t c, int64_t D);

// Chunks per group (one dH and one dW GEMM): enough that K = group * chunk
// reaches kDwMinK, so the fp32 dW read-modify-write (8 bytes per output
// element) is amortised over at least 2 * kDwMinK flops per element; capped
// at kMaxDwGroup.  8192 positions measured 2% faster per step than 4096 at
// the toy and long-context workloads, for 1 GiB more workspace at V = 131072.
#ifndef KD_DW_MIN_K
#define KD_DW_MIN_K 8192
#endif
constexpr int64_t kDwMinK = KD_DW_MIN_K;
#ifndef KD_MAX_DW_GROUP
#define KD_MAX_DW_GROUP 8
#endif
constexpr int kMaxDwGroup = KD_MAX_DW_GROUP;
int dw_group_for(int64_t c, int64_t N);

// Rows per dH GEMM within a group: one round of 256 x 256 tiles at D = 4096
// (a group of 8192 rows in one GEMM streams each XCD's G strips twice, and
// measured slower).
constexpr int64_t kDhRows = 4096;

// Pointer checks shared by the entry points.
bool aligned(const void* p, size_t a);

}  // namespace kd
