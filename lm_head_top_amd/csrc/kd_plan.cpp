// Argument checks and workspace layout (host only, no HIP calls).
#include "kd_plan.h"

#include <cmath>

namespace kd {

namespace {
constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
}  // namespace

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int dh_split_for(int64_t c, int64_t D) {
  // Output tiles of dH_c [c, D]; choose the smallest split that fills the
  // reference CU count to >= 90% per round, else the best-filling one.
  const int64_t tiles = ceil_div(c, kTile) * ceil_div(D, kTile);
  int best = 1;
  double best_eff = -1.0;
  for (int s = 1; s <= kMaxDhSplit; ++s) {
    const int64_t wg = tiles * s;
    const int64_t rounds = ceil_div(wg, kRefCUs);
    const double eff = double(wg) / double(rounds * kRefCUs);
    if (wg >= kRefCUs && eff >= 0.9) return s;
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = s;
    }
  }
  return best;
}

int dw_group_for(int64_t c, int64_t N) {
  int g = int((kDwMinK + c - 1) / c);
  if (g > kMaxDwGroup) g = kMaxDwGroup;
  const int64_t nch = N > 0 ? (N + c - 1) / c : 1;
  if (g > nch) g = int(nch);
  return g < 1 ? 1 : g;
}

kd_status make_plan(int64_t N, int64_t D, int64_t V, int32_t K, float T, int64_t chunk,
                    Plan* plan) {
  if (plan == nullptr) return KD_ERR_INVALID_ARG;
  if (N < 0 || D <= 0 || V <= 0 || K <= 0 || chunk <= 0) return KD_ERR_INVALID_ARG;
  if (!std::isfinite(T) || !(T > 0.f)) return KD_ERR_INVALID_ARG;
  if (K > V) return KD_ERR_INVALID_ARG;
  if (D % 8 != 0) return KD_ERR_INVALID_ARG;
  if (K > KD_MAX_K || V > KD_MAX_V) return KD_ERR_UNSUPPORTED;
  if (N > (int64_t(1) << 31) - 1 || D > (int64_t(1) << 20)) return KD_ERR_UNSUPPORTED;
  if (N * int64_t(K) > (int64_t(1) << 31) - 1) return KD_ERR_UNSUPPORTED;

  Plan p;
  p.N = N;
  p.D = D;
  p.V = V;
  p.K = K;
  p.T = T;
  const int64_t c = N > 0 ? (chunk < N ? chunk : N) : (chunk < kTile ? chunk : kTile);
  p.chunk = c;
  p.c_pad = ceil_div(c, kTile) * kTile;
  p.nvt = ceil_div(V, kTile);
  p.Vp = p.nvt * kTile;
  p.npt = p.c_pad / kTile;
  p.dh_split = dh_split_for(c, D);
  p.dw_group = dw_group_for(c, N);
  // Every bf16 GEMM operand is read through a buffer descriptor with 32-bit
  // byte offsets: W [V, D] whole, a chunk's H rows [c, D] in the logits GEMMs,
  // and in dH / dW a block of G rows [rows, Vp] and H rows [rows, D].  W and
  // a chunk of H must fit; the gradient GEMMs of a group are split into row
  // blocks of at most gemm_rows.  (G is written and dW accumulated through
  // 64-bit addresses.)
  constexpr int64_t kLim = (int64_t(1) << 31) - 64;  // elements
  if (V * D > kLim || p.Vp * D > kLim || c * D > kLim) return KD_ERR_UNSUPPORTED;
  int64_t gr = kLim / p.Vp;
  if (kLim / D < gr) gr = kLim / D;
  p.gemm_rows = gr / kTile * kTile;
  if (p.gemm_rows < kTile) return KD_ERR_UNSUPPORTED;
  int64_t dh_rows = p.dw_group * c < kDhRows ? p.dw_group * c : kDhRows;
  if (dh_rows > p.gemm_rows) dh_rows = p.gemm_rows;
  p.grp_pad = ceil_div(dh_rows, kTile) * kTile;
  p.grp_split = dh_split_for(dh_rows, D);

  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  // teacher probabilities, per-row sum p log p, bucket offsets and entries,
  // for the dw_group chunks of a group
  const size_t gch = size_t(p.dw_group);
  p.boff_stride = p.npt * (p.nvt + 1);
  p.ent_stride = p.npt * kTile * (int64_t(K) + 1);  // K cached ids and a label per row
  p.off_p = take(gch * size_t(p.c_pad) * K * 4);
  p.off_h = take(gch * size_t(p.c_pad) * 4);
  p.off_boff = take(gch * size_t(p.boff_stride) * 4);
  p.off_scalar = take(256);  // 1 / sum of the row weights
  p.off_ent = take(gch * size_t(p.ent_stride) * 4);
  const size_t shared_end = off;
  // forward-only region
  p.off_pm = take(size_t(p.nvt) * p.c_pad * 4);
  p.off_ps = take(size_t(p.nvt) * p.c_pad * 4);
  p.off_zsel = take(size_t(p.c_pad) * (K + 1) * 4);
  p.off_rowkl = take(size_t(N > 0 ? N : 1) * 4);
  const size_t fwd_end = off;
  // backward-only region aliases the forward-only one
  off = shared_end;
  // G rows of a group of dw_group consecutive chunks, in position order
  p.off_g = take(size_t(p.dw_group) * c * p.Vp * 2);
  // fp32 split-K partials of one dH GEMM
  p.off_dhp = take(p.grp_split > 1 ? size_t(p.grp_split) * p.grp_pad * D * 4 : 0);
  const size_t bwd_end = off;
  p.fwd_bytes = fwd_end;
  p.bytes = fwd_end > bwd_end ? fwd_end : bwd_end;
  *plan = p;
  return KD_OK;
}

kd_status make_keep_plan(int64_t N, int64_t D, int64_t V, int32_t K, float T, int64_t chunk,
                         KeepPlan* plan) {
  if (plan == nullptr) return KD_ERR_INVALID_ARG;
  KeepPlan kp;
  const kd_status st = make_plan(N, D, V, K, T, chunk, &kp.base);
  if (st != KD_OK) return st;
  const Plan& p = kp.base;
  // the forward-only region ends at off_rowkl + N * 4; everything kept goes after it
  size_t off = align_up(p.off_rowkl + size_t(N > 0 ? N : 1) * 4);
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  kp.off_z = take(size_t(p.chunk) * p.Vp * 4);
  kp.off_gall = take(size_t(N > 0 ? N : 1) * p.Vp * 2);
  kp.off_dhp = take(p.dh_split > 1 ? size_t(p.dh_split) * p.c_pad * D * 4 : 0);
  kp.bytes = off;
  // rows per dW GEMM: G and H are addressed with 32-bit offsets from the block's first row
  kp.dw_rows = N < p.gemm_rows ? (N > 0 ? N : 1) : p.gemm_rows;
  *plan = kp;
  return KD_OK;
}

kd_status make_keep_logits_plan(int64_t N, int64_t D, int64_t V, int32_t K, float T, int64_t chunk,
                                KeepLogitsPlan* plan) {
  if (plan == nullptr) return KD_ERR_INVALID_ARG;
  KeepLogitsPlan kp;
  const kd_status st = make_plan(N, D, V, K, T, chunk, &kp.base);
  if (st != KD_OK) return st;
  kp.off_z = align_up(kp.base.bytes);
  kp.bytes = align_up(kp.off_z + size_t(N > 0 ? N : 1) * size_t(kp.base.Vp) * 4);
  *plan = kp;
  return KD_OK;
}

kd_status make_dense_plan(int64_t N, int64_t D, int64_t V, float T, int64_t chunk, DensePlan* plan) {
  if (plan == nullptr) return KD_ERR_INVALID_ARG;
  if (V % 4 != 0) return KD_ERR_INVALID_ARG;  // the teacher is read 4 logits at a time
  DensePlan dp;
  const kd_status st = make_plan(N, D, V, 1, T, chunk, &dp.base);
  if (st != KD_OK) return st;
  const Plan& p = dp.base;
  size_t off = align_up(p.bytes);
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  const size_t part = size_t(p.nvt) * p.c_pad * 4;
  dp.off_tm = take(part);
  dp.off_ts0 = take(part);
  dp.off_ts1 = take(part);
  dp.bytes = off;
  *plan = dp;
  return KD_OK;
}

}  // namespace kd
