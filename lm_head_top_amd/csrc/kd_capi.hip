// C ABI of the fused chunked top-K KL loss: argument checks, the chunk loop
// and kernel launches on the caller's stream.  Declared in include/kdtopk.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "kd_kernels.h"
#include "kd_plan.h"
#include "kdtopk.h"

namespace {

// ---- optional per-kernel event timing (measurement aid) ----
std::mutex g_prof_mu;
uint32_t g_prof_mask = 0;
struct EventPair {
  hipEvent_t a, b;
};
std::vector<EventPair> g_prof_events[KD_KERNEL_COUNT];

template <class F>
hipError_t timed(int id, hipStream_t s, F&& launch) {
  uint32_t mask;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    mask = g_prof_mask;
  }
  if (!(mask & (1u << id))) return launch();
  EventPair ev{nullptr, nullptr};
  auto drop = [&ev](hipError_t err) {
    if (ev.a != nullptr) (void)hipEventDestroy(ev.a);
    if (ev.b != nullptr) (void)hipEventDestroy(ev.b);
    return err;
  };
  hipError_t e = hipEventCreate(&ev.a);
  if (e == hipSuccess) e = hipEventCreate(&ev.b);
  if (e == hipSuccess) e = hipEventRecord(ev.a, s);
  if (e != hipSuccess) return drop(e);
  e = launch();
  if (e != hipSuccess) return drop(e);
  e = hipEventRecord(ev.b, s);
  if (e != hipSuccess) return drop(e);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_events[id].push_back(ev);
  return hipSuccess;
}

// The HIP error behind the calling thread's most recent KD_ERR_HIP.
thread_local hipError_t t_last_hip = hipSuccess;

kd_status hip_failed(hipError_t e) {
  t_last_hip = e;
  return KD_ERR_HIP;
}

#define KD_LAUNCH(id, stream, call)                                    \
  do {                                                                 \
    const hipError_t kd_e_ = timed((id), (stream), [&] { return (call); }); \
    if (kd_e_ != hipSuccess) return hip_failed(kd_e_);                 \
  } while (0)

bool bad_ptr(const void* p, size_t align) { return p == nullptr || !kd::aligned(p, align); }

// KD_VALIDATE=1 in the environment (read at every call): the top-K entry
// points first check the cache's ids on their stream and wait for the answer.
bool validate_requested() {
  const char* v = std::getenv("KD_VALIDATE");
  return v != nullptr && v[0] == '1' && v[1] == '\0';
}

// The ids check of KD_VALIDATE=1 (flags: a device int32 the call may use).
kd_status validate_if_requested(const int32_t* topk_idx, int64_t N, int32_t K, int64_t V, int32_t* flags,
                                hipStream_t s) {
  if (topk_idx == nullptr || N == 0 || !validate_requested()) return KD_OK;
  hipError_t e = kd::launch_validate(topk_idx, N, K, V, flags, s);
  int32_t h = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&h, flags, sizeof h, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_failed(e);
  return (h & 1) != 0 ? KD_ERR_INVALID_IDS : KD_OK;
}

// End of a top-K call: in debug builds, waits for the stream and reports a
// failed device-side bounds check; otherwise KD_OK at once.
kd_status debug_done(hipStream_t s) {
  unsigned bits = 0;
  const hipError_t e = kd::debug_fault_take(&bits, s);
  if (e != hipSuccess) return hip_failed(e);
  return bits != 0 ? KD_ERR_DEBUG_CHECK : KD_OK;
}

}  // namespace

extern "C" {

const char* kd_status_string(kd_status s) {
  // A C caller may pass any int; in C++ an enum value outside the
  // enumerators' range is undefined, so read the bits as an int.
  static_assert(sizeof(kd_status) == sizeof(int), "kd_status is an int");
  int v;
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case KD_OK:
      return "ok";
    case KD_ERR_INVALID_ARG:
      return "invalid argument";
    case KD_ERR_UNSUPPORTED:
      return "unsupported problem size";
    case KD_ERR_WORKSPACE:
      return "workspace too small";
    case KD_ERR_HIP:
      return "HIP launch failed";
    case KD_ERR_INVALID_IDS:
      return "cached id outside [0, V)";
    case KD_ERR_DEBUG_CHECK:
      return "device bounds check failed";
  }
  return "unknown status";
}

const char* kd_last_hip_error(void) {
  return t_last_hip == hipSuccess ? "" : hipGetErrorName(t_last_hip);
}

size_t kd_topk_kl_workspace_size(int64_t N, int64_t D, int64_t V, int32_t K, int64_t chunk) {
  kd::Plan p;
  if (kd::make_plan(N, D, V, K, 1.f, chunk, &p) != KD_OK) return 0;
  return p.bytes;
}

}  // extern "C"

namespace {

// Loss extensions: per-position weights, hard labels mixed in with weight
// beta beside the KL term's alpha, and an overall factor (T^2 or 1).
struct LossExt {
  const float* row_w = nullptr;
  const int32_t* labels = nullptr;
  float alpha = 1.f, beta = 0.f, scale = 1.f;
};

// Teacher probabilities and id buckets for the group of chunks that starts
// at row0: up to p.dw_group chunks, one launch each over all of them.  Chunk
// j's rows sit at j * chunk in pw / hw and its buckets at j * boff_stride /
// j * ent_stride.
kd_status prepare_group(const kd::Plan& p, const int32_t* topk_idx, const float* topk_logit,
                        const int32_t* labels, int64_t N, int64_t V, int32_t K, int KE, float invT,
                        int64_t row0, float* pw, float* hw, int32_t* boff, uint32_t* ent, hipStream_t s) {
  const int64_t span = int64_t(p.dw_group) * p.chunk;
  const int grows = int(N - row0 < span ? N - row0 : span);
  const int nch = int((grows + p.chunk - 1) / p.chunk);
  kd::TeacherArgs ta{topk_logit + row0 * K, grows, K, invT, pw, hw};
  KD_LAUNCH(KD_KERNEL_TEACHER, s, kd::launch_teacher(ta, s));
  kd::BucketArgs ba{};
  ba.idx = topk_idx + row0 * K;
  ba.rows = grows;
  ba.K = K;
  ba.V = int(V);
  ba.nvt = int(p.nvt);
  ba.chunk = int(p.chunk);
  ba.KE = KE;
  ba.labels = labels != nullptr ? labels + row0 : nullptr;
  ba.boff = boff;
  ba.ent = ent;
  ba.boff_stride = p.boff_stride;
  ba.ent_stride = p.ent_stride;
  KD_LAUNCH(KD_KERNEL_BUCKET, s, kd::launch_bucket(ba, int(p.npt), nch, s));
  return KD_OK;
}

// The forward's chunk loop.  With zkeep / gall set (kept-gradient mode) each
// chunk's fp32 logits are kept and turned into its G rows of gall.  With
// zall set (kept-logits mode) every chunk's fp32 logits are kept in zall
// [N, Vp] for the backward.
kd_status run_forward(const kd::Plan& p, const uint16_t* H, const uint16_t* W, const int32_t* topk_idx,
                      const float* topk_logit, int64_t N, int64_t D, int64_t V, int32_t K, float T,
                      float* loss, float* lse, float* row_kl, char* ws, float* zkeep, uint16_t* gall,
                      hipStream_t s, const LossExt& ext = LossExt(), float* zall = nullptr) {
  float* pw = reinterpret_cast<float*>(ws + p.off_p);
  float* hw = reinterpret_cast<float*>(ws + p.off_h);
  int32_t* boff = reinterpret_cast<int32_t*>(ws + p.off_boff);
  uint32_t* ent = reinterpret_cast<uint32_t*>(ws + p.off_ent);
  float* pm = reinterpret_cast<float*>(ws + p.off_pm);
  float* ps = reinterpret_cast<float*>(ws + p.off_ps);
  float* zsel = reinterpret_cast<float*>(ws + p.off_zsel);
  float* rowkl = row_kl != nullptr ? row_kl : reinterpret_cast<float*>(ws + p.off_rowkl);
  const float invT = 1.f / T;
  const float g_scale = float(1.0 / (double(N) * double(T)));
  {
    const kd_status vs =
        validate_if_requested(topk_idx, N, K, V, reinterpret_cast<int32_t*>(ws + p.off_scalar + 64), s);
    if (vs != KD_OK) return vs;
  }

  const int KE = K + (ext.labels != nullptr ? 1 : 0);
  int gj = 0;  // chunk within its group
  for (int64_t row0 = 0; row0 < N; row0 += p.chunk) {
    const int rows = int(N - row0 < p.chunk ? N - row0 : p.chunk);
    const int npt = (rows + kd::kTile - 1) / kd::kTile;
    if (gj == 0) {
      const kd_status st =
          prepare_group(p, topk_idx, topk_logit, ext.labels, N, V, K, KE, invT, row0, pw, hw, boff, ent, s);
      if (st != KD_OK) return st;
    }
    float* const pc = pw + int64_t(gj) * p.chunk * K;
    float* const hc = hw + int64_t(gj) * p.chunk;
    int32_t* const boffc = boff + gj * p.boff_stride;
    uint32_t* const entc = ent + gj * p.ent_stride;
    gj = gj + 1 == p.dw_group ? 0 : gj + 1;
    kd::LogitsArgs la{};
    la.KE = KE;
    la.W = W;
    la.Hc = H + row0 * D;
    la.rows = rows;
    la.D = int(D);
    la.V = int(V);
    la.K = K;
    la.nvt = int(p.nvt);
    la.npt = npt;
    la.c_pad = p.c_pad;
    la.Vp = p.Vp;
    la.invT = invT;
    la.boff = boffc;
    la.ent = entc;
    la.zkeep = zall != nullptr ? zall + row0 * p.Vp : zkeep;
    la.pm = pm;
    la.ps = ps;
    la.zsel = zsel;
    KD_LAUNCH(KD_KERNEL_LOGITS_FWD, s, kd::launch_logits_fwd(la, s));
    kd::CombineArgs ca{};
    ca.pm = pm;
    ca.ps = ps;
    ca.zsel = zsel;
    ca.p = pc;
    ca.h = hc;
    ca.rows = rows;
    ca.K = K;
    ca.nvt = int(p.nvt);
    ca.KE = KE;
    ca.V = int(V);
    ca.labels = ext.labels != nullptr ? ext.labels + row0 : nullptr;
    ca.alpha = ext.alpha;
    ca.beta = ext.beta;
    ca.scale = ext.scale;
    ca.c_pad = p.c_pad;
    ca.lse = lse + row0;
    ca.rowkl = rowkl + row0;
    KD_LAUNCH(KD_KERNEL_COMBINE, s, kd::launch_combine(ca, s));
    if (zkeep != nullptr)
      KD_LAUNCH(KD_KERNEL_KEEP_GRAD, s,
                kd::launch_keep_grad(zkeep, lse + row0, topk_idx + row0 * K, pc, rows, K, int(V), p.Vp,
                                     g_scale, gall + row0 * p.Vp, s));
  }
  KD_LAUNCH(KD_KERNEL_FINALIZE, s, kd::launch_finalize(rowkl, ext.row_w, N, loss, nullptr, s));
  return debug_done(s);
}

// The backward's chunk loop: recompute each chunk's logits and form G_c (top-K
// cache, or a dense teacher when tlog is set); every dw_group chunks, dH of
// the group = G W and dW += G^T H.
kd_status run_backward(const kd::Plan& p, const uint16_t* H, const uint16_t* W, const int32_t* topk_idx,
                       const float* topk_logit, const void* tlog, int t_dtype, const float* lse,
                       const float* lse_t, const float* grad_loss, int64_t N, int64_t D, int64_t V,
                       int32_t K, float T, uint16_t* dH, float* dW, char* ws, hipStream_t s,
                       const LossExt& ext = LossExt(), float* zall = nullptr) {
  float* pw = reinterpret_cast<float*>(ws + p.off_p);
  float* hw = reinterpret_cast<float*>(ws + p.off_h);
  int32_t* boff = reinterpret_cast<int32_t*>(ws + p.off_boff);
  uint32_t* ent = reinterpret_cast<uint32_t*>(ws + p.off_ent);
  uint16_t* G = reinterpret_cast<uint16_t*>(ws + p.off_g);
  float* dhp = reinterpret_cast<float*>(ws + p.off_dhp);
  float* inv_wsum = reinterpret_cast<float*>(ws + p.off_scalar);
  const float invT = 1.f / T;
  // the per-row factor is 1/N without weights, w_n / sum w with them
  const float g_scale = ext.row_w != nullptr ? float(double(ext.scale) / double(T))
                                             : float(double(ext.scale) / (double(N) * double(T)));
  const int ktiles = int(p.Vp / kd::gemm_bk());
  const int kps = (ktiles + p.grp_split - 1) / p.grp_split;
  const size_t esz = t_dtype == KD_DTYPE_F32 ? 4 : 2;
  if (tlog == nullptr) {
    const kd_status vs =
        validate_if_requested(topk_idx, N, K, V, reinterpret_cast<int32_t*>(ws + p.off_scalar + 64), s);
    if (vs != KD_OK) return vs;
  }
  if (ext.row_w != nullptr)
    KD_LAUNCH(KD_KERNEL_FINALIZE, s, kd::launch_finalize(nullptr, ext.row_w, N, nullptr, inv_wsum, s));
  const int KE = K + (ext.labels != nullptr ? 1 : 0);

  // The G rows of up to dw_group consecutive chunks are kept one after
  // another (position order, row stride Vp) and feed one dH GEMM (the group's
  // rows of dH) and one dW GEMM with K = the group's positions; H rows of the
  // group are consecutive in H already.
  int gj = 0;
  int64_t group_row0 = 0;
  for (int64_t row0 = 0; row0 < N; row0 += p.chunk) {
    const int rows = int(N - row0 < p.chunk ? N - row0 : p.chunk);
    const int npt = (rows + kd::kTile - 1) / kd::kTile;
    if (gj == 0) group_row0 = row0;
    uint16_t* Gc = G + (row0 - group_row0) * p.Vp;
    kd::LogitsArgs la{};
    if (tlog == nullptr) {
      if (gj == 0) {
        const kd_status st =
            prepare_group(p, topk_idx, topk_logit, ext.labels, N, V, K, KE, invT, row0, pw, hw, boff, ent, s);
        if (st != KD_OK) return st;
      }
      la.boff = boff + gj * p.boff_stride;
      la.ent = ent + gj * p.ent_stride;
      la.p = pw + int64_t(gj) * p.chunk * K;
    } else {
      la.tlog = static_cast<const char*>(tlog) + row0 * V * esz;
      la.t_dtype = t_dtype;
      la.lse_t = lse_t + row0;
    }
    la.W = W;
    la.Hc = H + row0 * D;
    la.rows = rows;
    la.D = int(D);
    la.V = int(V);
    la.K = K;
    la.nvt = int(p.nvt);
    la.npt = npt;
    la.c_pad = p.c_pad;
    la.Vp = p.Vp;
    la.invT = invT;
    la.lse = lse + row0;
    la.grad_loss = grad_loss;
    la.g_scale = g_scale;
    la.KE = KE;
    la.row_w = ext.row_w != nullptr ? ext.row_w + row0 : nullptr;
    la.inv_wsum = inv_wsum;
    la.labels = ext.labels != nullptr ? ext.labels + row0 : nullptr;
    la.alpha = ext.alpha;
    la.beta = ext.beta;
    la.G = Gc;
    if (zall != nullptr) {
      // kept-logits mode: G_c = bf16((softmax - p scattered) / (N T)) from the
      // chunk's fp32 logits the forward kept (overwritten); grad_loss scales
      // the dH and dW GEMMs below
      KD_LAUNCH(KD_KERNEL_KEEP_GRAD, s,
                kd::launch_keep_grad(zall + row0 * p.Vp, lse + row0, topk_idx + row0 * K, la.p, rows, K,
                                     int(V), p.Vp, float(1.0 / (double(N) * double(T))), Gc, s));
    } else {
      KD_LAUNCH(KD_KERNEL_LOGITS_BWD, s, kd::launch_logits_bwd(la, s));
    }
    ++gj;
    const bool last = row0 + p.chunk >= N;
    if (gj == p.dw_group || last) {
      const int grows = int(row0 + rows - group_row0);
      // dH of the group in blocks of at most grp_pad rows
      for (int64_t b0 = 0; b0 < grows; b0 += p.grp_pad) {
        const int brows = int(grows - b0 < p.grp_pad ? grows - b0 : p.grp_pad);
        uint16_t* dHb = dH + (group_row0 + b0) * D;
        kd::DhArgs da{G + b0 * p.Vp, W,          brows,      int(D), int(V), p.Vp, p.grp_split, kps, dhp, dHb,
                      p.grp_pad,         zall != nullptr ? grad_loss : nullptr};
        KD_LAUNCH(KD_KERNEL_DH, s, kd::launch_dh(da, s));
        if (p.grp_split > 1)
          KD_LAUNCH(KD_KERNEL_DH_REDUCE, s,
                    kd::launch_dh_reduce(dhp, p.grp_split, brows, int(D), p.grp_pad, dHb, s));
      }
      // dW += G^T H over the group, in row blocks of at most gemm_rows (one
      // block unless G's rows outgrow 32-bit offsets); each block adds once
      for (int64_t b0 = 0; b0 < grows; b0 += p.gemm_rows) {
        const int brows = int(grows - b0 < p.gemm_rows ? grows - b0 : p.gemm_rows);
        kd::DwArgs wa{G + b0 * p.Vp, H + (group_row0 + b0) * D, brows, int(D), int(V), p.Vp, dW,
                      zall != nullptr ? grad_loss : nullptr};
        KD_LAUNCH(KD_KERNEL_DW, s, kd::launch_dw(wa, s));
      }
      gj = 0;
    }
  }
  return debug_done(s);
}

kd_status check_forward_ptrs(const uint16_t* H, const uint16_t* W, const int32_t* topk_idx,
                             const float* topk_logit, int64_t N, float* loss, float* lse, float* row_kl) {
  if (bad_ptr(loss, 4)) return KD_ERR_INVALID_ARG;
  if (N > 0 && (bad_ptr(H, 16) || bad_ptr(W, 16) || bad_ptr(topk_idx, 4) ||
                bad_ptr(topk_logit, 4) || bad_ptr(lse, 4)))
    return KD_ERR_INVALID_ARG;
  if (row_kl != nullptr && !kd::aligned(row_kl, 4)) return KD_ERR_INVALID_ARG;
  return KD_OK;
}

kd_status check_forward_args(const kd::Plan& p, const uint16_t* H, const uint16_t* W, const int32_t* topk_idx,
                             const float* topk_logit, int64_t N, float* loss, float* lse, float* row_kl,
                             void* workspace, size_t workspace_bytes, size_t need) {
  const kd_status st = check_forward_ptrs(H, W, topk_idx, topk_logit, N, loss, lse, row_kl);
  if (st != KD_OK) return st;
  if (N > 0 && (workspace == nullptr || workspace_bytes < need)) return KD_ERR_WORKSPACE;
  if (workspace != nullptr && !kd::aligned(workspace, 256)) return KD_ERR_INVALID_ARG;
  (void)p;
  return KD_OK;
}

}  // namespace

// ---- allocation-free forward: its scratch is a file-scope device array ----

// Size of the array; kd_topk_kl_forward_noalloc rejects problems whose
// forward workspace region is larger.  Each GPU the library runs on holds one
// copy until the process ends.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kNoallocScratchBytes];

namespace {

// Device address of `scratch` per device.  In host code the array's name is
// a host-side stand-in, not a device address, so kernels get this pointer.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Looks up the current device's copy of `scratch` on its first use there.
hipError_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr || !kd::aligned(ptr, 256)) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

kd_status kd_topk_kl_forward(const uint16_t* H, const uint16_t* W, const int32_t* topk_idx,
                             const float* topk_logit, int64_t N, int64_t D, int64_t V, int32_t K,
                             float T, int64_t chunk, float* loss, float* lse, float* row_kl,
                             void* workspace, size_t workspace_bytes, void* hip_stream) {
  // the extended loss at its neutral settings: no weights, no labels, kd_weight 1
  return kd_topk_kl_forward_ex(H, W, topk_idx, topk_logit, N, D, V, K, T, chunk, nullptr, nullptr, 1.f, 0.f, 0,
                               loss, lse, row_kl, workspace, workspace_bytes, hip_stream);
}

kd_status kd_topk_kl_forward_noalloc(const uint16_t* H, const uint16_t* W, const int32_t* topk_idx,
                                     const float* topk_logit, int64_t N, int64_t D, int64_t V, int32_t K,
                                     float T, int64_t chunk, float* loss, float* lse, float* row_kl,
                                     void* hip_stream) {
  kd::Plan p;
  kd_status st = kd::make_plan(N, D, V, K, T, chunk, &p);
  if (st != KD_OK) return st;
  st = check_forward_ptrs(H, W, topk_idx, topk_logit, N, loss, lse, row_kl);
  if (st != KD_OK) return st;
  if (p.fwd_bytes > kNoallocScratchBytes) return KD_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (N == 0) {
    KD_LAUNCH(KD_KERNEL_FINALIZE, s, kd::launch_fill_f32(loss, 1, 0.f, s));
    return KD_OK;
  }
  void* ws = nullptr;
  const hipError_t e = scratch_ptr(&ws);
  if (e != hipSuccess) return hip_failed(e);
  // nothing in the scratch has to start at zero: with ids in [0, V) every
  // forward buffer is written before it is read within the call (other ids
  // give unspecified results, as with a caller's workspace)
  return run_forward(p, H, W, topk_idx, topk_logit, N, D, V, K, T, loss, lse, row_kl, static_cast<char*>(ws),
                     nullptr, nullptr, s);
}

size_t kd_topk_kl_keep_workspace_size(int64_t N, int64_t D, int64_t V, int32_t K, int64_t chunk) {
  kd::KeepPlan kp;
  if (kd::make_keep_plan(N, D, V, K, 1.f, chunk, &kp) != KD_OK) return 0;
  return kp.bytes;
}

kd_status kd_topk_kl_forward_keep(const uint16_t* H, const uint16_t* W, const int32_t* topk_idx,
                                  const float* topk_logit, int64_t N, int64_t D, int64_t V, int32_t K,
                                  float T, int64_t chunk, float* loss, float* lse, float* row_kl,
                                  void* workspace, size_t workspace_bytes, void* hip_stream) {
  kd::KeepPlan kp;
  kd_status st = kd::make_keep_plan(N, D, V, K, T, chunk, &kp);
  if (st != KD_OK) return st;
  st = check_forward_args(kp.base, H, W, topk_idx, topk_logit, N, loss, lse, row_kl, workspace,
                          workspace_bytes, kp.bytes);
  if (st != KD_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (N == 0) {
    KD_LAUNCH(KD_KERNEL_FINALIZE, s, kd::launch_fill_f32(loss, 1, 0.f, s));
    return KD_OK;
  }
  char* ws = static_cast<char*>(workspace);
  return run_forward(kp.base, H, W, topk_idx, topk_logit, N, D, V, K, T, loss, lse, row_kl, ws,
                     reinterpret_cast<float*>(ws + kp.off_z), reinterpret_cast<uint16_t*>(ws + kp.off_gall), s);
}

kd_status kd_topk_kl_backward_keep(const uint16_t* H, const uint16_t* W, const float* grad_loss,
                                   int64_t N, int64_t D, int64_t V, int32_t K, float T, int64_t chunk,
                                   uint16_t* dH, float* dW, void* workspace, size_t workspace_bytes,
                                   void* hip_stream) {
  kd::KeepPlan kp;
  const kd_status st = kd::make_keep_plan(N, D, V, K, T, chunk, &kp);
  if (st != KD_OK) return st;
  const kd::Plan& p = kp.base;
  if (bad_ptr(dW, 16)) return KD_ERR_INVALID_ARG;
  if (N > 0 && (bad_ptr(H, 16) || bad_ptr(W, 16) || bad_ptr(dH, 16))) return KD_ERR_INVALID_ARG;
  if (grad_loss != nullptr && !kd::aligned(grad_loss, 4)) return KD_ERR_INVALID_ARG;
  if (N > 0 && (workspace == nullptr || workspace_bytes < kp.bytes)) return KD_ERR_WORKSPACE;
  if (workspace != nullptr && !kd::aligned(workspace, 256)) return KD_ERR_INVALID_ARG;
  if (N == 0) return KD_OK;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  char* ws = static_cast<char*>(workspace);
  const uint16_t* gall = reinterpret_cast<const uint16_t*>(ws + kp.off_gall);
  float* dhp = reinterpret_cast<float*>(ws + kp.off_dhp);
  const int ktiles = int(p.Vp / kd::gemm_bk());
  const int kps = (ktiles + p.dh_split - 1) / p.dh_split;
  // dH in blocks of one chunk (or fewer rows when a chunk of G outgrows 32-bit offsets)
  const int64_t hstep = p.chunk < p.gemm_rows ? p.chunk : p.gemm_rows;
  for (int64_t row0 = 0; row0 < N; row0 += hstep) {
    const int rows = int(N - row0 < hstep ? N - row0 : hstep);
    kd::DhArgs da{gall + row0 * p.Vp, W, rows, int(D), int(V), p.Vp, p.dh_split, kps, dhp, dH + row0 * D,
                  p.c_pad, grad_loss};
    KD_LAUNCH(KD_KERNEL_DH, s, kd::launch_dh(da, s));
    if (p.dh_split > 1)
      KD_LAUNCH(KD_KERNEL_DH_REDUCE, s,
                kd::launch_dh_reduce(dhp, p.dh_split, rows, int(D), p.c_pad, dH + row0 * D, s));
  }
  for (int64_t r0 = 0; r0 < N; r0 += kp.dw_rows) {
    const int rows = int(N - r0 < kp.dw_rows ? N - r0 : kp.dw_rows);
    kd::DwArgs wa{gall + r0 * p.Vp, H + r0 * D, rows, int(D), int(V), p.Vp, dW, grad_loss};
    KD_LAUNCH(KD_KERNEL_DW, s, kd::launch_dw(wa, s));
  }
  return KD_OK;
}

size_t kd_topk_kl_keep_logits_workspace_size(int64_t N, int64_t D, int64_t V, int32_t K, int64_t chunk) {
  kd::KeepLogitsPlan kp;
  if (kd::make_keep_logits_plan(N, D, V, K, 1.f, chunk, &kp) != KD_OK) return 0;
  return kp.bytes;
}

kd_status kd_topk_kl_forward_keep_logits(const uint16_t* H, const uint16_t* W, const int32_t* topk_idx,
                                         const float* topk_logit, int64_t N, int64_t D, int64_t V, int32_t K,
                                         float T, int64_t chunk, float* loss, float* lse, float* row_kl,
                                         void* workspace, size_t workspace_bytes, void* hip_stream) {
  kd::KeepLogitsPlan kp;
  kd_status st = kd::make_keep_logits_plan(N, D, V, K, T, chunk, &kp);
  if (st != KD_OK) return st;
  st = check_forward_args(kp.base, H, W, topk_idx, topk_logit, N, loss, lse, row_kl, workspace,
                          workspace_bytes, kp.bytes);
  if (st != KD_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (N == 0) {
    KD_LAUNCH(KD_KERNEL_FINALIZE, s, kd::launch_fill_f32(loss, 1, 0.f, s));
    return KD_OK;
  }
  char* ws = static_cast<char*>(workspace);
  return run_forward(kp.base, H, W, topk_idx, topk_logit, N, D, V, K, T, loss, lse, row_kl, ws, nullptr,
                     nullptr, s, LossExt(), reinterpret_cast<float*>(ws + kp.off_z));
}

kd_status kd_topk_kl_backward_keep_logits(const uint16_t* H, const uint16_t* W, const int32_t* topk_idx,
                                          const float* topk_logit, const float* lse, const float* grad_loss,
                                          int64_t N, int64_t D, int64_t V, int32_t K, float T, int64_t chunk,
                                          uint16_t* dH, float* dW, void* workspace, size_t workspace_bytes,
                                          void* hip_stream) {
  kd::KeepLogitsPlan kp;
  const kd_status st = kd::make_keep_logits_plan(N, D, V, K, T, chunk, &kp);
  if (st != KD_OK) return st;
  if (bad_ptr(dW, 16)) return KD_ERR_INVALID_ARG;
  if (N > 0 && (bad_ptr(H, 16) || bad_ptr(W, 16) || bad_ptr(topk_idx, 4) || bad_ptr(topk_logit, 4) ||
                bad_ptr(lse, 4) || bad_ptr(dH, 16)))
    return KD_ERR_INVALID_ARG;
  if (grad_loss != nullptr && !kd::aligned(grad_loss, 4)) return KD_ERR_INVALID_ARG;
  if (N > 0 && (workspace == nullptr || workspace_bytes < kp.bytes)) return KD_ERR_WORKSPACE;
  if (workspace != nullptr && !kd::aligned(workspace, 256)) return KD_ERR_INVALID_ARG;
  if (N == 0) return KD_OK;
  char* ws = static_cast<char*>(workspace);
  return run_backward(kp.base, H, W, topk_idx, topk_logit, nullptr, 0, lse, nullptr, grad_loss, N, D, V, K, T,
                      dH, dW, ws, static_cast<hipStream_t>(hip_stream), LossExt(),
                      reinterpret_cast<float*>(ws + kp.off_z));
}

kd_status kd_topk_kl_backward(const uint16_t* H, const uint16_t* W, const int32_t* topk_idx,
                              const float* topk_logit, const float* lse, const float* grad_loss,
                              int64_t N, int64_t D, int64_t V, int32_t K, float T, int64_t chunk,
                              uint16_t* dH, float* dW, void* workspace, size_t workspace_bytes,
                              void* hip_stream) {
  return kd_topk_kl_backward_ex(H, W, topk_idx, topk_logit, lse, grad_loss, N, D, V, K, T, chunk, nullptr,
                                nullptr, 1.f, 0.f, 0, dH, dW, workspace, workspace_bytes, hip_stream);
}

kd_status kd_topk_kl_forward_ex(const uint16_t* H, const uint16_t* W, const int32_t* topk_idx,
                                const float* topk_logit, int64_t N, int64_t D, int64_t V, int32_t K,
                                float T, int64_t chunk, const float* row_weight, const int32_t* labels,
                                float kd_weight, float ce_weight, int32_t flags, float* loss, float* lse,
                                float* row_loss, void* workspace, size_t workspace_bytes, void* hip_stream) {
  kd::Plan p;
  kd_status st = kd::make_plan(N, D, V, K, T, chunk, &p);
  if (st != KD_OK) return st;
  if ((flags & ~KD_SCALE_T2) != 0 || !std::isfinite(kd_weight) || !std::isfinite(ce_weight))
    return KD_ERR_INVALID_ARG;
  if (N > 0 && ((row_weight != nullptr && !kd::aligned(row_weight, 4)) ||
                (labels != nullptr && !kd::aligned(labels, 4))))
    return KD_ERR_INVALID_ARG;
  st = check_forward_args(p, H, W, topk_idx, topk_logit, N, loss, lse, row_loss, workspace, workspace_bytes,
                          p.bytes);
  if (st != KD_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (N == 0) {
    KD_LAUNCH(KD_KERNEL_FINALIZE, s, kd::launch_fill_f32(loss, 1, 0.f, s));
    return KD_OK;
  }
  LossExt ext;
  ext.row_w = row_weight;
  ext.labels = labels;
  ext.alpha = kd_weight;
  ext.beta = labels != nullptr ? ce_weight : 0.f;
  ext.scale = (flags & KD_SCALE_T2) ? T * T : 1.f;
  return run_forward(p, H, W, topk_idx, topk_logit, N, D, V, K, T, loss, lse, row_loss,
                     static_cast<char*>(workspace), nullptr, nullptr, s, ext);
}

kd_status kd_topk_kl_backward_ex(const uint16_t* H, const uint16_t* W, const int32_t* topk_idx,
                                 const float* topk_logit, const float* lse, const float* grad_loss,
                                 int64_t N, int64_t D, int64_t V, int32_t K, float T, int64_t chunk,
                                 const float* row_weight, const int32_t* labels, float kd_weight,
                                 float ce_weight, int32_t flags, uint16_t* dH, float* dW, void* workspace,
                                 size_t workspace_bytes, void* hip_stream) {
  kd::Plan p;
  const kd_status st = kd::make_plan(N, D, V, K, T, chunk, &p);
  if (st != KD_OK) return st;
  if ((flags & ~KD_SCALE_T2) != 0 || !std::isfinite(kd_weight) || !std::isfinite(ce_weight))
    return KD_ERR_INVALID_ARG;
  if (bad_ptr(dW, 16)) return KD_ERR_INVALID_ARG;
  if (N > 0 && (bad_ptr(H, 16) || bad_ptr(W, 16) || bad_ptr(topk_idx, 4) ||
                bad_ptr(topk_logit, 4) || bad_ptr(lse, 4) || bad_ptr(dH, 16) ||
                (row_weight != nullptr && !kd::aligned(row_weight, 4)) ||
                (labels != nullptr && !kd::aligned(labels, 4))))
    return KD_ERR_INVALID_ARG;
  if (grad_loss != nullptr && !kd::aligned(grad_loss, 4)) return KD_ERR_INVALID_ARG;
  if (N > 0 && (workspace == nullptr || workspace_bytes < p.bytes)) return KD_ERR_WORKSPACE;
  if (workspace != nullptr && !kd::aligned(workspace, 256)) return KD_ERR_INVALID_ARG;
  if (N == 0) return KD_OK;
  LossExt ext;
  ext.row_w = row_weight;
  ext.labels = labels;
  ext.alpha = kd_weight;
  ext.beta = labels != nullptr ? ce_weight : 0.f;
  ext.scale = (flags & KD_SCALE_T2) ? T * T : 1.f;
  return run_backward(p, H, W, topk_idx, topk_logit, nullptr, 0, lse, nullptr, grad_loss, N, D, V, K, T, dH,
                      dW, static_cast<char*>(workspace), static_cast<hipStream_t>(hip_stream), ext);
}

size_t kd_dense_kl_workspace_size(int64_t N, int64_t D, int64_t V, int64_t chunk) {
  kd::DensePlan dp;
  if (kd::make_dense_plan(N, D, V, 1.f, chunk, &dp) != KD_OK) return 0;
  return dp.bytes;
}

kd_status kd_dense_kl_forward(const uint16_t* H, const uint16_t* W, const void* teacher_logits,
                              int32_t t_dtype, int64_t N, int64_t D, int64_t V, float T, int64_t chunk,
                              float* loss, float* lse, float* lse_t, float* row_kl, void* workspace,
                              size_t workspace_bytes, void* hip_stream) {
  kd::DensePlan dp;
  kd_status st = kd::make_dense_plan(N, D, V, T, chunk, &dp);
  if (st != KD_OK) return st;
  if (t_dtype != KD_DTYPE_F32 && t_dtype != KD_DTYPE_BF16) return KD_ERR_INVALID_ARG;
  if (bad_ptr(loss, 4)) return KD_ERR_INVALID_ARG;
  if (N > 0 && (bad_ptr(H, 16) || bad_ptr(W, 16) || bad_ptr(lse, 4) || bad_ptr(lse_t, 4) ||
                bad_ptr(teacher_logits, t_dtype == KD_DTYPE_F32 ? 16 : 8)))
    return KD_ERR_INVALID_ARG;
  if (row_kl != nullptr && !kd::aligned(row_kl, 4)) return KD_ERR_INVALID_ARG;
  if (N > 0 && (workspace == nullptr || workspace_bytes < dp.bytes)) return KD_ERR_WORKSPACE;
  if (workspace != nullptr && !kd::aligned(workspace, 256)) return KD_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (N == 0) {
    KD_LAUNCH(KD_KERNEL_FINALIZE, s, kd::launch_fill_f32(loss, 1, 0.f, s));
    return KD_OK;
  }
  const kd::Plan& p = dp.base;
  char* ws = static_cast<char*>(workspace);
  float* pm = reinterpret_cast<float*>(ws + p.off_pm);
  float* ps = reinterpret_cast<float*>(ws + p.off_ps);
  float* tm = reinterpret_cast<float*>(ws + dp.off_tm);
  float* ts0 = reinterpret_cast<float*>(ws + dp.off_ts0);
  float* ts1 = reinterpret_cast<float*>(ws + dp.off_ts1);
  float* rowkl = row_kl != nullptr ? row_kl : reinterpret_cast<float*>(ws + p.off_rowkl);
  const size_t esz = t_dtype == KD_DTYPE_F32 ? 4 : 2;
  for (int64_t row0 = 0; row0 < N; row0 += p.chunk) {
    const int rows = int(N - row0 < p.chunk ? N - row0 : p.chunk);
    kd::LogitsArgs la{};
    la.W = W;
    la.Hc = H + row0 * D;
    la.rows = rows;
    la.D = int(D);
    la.V = int(V);
    la.K = 1;
    la.nvt = int(p.nvt);
    la.npt = (rows + kd::kTile - 1) / kd::kTile;
    la.c_pad = p.c_pad;
    la.Vp = p.Vp;
    la.invT = 1.f / T;
    la.tlog = static_cast<const char*>(teacher_logits) + row0 * V * esz;
    la.t_dtype = t_dtype;
    la.tm = tm;
    la.ts0 = ts0;
    la.ts1 = ts1;
    la.pm = pm;
    la.ps = ps;
    KD_LAUNCH(KD_KERNEL_LOGITS_FWD, s, kd::launch_logits_fwd(la, s));
    kd::DenseCombineArgs ca{pm, ps, tm, ts0, ts1, rows, int(p.nvt), p.c_pad, lse + row0, lse_t + row0,
                            rowkl + row0};
    KD_LAUNCH(KD_KERNEL_COMBINE, s, kd::launch_dense_combine(ca, s));
  }
  KD_LAUNCH(KD_KERNEL_FINALIZE, s, kd::launch_finalize(rowkl, nullptr, N, loss, nullptr, s));
  return KD_OK;
}

kd_status kd_dense_kl_backward(const uint16_t* H, const uint16_t* W, const void* teacher_logits,
                               int32_t t_dtype, const float* lse, const float* lse_t,
                               const float* grad_loss, int64_t N, int64_t D, int64_t V, float T,
                               int64_t chunk, uint16_t* dH, float* dW, void* workspace,
                               size_t workspace_bytes, void* hip_stream) {
  kd::DensePlan dp;
  const kd_status st = kd::make_dense_plan(N, D, V, T, chunk, &dp);
  if (st != KD_OK) return st;
  if (t_dtype != KD_DTYPE_F32 && t_dtype != KD_DTYPE_BF16) return KD_ERR_INVALID_ARG;
  if (bad_ptr(dW, 16)) return KD_ERR_INVALID_ARG;
  if (N > 0 && (bad_ptr(H, 16) || bad_ptr(W, 16) || bad_ptr(lse, 4) || bad_ptr(lse_t, 4) ||
                bad_ptr(dH, 16) || bad_ptr(teacher_logits, t_dtype == KD_DTYPE_F32 ? 16 : 8)))
    return KD_ERR_INVALID_ARG;
  if (grad_loss != nullptr && !kd::aligned(grad_loss, 4)) return KD_ERR_INVALID_ARG;
  if (N > 0 && (workspace == nullptr || workspace_bytes < dp.bytes)) return KD_ERR_WORKSPACE;
  if (workspace != nullptr && !kd::aligned(workspace, 256)) return KD_ERR_INVALID_ARG;
  if (N == 0) return KD_OK;
  return run_backward(dp.base, H, W, nullptr, nullptr, teacher_logits, t_dtype, lse, lse_t, grad_loss, N, D,
                      V, 1, T, dH, dW, static_cast<char*>(workspace), static_cast<hipStream_t>(hip_stream));
}

kd_status kd_topk_kl_validate(const int32_t* topk_idx, int64_t N, int32_t K, int64_t V,
                              int32_t* d_flags, void* hip_stream) {
  if (d_flags == nullptr || !kd::aligned(d_flags, 4)) return KD_ERR_INVALID_ARG;
  if (N < 0 || K <= 0 || V <= 0 || K > KD_MAX_K) return KD_ERR_INVALID_ARG;
  if (N > 0 && bad_ptr(topk_idx, 4)) return KD_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const hipError_t e = kd::launch_validate(topk_idx, N, K, V, d_flags, s);
  if (e != hipSuccess) return hip_failed(e);
  return KD_OK;
}

kd_status kd_topk_select(const void* logits, int32_t dtype, int64_t N, int64_t V, int32_t K,
                         int32_t* topk_idx, float* topk_logit, void* hip_stream) {
  if (dtype != KD_DTYPE_F32 && dtype != KD_DTYPE_BF16) return KD_ERR_INVALID_ARG;
  if (N < 0 || V <= 0 || K <= 0 || K > V) return KD_ERR_INVALID_ARG;
  if (K > KD_MAX_K || V > (int64_t(1) << 31) - 1 || N > (int64_t(1) << 31) - 1) return KD_ERR_UNSUPPORTED;
  const size_t esz = dtype == KD_DTYPE_F32 ? 4 : 2;
  if (N == 0) return KD_OK;
  if (bad_ptr(logits, esz) || bad_ptr(topk_idx, 4) || bad_ptr(topk_logit, 4)) return KD_ERR_INVALID_ARG;
  const bool vec = (V * int64_t(esz)) % 16 == 0 && kd::aligned(logits, 16);
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  KD_LAUNCH(KD_KERNEL_TOPK_SELECT, s,
            kd::launch_topk_select(logits, dtype, vec, N, V, K, topk_idx, topk_logit, s));
  return KD_OK;
}

kd_status kd_profile_enable(uint32_t kernel_mask) {
  if (kernel_mask >> KD_KERNEL_COUNT) return KD_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_mask = kernel_mask;
  return KD_OK;
}

kd_status kd_profile_read(int32_t kernel_id, double* total_ms, int64_t* launches) {
  if (kernel_id < 0 || kernel_id >= KD_KERNEL_COUNT || total_ms == nullptr || launches == nullptr)
    return KD_ERR_INVALID_ARG;
  std::vector<EventPair> evs;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    evs.swap(g_prof_events[kernel_id]);
  }
  double tot = 0.0;
  kd_status st = KD_OK;
  for (auto& e : evs) {
    float ms = 0.f;
    if (hipEventSynchronize(e.b) != hipSuccess || hipEventElapsedTime(&ms, e.a, e.b) != hipSuccess)
      st = KD_ERR_HIP;
    tot += ms;
    (void)hipEventDestroy(e.a);
    (void)hipEventDestroy(e.b);
  }
  *total_ms = tot;
  *launches = int64_t(evs.size());
  return st;
}

}  // extern "C"
