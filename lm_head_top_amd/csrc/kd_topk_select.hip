// gfx950 kernel of the teacher top-K cache writer: per row of full-vocabulary
// teacher logits, the K largest logits and their token ids, largest first,
// equal logits by lower id ("Distilling an LLM on One GPU", section "The two
// changes"; "The $250GB Memory Spike That Killed Distillation Projects Is Now
// Optional", section "Offline Top-K").
//
// One workgroup per row, one pass over the row in HBM.  Every logit becomes a
// 64-bit key (order-preserving bits of the logit, then the complement of the
// id), so "larger key" is exactly "larger logit, or equal logit and lower id"
// and all keys of a row are distinct.  Keys above the running threshold (the
// K-th best key kept so far) are appended to an LDS candidate list; when the
// list holds TRIG keys (and at least K) it is sorted (bitonic, in LDS), cut to
// the K best and the threshold raised.  For random logits a row of 131072 admits a
// few thousand candidates, so the row is read once and sorted about three
// times.  The next batch of the row is loaded into registers while the
// current one is filtered.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kd_kernels.h"

namespace kd {
namespace {

#ifndef KD_TOPK_THREADS
#define KD_TOPK_THREADS 256
#endif
#ifndef KD_TOPK_BATCH
#define KD_TOPK_BATCH 2048
#endif
#ifndef KD_TOPK_TRIG
#define KD_TOPK_TRIG 512
#endif
constexpr int TS = KD_TOPK_THREADS;      // threads per row
constexpr int PER_IT = KD_TOPK_BATCH;    // logits per batch
constexpr int CAP = 2 * PER_IT;          // candidate keys in LDS (32 KiB at 2048: 4 rows per CU)
// The list is compacted (and the threshold raised) once it holds TRIG keys,
// so the threshold follows the running K-th best closely; at most CAP - PER_IT.
constexpr int TRIG = KD_TOPK_TRIG < CAP - PER_IT ? KD_TOPK_TRIG : CAP - PER_IT;
static_assert(CAP >= 2 * PER_IT && CAP - PER_IT >= 256, "a batch must fit beside a full list");
static_assert(PER_IT % (TS * 8) == 0, "a batch is whole 16-byte loads of bf16 for every thread");

// Order-preserving 32-bit image of a float with -0.0 taken as +0.0.
__device__ __forceinline__ uint32_t sortable(float x) {
  const uint32_t b = __float_as_uint(x == 0.f ? 0.f : x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float unsortable(uint32_t s) {
  return __uint_as_float((s & 0x80000000u) ? (s & 0x7fffffffu) : ~s);
}

__device__ __forceinline__ uint64_t make_key(float x, uint32_t id) {
  return (uint64_t(sortable(x)) << 32) | uint64_t(~id);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Smallest float that can still carry a key above thr: every key above thr
// has sortable(x) >= its high word, i.e. x >= this value (-0.0 and +0.0 alike).
// Below sortable(-inf) lie only NaN patterns; then every non-NaN float passes.
__device__ __forceinline__ float key_floor(uint64_t thr) {
  const uint32_t hi = uint32_t(thr >> 32);
  return hi <= sortable(-INFINITY) ? -INFINITY : unsortable(hi);
}

// Appends the keys above thr (one wave-aggregated LDS atomic per wave).
__device__ __forceinline__ void append(uint64_t key, bool valid, uint64_t thr, uint64_t* cand, int* cnt,
                                       int lane) {
  const bool take = valid && key > thr;
  const uint64_t m = __ballot(take);
  if (m == 0) return;
  int base = 0;
  if (lane == 0) base = atomicAdd(cnt, __popcll(m));
  base = __shfl(base, 0);
  if (take) cand[base + __popcll(m & ((uint64_t(1) << lane) - 1))] = key;
}

// Sorts cand[0, n) descending (pads to a power of two with key 0, which is
// below every real key), leaves the K best at the front and returns the new
// list length min(n, K).  All threads call it.  Each bitonic stage first loads
// every pair a thread owns, then compares and stores, so a stage costs one LDS
// round trip rather than one per pair (the pairs of a stage are disjoint).
__device__ int compact(uint64_t* cand, int n, int K) {
  int P = 2;
  while (P < n) P <<= 1;
  for (int i = n + threadIdx.x; i < P; i += TS) cand[i] = 0;
  __syncthreads();
  constexpr int MAXU = CAP / 2 / TS;  // pairs per thread at P = CAP
  const int npairs = P >> 1;
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int lj = __builtin_ctz(j);
      uint64_t a[MAXU], b[MAXU];
      int ia[MAXU];
#pragma unroll
      for (int u = 0; u < MAXU; ++u) {
        const int p = threadIdx.x + u * TS;
        // pair p: i has bit lj clear, its partner sets it
        const int i = ((p >> lj) << (lj + 1)) | (p & (j - 1));
        ia[u] = i;
        if (p < npairs) {
          a[u] = cand[i];
          b[u] = cand[i | j];
        }
      }
#pragma unroll
      for (int u = 0; u < MAXU; ++u) {
        const int p = threadIdx.x + u * TS;
        if (p < npairs) {
          const int i = ia[u];
          const bool desc = (i & k) == 0;
          if (desc ? (a[u] < b[u]) : (a[u] > b[u])) {
            cand[i] = b[u];
            cand[i | j] = a[u];
          }
        }
      }
      __syncthreads();
    }
  }
  return n < K ? n : K;
}

// DT 0: fp32 logits, DT 1: bf16 logits.  VEC: 16-byte loads (the row length is
// a multiple of 16 bytes and the base 16-byte aligned), else 2- or 4-byte loads.
template <int DT, bool VEC>
__global__ __launch_bounds__(TS) void topk_select_kernel(const void* __restrict__ logits, int64_t V, int K,
                                                         int32_t* __restrict__ out_idx,
                                                         float* __restrict__ out_val) {
  __shared__ uint64_t cand[CAP];
  __shared__ int cnt;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  constexpr int ESZ = DT == 0 ? 4 : 2;
  constexpr int EPL = 16 / ESZ;                   // elements per 16-byte load
  constexpr int NL = VEC ? PER_IT / (TS * EPL) : PER_IT / TS;  // loads per thread per batch
  const char* base = static_cast<const char*>(logits) + row * V * ESZ;
  if (tid == 0) cnt = 0;
  uint64_t thr = 0;
  int n = 0;  // list length, the same in every thread after each barrier

  // One batch: NL loads of 16 bytes (VEC) or of one element per thread.
  using Reg = typename std::conditional<VEC, uint4, uint32_t>::type;
  auto load = [&](int64_t e0, Reg (&r)[NL]) {
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      if constexpr (VEC) {
        const int64_t e = e0 + int64_t(u * TS + tid) * EPL;
        r[u] = e < V ? *reinterpret_cast<const uint4*>(base + e * ESZ) : make_uint4(0, 0, 0, 0);
      } else {
        const int64_t e = e0 + u * TS + tid;
        r[u] = e >= V ? 0u
                      : (DT == 0 ? reinterpret_cast<const uint32_t*>(base)[e]
                                 : uint32_t(reinterpret_cast<const uint16_t*>(base)[e]));
      }
    }
  };
  // Most logits cannot beat the threshold: each is first compared as a float
  // against key_floor(thr) (a superset of the exact test), one ballot drops a
  // batch for the whole wave, and the 64-bit key, the exact test and the
  // append run only for slots where some lane passes.
  float thr_f = -INFINITY;
  auto filter = [&](int64_t e0, const Reg (&r)[NL]) {
    bool any = false;
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      if constexpr (VEC) {
        const int64_t e = e0 + int64_t(u * TS + tid) * EPL;  // the row holds whole 16-byte chunks
        const uint32_t w[4] = {r[u].x, r[u].y, r[u].z, r[u].w};
#pragma unroll
        for (int q = 0; q < EPL; ++q) {
          const float x = DT == 0 ? __uint_as_float(w[q]) : bf16_to_f32((w[q / 2] >> (16 * (q & 1))) & 0xffffu);
          any |= e < V && x >= thr_f;
        }
      } else {
        const int64_t e = e0 + u * TS + tid;
        const float x = DT == 0 ? __uint_as_float(r[u]) : bf16_to_f32(r[u]);
        any |= e < V && x >= thr_f;
      }
    }
    if (__ballot(any) == 0) return;
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      if constexpr (VEC) {
        const int64_t e = e0 + int64_t(u * TS + tid) * EPL;
        const uint32_t w[4] = {r[u].x, r[u].y, r[u].z, r[u].w};
#pragma unroll
        for (int q = 0; q < EPL; ++q) {
          const float x = DT == 0 ? __uint_as_float(w[q]) : bf16_to_f32((w[q / 2] >> (16 * (q & 1))) & 0xffffu);
          const bool pass = e < V && x >= thr_f;
          if (__ballot(pass) == 0) continue;
          append(make_key(x, uint32_t(e + q)), pass, thr, cand, &cnt, lane);
        }
      } else {
        const int64_t e = e0 + u * TS + tid;
        const float x = DT == 0 ? __uint_as_float(r[u]) : bf16_to_f32(r[u]);
        const bool pass = e < V && x >= thr_f;
        if (__ballot(pass) == 0) continue;
        append(make_key(x, uint32_t(e)), pass, thr, cand, &cnt, lane);
      }
    }
  };

  __syncthreads();
  Reg nxt[NL], cur[NL];
  load(0, nxt);
  for (int64_t e0 = 0; e0 < V; e0 += PER_IT) {
#pragma unroll
    for (int u = 0; u < NL; ++u) cur[u] = nxt[u];
    if (e0 + PER_IT < V) load(e0 + PER_IT, nxt);  // the next batch is in flight during the filter
    filter(e0, cur);
    __syncthreads();
    n = cnt;
    __syncthreads();  // every thread has the same n before any thread appends again
    if (n >= TRIG && n >= K) {
      n = compact(cand, n, K);
      thr = cand[K - 1];  // n >= K keys were admitted, so n == K now
      thr_f = key_floor(thr);
      if (tid == 0) cnt = n;
      __syncthreads();
    }
  }
  n = compact(cand, n, K);
  for (int i = tid; i < n; i += TS) {
    const uint64_t key = cand[i];
    out_idx[row * K + i] = int32_t(~uint32_t(key));
    out_val[row * K + i] = unsortable(uint32_t(key >> 32));
  }
}

}  // namespace

hipError_t launch_topk_select(const void* logits, int dtype, bool vec, int64_t N, int64_t V, int K,
                              int32_t* idx, float* val, hipStream_t s) {
  const dim3 grid{unsigned(N), 1, 1}, block{unsigned(TS), 1, 1};
  if (dtype == 0) {
    if (vec)
      hipLaunchKernelGGL((topk_select_kernel<0, true>), grid, block, 0, s, logits, V, K, idx, val);
    else
      hipLaunchKernelGGL((topk_select_kernel<0, false>), grid, block, 0, s, logits, V, K, idx, val);
  } else {
    if (vec)
      hipLaunchKernelGGL((topk_select_kernel<1, true>), grid, block, 0, s, logits, V, K, idx, val);
    else
      hipLaunchKernelGGL((topk_select_kernel<1, false>), grid, block, 0, s, logits, V, K, idx, val);
  }
  return hipGetLastError();
}

}  // namespace kd
