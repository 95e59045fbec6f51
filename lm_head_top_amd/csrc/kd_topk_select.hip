// gfx950 kernel of the teacher top-K cache writer: per row of full-vocabulary
// teacher logits, the K largest logits and their token ids, largest first,
// equal logits by lower id ("Distilling an LLM on One GPU", section "The two
// changes"; "The $250GB Memory Spike That Killed Distillation Projects Is Now
// Optional", section "Offline Top-K").
//
// One wave per row, one pass over the row in HBM, no workgroup barriers.
// Every logit becomes a 64-bit key (order-preserving bits of the logit, then
// the complement of the id), so "larger key" is exactly "larger logit, or
// equal logit and lower id" and all keys of a row are distinct.  The row
// streams in batches of 1024 logits through a buffer descriptor (16-byte
// loads, 1 KiB per load instruction, zeros past the row), two batches in
// flight while a third is filtered.  Each load's values are first tested as
// floats: their max against the float floor of the threshold (the K-th best
// key kept so far), one wave-wide test per load.  Only when some lane passes
// are the 64-bit keys formed and those above the threshold appended to the
// wave's candidate list in LDS.  After every EI logits, a list of TRIG keys
// or more is cut to the K best: a 64-step bitwise search finds the K-th
// largest key (counting with ballots), the keys at or above it are packed to
// the front, and it becomes the threshold.  At the end the K survivors are
// sorted in registers (bitonic, across the wave's lanes).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kd_kernels.h"

namespace kd {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// logits that enter the candidate list between cut checks (at least one
// load's worth): larger leaves more room below the cut trigger, so fewer
// cuts per row
#ifndef KD_TOPK_EI
#define KD_TOPK_EI 512
#endif

constexpr int TW = 4;            // rows (waves) per workgroup
constexpr int EB = 1024;         // logits per batch per wave
constexpr int CAPW = 1280;       // candidate keys per wave in LDS (4 waves: 40 KiB per workgroup)
constexpr int KPL = CAPW / 64;   // list keys per lane when the list is cut
static_assert(KD_MAX_K <= 256, "the final sort holds 4 keys per lane");

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

__device__ __forceinline__ uint64_t lanes_below(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Orders this wave's LDS accesses for the compiler: LDS serves one wave's
// instructions in issue order, so the wave sees its own earlier writes.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Cuts the wave's list cand[0, n) (n > K) to its K largest keys, packed at
// the front; returns the K-th largest key T, found bit by bit from the top
// as the largest value with at least K keys at or above it (each step counts
// with one ballot per 64-key slot; branch-free over all slots, which measured
// faster than limiting the scan to the slots in use or searching the value
// and id words separately).
__device__ uint64_t cut_list(uint64_t* cand, int n, int K, int lane) {
  uint64_t key[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int i = j * 64 + lane;
    key[j] = i < n ? cand[i] : 0ull;  // key 0 lies below every real key
  }
  // keys are distinct, so that largest value is itself a key
  uint64_t T = 0;
  for (int bit = 63; bit >= 0; --bit) {
    const uint64_t c = T | (1ull << bit);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) cnt += __popcll(__ballot(key[j] >= c));
    if (cnt >= K) T = c;
  }
  wave_lds_fence();
  int pos = 0;
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const bool keep = key[j] >= T && key[j] != 0ull;
    const uint64_t m = __ballot(keep);
    if (keep) cand[pos + __popcll(m & lanes_below(lane))] = key[j];
    pos += __popcll(m);
  }
  wave_lds_fence();
  return T;
}

// Compare-exchange of bitonic stage (k, j) for the 4 keys of this lane
// (element i = 4 lane + r): the pair (i, i ^ j), larger first where i & k is 0.
__device__ __forceinline__ void bitonic_step(uint64_t (&v)[4], int lane, int k, int j) {
  if (j >= 4) {
    const int lj = j >> 2;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t lo = __shfl_xor(uint32_t(v[r]), lj);
      const uint32_t hi = __shfl_xor(uint32_t(v[r] >> 32), lj);
      const uint64_t o = (uint64_t(hi) << 32) | lo;
      const int i = 4 * lane + r;
      const bool lower = (i & j) == 0;  // the lower element of its pair
      const bool desc = (i & k) == 0;
      const bool keep_max = lower == desc;
      v[r] = keep_max ? (v[r] > o ? v[r] : o) : (v[r] < o ? v[r] : o);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if ((r & j) != 0) continue;
      const int i = 4 * lane + r;
      const bool desc = (i & k) == 0;
      const uint64_t a = v[r], b = v[r | j];
      const bool swap = desc ? (a < b) : (a > b);
      v[r] = swap ? b : a;
      v[r | j] = swap ? a : b;
    }
  }
}

// DT 0: fp32 logits, DT 1: bf16 logits.  VEC: 16-byte loads (the row length is
// a multiple of 16 bytes and the base 16-byte aligned), else 2- or 4-byte loads.
template <int DT, bool VEC>
__global__ __launch_bounds__(TW * 64) __attribute__((amdgpu_waves_per_eu(4, 8)))
void topk_select_kernel(const void* __restrict__ logits, int64_t N, int64_t V, int K,
                        int32_t* __restrict__ out_idx, float* __restrict__ out_val) {
  __shared__ uint64_t cand_all[TW * CAPW];
  // the wave index is uniform: say so, so the row's buffer descriptor sits in
  // scalar registers
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = int64_t(blockIdx.x) * TW + wave;
  if (row >= N) return;  // the whole wave; nothing below synchronises the workgroup
  uint64_t* cand = cand_all + wave * CAPW;
  constexpr int ESZ = DT == 0 ? 4 : 2;
  constexpr int EPL = VEC ? 16 / ESZ : 1;  // logits per load
  constexpr int U = EB / (64 * EPL);  // loads per lane per batch
  // logits that enter the list between cut checks (whole loads), and the
  // list length that triggers a cut: a list below TRIG takes EI more keys
  constexpr int EI = KD_TOPK_EI > 64 * EPL ? KD_TOPK_EI : 64 * EPL;
  constexpr int UH = EI / (64 * EPL);
  constexpr int TRIG = CAPW - EI;
  static_assert(U % UH == 0 && TRIG >= KD_MAX_K, "cut checks at whole loads; a cut list fits below TRIG");
  using Reg = typename std::conditional<VEC, u32x4, uint32_t>::type;
  const char* base = static_cast<const char*>(logits) + row * V * ESZ;
  // VEC rows (under 2^31 bytes) load through a buffer descriptor: a load past
  // the row returns zeros with no branch, so every batch issues the same
  // loads and the loop keeps its two batches in flight
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, VEC ? int(V * ESZ) : 0, 0x00020000);

  // logit index of load u, element q of this lane in the batch at e0
  // indices within the row in 32 bits: V < 2^31, and e0 stays below V + 6 EB
  const uint32_t Vu = uint32_t(V);
  auto elem_index = [&](uint32_t e0, int u, int q) -> uint32_t { return e0 + uint32_t((u * 64 + lane) * EPL + q); };
  auto load = [&](uint32_t e0, Reg (&r)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t e = elem_index(e0, u, 0);
      if constexpr (VEC) {
        const uint32_t off = e < Vu ? e * uint32_t(ESZ) : 0xFFFFFFF0u;
        r[u] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, int(off), 0, 0);
      } else {
        r[u] = e >= Vu ? 0u
                      : (DT == 0 ? reinterpret_cast<const uint32_t*>(base)[e]
                                 : uint32_t(reinterpret_cast<const uint16_t*>(base)[e]));
      }
    }
  };
  auto value = [&](const Reg (&r)[U], int u, int q) -> float {
    if constexpr (VEC) {
      const uint32_t w[4] = {r[u].x, r[u].y, r[u].z, r[u].w};
      return DT == 0 ? __uint_as_float(w[q]) : bf16_to_f32((w[q / 2] >> (16 * (q & 1))) & 0xffffu);
    } else {
      return DT == 0 ? __uint_as_float(r[u]) : bf16_to_f32(r[u]);
    }
  };

  uint64_t thr = 0;  // keys above thr may enter the list
  float thr_f = -INFINITY;
  int n = 0;  // keys in the list (the same in every lane)
  auto filter = [&](uint32_t e0, const Reg (&r)[U]) {
    if (e0 >= Vu) return;
    // the max of one load's values (past the row: -inf)
    auto load_max = [&](int u) -> float {
      float mx = -INFINITY;
      if (e0 + EB <= Vu) {  // a whole batch (uniform): no per-logit bounds test
#pragma unroll
        for (int q = 0; q < EPL; ++q) mx = fmaxf(mx, value(r, u, q));
      } else {
#pragma unroll
        for (int q = 0; q < EPL; ++q) mx = elem_index(e0, u, q) < Vu ? fmaxf(mx, value(r, u, q)) : mx;
      }
      return mx;
    };
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // a load none of whose values can enter is skipped whole: one
      // wave-wide test per load
      if (__ballot(load_max(u) >= thr_f) != 0) {
        wave_lds_fence();
#pragma unroll
        for (int q = 0; q < EPL; ++q) {
          const float x = value(r, u, q);
          const uint32_t e = elem_index(e0, u, q);
          const bool pass = e < Vu && x >= thr_f;
          if (__ballot(pass) == 0) continue;
          const uint64_t key = make_key(x, e);
          const bool take = pass && key > thr;
          const uint64_t mk = __ballot(take);
          if (take) cand[n + __popcll(mk & lanes_below(lane))] = key;
          n += __popcll(mk);
        }
      }
      if ((u + 1) % UH == 0) {
        // EI logits have entered (n < TRIG before them): cut before the next
        // EI could overflow the list
        wave_lds_fence();
        if (n >= TRIG && n > K) {
          thr = cut_list(cand, n, K, lane);
          thr_f = key_floor(thr);
          n = K;
        }
      }
    }
  };

  // three register sets: two batches in flight while the third is filtered
  // (a fourth set measured no faster)
  // The loads go out in the order ra, rb, rc before the loop and in the loop
  // alike (scheduling barriers keep the compiler from reordering them), so
  // at the loop head ra's loads are the oldest in both cases and the wait
  // for them leaves rb's and rc's in flight.
  Reg ra[U], rb[U], rc[U];
  auto load_in_order = [&](uint32_t e, Reg (&r)[U]) {
    __builtin_amdgcn_sched_barrier(0);
    load(e, r);
    __builtin_amdgcn_sched_barrier(0);
  };
  load_in_order(0, ra);
  load_in_order(EB, rb);
  load_in_order(2 * EB, rc);
  for (uint32_t e0 = 0; e0 < Vu; e0 += 3 * EB) {
    filter(e0, ra);
    load_in_order(e0 + 3 * EB, ra);
    filter(e0 + EB, rb);
    load_in_order(e0 + 4 * EB, rb);
    filter(e0 + 2 * EB, rc);
    load_in_order(e0 + 5 * EB, rc);
  }
  if (n > K) {
    cut_list(cand, n, K, lane);
    n = K;
  }
  // sort the n <= K <= 256 survivors (padded with key 0) largest first
  uint64_t v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 4 * lane + r;
    v[r] = i < n ? cand[i] : 0ull;
  }
  for (int k = 2; k <= 256; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) bitonic_step(v, lane, k, j);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 4 * lane + r;
    if (i < n) {
      out_idx[row * K + i] = int32_t(~uint32_t(v[r]));
      out_val[row * K + i] = unsortable(uint32_t(v[r] >> 32));
    }
  }
}

}  // namespace

hipError_t launch_topk_select(const void* logits, int dtype, bool vec, int64_t N, int64_t V, int K,
                              int32_t* idx, float* val, hipStream_t s) {
  const dim3 grid{unsigned((N + TW - 1) / TW), 1, 1}, block{unsigned(TW * 64), 1, 1};
  // the 16-byte path addresses a row with 32-bit buffer offsets
  if (V * (dtype == 0 ? 4 : 2) > int64_t(0x7FFFFFF0)) vec = false;
  if (dtype == 0) {
    if (vec)
      hipLaunchKernelGGL((topk_select_kernel<0, true>), grid, block, 0, s, logits, N, V, K, idx, val);
    else
      hipLaunchKernelGGL((topk_select_kernel<0, false>), grid, block, 0, s, logits, N, V, K, idx, val);
  } else {
    if (vec)
      hipLaunchKernelGGL((topk_select_kernel<1, true>), grid, block, 0, s, logits, N, V, K, idx, val);
    else
      hipLaunchKernelGGL((topk_select_kernel<1, false>), grid, block, 0, s, logits, N, V, K, idx, val);
  }
  return hipGetLastError();
}

}  // namespace kd
