// gfx950 kernels of the fused chunked top-K KL distillation loss.
//
// The method (developersdigest.tech blog, section "The two changes";
// andresseo.expert article, section "Fused Chunked KL"): one chunk of positions
// at a time, project the hidden states to logits, fold them into the running
// loss and drop them; the backward recomputes each chunk's logits.  Here every
// chunk runs as
//
//   prep      teacher probabilities p = softmax_K(t/T), h = sum p log p, and the
//             chunk's (row, id, k) cache entries bucketed by (position tile,
//             vocab tile) so that each logits tile finds its own entries;
//   logits    z^T = W H_c^T / T for one 256 x 256 (vocab, position) tile on bf16
//             MFMA (v_mfma_f32_32x32x16_bf16) with LDS-staged operands, then
//             forward: per-position tile max / sum-exp and the logits at the
//                      cached ids (never the tile itself) go to small buffers;
//             backward: G = g/(N T) (exp(z - lse) - p scattered at the ids),
//                      rounded to bf16 into the chunk's G_c[c, V];
//   combine   forward: merge the vocab-tile partials into lse and KL per row;
//   dh / dw   dH_c = G_c W (split over V, fp32 partials) and dW += G_c^T H_c.
//
// All four GEMMs share one MFMA main loop: 256 threads (2 x 2 waves of 64),
// a 256 x 256 output tile with a 128 x 128 tile per wave held as 4 x 4 MFMA
// 32x32 accumulators, K steps of 64 through double-buffered LDS.  Operands
// whose K axis is contiguous in memory are copied to LDS as 16-byte vectors;
// operands whose M/N axis is contiguous are transposed 8 x 8 in registers on
// the way in, so the LDS layout (K contiguous, 144-byte rows) and the MFMA
// reads are the same for both.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kd_kernels.h"

namespace kd {
namespace {

constexpr int NT = 256;                       // threads per workgroup
constexpr int BK = 64;                        // K step
constexpr int LDK = BK + 8;                   // LDS row stride (bf16): 144 B, conflict-free 16 B reads
constexpr int OPER = kTile * LDK;             // bf16 elements per operand per stage
constexpr int SMEM_ELEMS = 4 * OPER;          // 2 stages x 2 operands
constexpr int SLD = kTile + 4;                // fp32 row stride of the epilogue staging tile
constexpr int STAGE_FLOATS = 128 * SLD;       // half a tile: 128 positions x 256 vocab
constexpr float LOG2E = 1.4426950408889634f;

static_assert((STAGE_FLOATS + 4 * kTile) * 4 <= SMEM_ELEMS * 2, "epilogue staging must fit in LDS");

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// (m, s) <- merge of two (max, sum exp(x - max)) pairs.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) {
    m = M;
    s = 0.f;
    return;
  }
  s = s * exp2_fast((m - M) * LOG2E) + s2 * exp2_fast((m2 - M) * LOG2E);
  m = M;
}

// Workgroups are dealt to the 8 XCDs round-robin; give each XCD a contiguous
// range of logical tiles so tiles that share operands share an L2.
__device__ __forceinline__ int xcd_remap(int b, int total) {
  const int nx = 8;
  const int x = b % nx, i = b / nx;
  const int per = total / nx, rem = total % nx;
  return x * per + (x < rem ? x : rem) + i;
}

// ---------------------------------------------------------------- loaders ---

// Operand stored K-contiguous: X[mn][k] with leading dimension ld.  A 256 x 64
// tile is 2048 16-byte vectors, 8 per thread.  Requires k_lim % 8 == 0.
struct LoadKC {
  uint4 r[8];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ X, int64_t ld, int mn0,
                                       int mn_lim, int k0, int k_lim) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int v = i * NT + t;
      const int row = v >> 3, kk = (v & 7) * 8;
      const int mn = mn0 + row, k = k0 + kk;
      if (mn < mn_lim && k < k_lim)
        r[i] = *reinterpret_cast<const uint4*>(X + int64_t(mn) * ld + k);
      else
        r[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __device__ __forceinline__ void store(uint16_t* s) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int v = i * NT + t;
      const int row = v >> 3, kk = (v & 7) * 8;
      *reinterpret_cast<uint4*>(s + row * LDK + kk) = r[i];
    }
  }
};

// Operand stored M/N-contiguous: X[k][mn] with leading dimension ld.  Thread t
// owns the 8 x 8 block (k = kb*8.., mn = mb*8..) with kb = t % 8, mb = t / 8,
// loads it as 8 row vectors and writes it transposed (8 K-contiguous vectors).
// Requires mn_lim % 8 == 0.
struct LoadMC {
  uint4 r[8];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ X, int64_t ld, int mn0,
                                       int mn_lim, int k0, int k_lim) {
    const int t = threadIdx.x;
    const int kb = t & 7, mb = t >> 3;
    const int mn = mn0 + mb * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = k0 + kb * 8 + j;
      if (mn < mn_lim && k < k_lim)
        r[j] = *reinterpret_cast<const uint4*>(X + int64_t(k) * ld + mn);
      else
        r[j] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __device__ __forceinline__ void store(uint16_t* s) const {
    const int t = threadIdx.x;
    const int kb = t & 7, mb = t >> 3;
    const uint32_t* w = reinterpret_cast<const uint32_t*>(r);  // w[j*4 + q]: row j, elements 2q, 2q+1
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int q = c >> 1;
      uint32_t o[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t x = w[(2 * d) * 4 + q], y = w[(2 * d + 1) * 4 + q];
        o[d] = (c & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
      }
      *reinterpret_cast<uint4*>(s + (mb * 8 + c) * LDK + kb * 8) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
};

// ------------------------------------------------------------- main loop ---

// One 64-deep K step of the wave's 128 x 128 tile from LDS.
// MFMA 32x32x16 operand layout: lane l supplies row (l % 32) and the 8
// consecutive k values 8 * (l / 32) .. +7 of A, and the same for B's column.
__device__ __forceinline__ void mma_step(const uint16_t* __restrict__ sA,
                                         const uint16_t* __restrict__ sB, f32x16 (&acc)[4][4],
                                         int wm, int wn, int lane) {
#pragma unroll
  for (int kk = 0; kk < BK; kk += 16) {
    bf16x8 a[4], b[4];
    const int koff = kk + (lane >> 5) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const bf16x8*>(sA + (wm * 128 + i * 32 + (lane & 31)) * LDK + koff);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = *reinterpret_cast<const bf16x8*>(sB + (wn * 128 + j * 32 + (lane & 31)) * LDK + koff);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// acc[i][j] (wave (wm, wn)) register r holds C[m][n] with
//   m = wm*128 + i*32 + 8*(r/4) + 4*(lane/32) + r%4,   n = wn*128 + j*32 + lane%32.
template <class LA, class LB>
__device__ __forceinline__ void gemm_mainloop(const uint16_t* __restrict__ A, int64_t lda, int a_mn0,
                                              int a_mn_lim, int a_k_lim,
                                              const uint16_t* __restrict__ B, int64_t ldb, int b_mn0,
                                              int b_mn_lim, int b_k_lim, int k_begin, int k_end,
                                              f32x16 (&acc)[4][4], uint16_t* smem) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int nk = (k_end - k_begin + BK - 1) / BK;
  if (nk <= 0) return;
  const int ak = a_k_lim < k_end ? a_k_lim : k_end;
  const int bk = b_k_lim < k_end ? b_k_lim : k_end;
  LA la;
  LB lb;
  la.load(A, lda, a_mn0, a_mn_lim, k_begin, ak);
  lb.load(B, ldb, b_mn0, b_mn_lim, k_begin, bk);
  la.store(smem);
  lb.store(smem + OPER);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const uint16_t* sA = smem + cur * 2 * OPER;
    const uint16_t* sB = sA + OPER;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k0 = k_begin + (kt + 1) * BK;
      la.load(A, lda, a_mn0, a_mn_lim, k0, ak);
      lb.load(B, ldb, b_mn0, b_mn_lim, k0, bk);
    }
    mma_step(sA, sB, acc, wm, wn, lane);
    if (more) {
      uint16_t* nA = smem + (cur ^ 1) * 2 * OPER;
      la.store(nA);
      lb.store(nA + OPER);
    }
    __syncthreads();
  }
}

// Row (within the 256-row tile) of accumulator register r of block i.
__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane) {
  return wm * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Writes the waves (wm, wn == half) of the tile to the staging area
// S[position - half*128][vocab] (fp32, row stride SLD).
__device__ __forceinline__ void stage_half(float* S, const f32x16 (&acc)[4][4], int wm, int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int pl = j * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int vl = wm * 128 + i * 32 + 8 * g + 4 * (lane >> 5);
        *reinterpret_cast<float4*>(S + pl * SLD + vl) =
            make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
      }
  }
}

// ---------------------------------------------------------------- kernels ---

__global__ __launch_bounds__(NT) void prep_kernel(PrepArgs a) {
  __shared__ int cnt[kMaxVocabTiles];
  __shared__ int part[NT];
  const int pt = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = pt * kTile;
  const int nr = min(kTile, a.rows - r0);
  const int K = a.K;

  // teacher distribution renormalised over the K cached logits at temperature T
  for (int rr = wave; rr < nr; rr += NT / 64) {
    const int64_t row = r0 + rr;
    float av[4];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = lane + 64 * u;
      av[u] = k < K ? a.t[row * K + k] * a.invT : -INFINITY;
      mx = fmaxf(mx, av[u]);
    }
    mx = wave_max(mx);
    float e[4], se = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      e[u] = mx == -INFINITY ? 0.f : exp2_fast((av[u] - mx) * LOG2E);
      se += e[u];
    }
    se = wave_sum(se);
    const float lnorm = mx + logf(se);
    float hs = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = lane + 64 * u;
      if (k < K) {
        const float pk = se > 0.f ? e[u] / se : 0.f;
        a.p[row * K + k] = pk;
        if (pk > 0.f) hs += pk * (av[u] - lnorm);
      }
    }
    hs = wave_sum(hs);
    if (lane == 0) a.h[row] = hs;
  }

  // bucket the tile's entries by vocab tile (counting sort in LDS)
  const int nvt = a.nvt;
  for (int v = tid; v < nvt; v += NT) cnt[v] = 0;
  __syncthreads();
  const int ne = nr * K;
  const int32_t* idx = a.idx + int64_t(r0) * K;
  for (int e = tid; e < ne; e += NT) {
    const int id = idx[e];
    if (unsigned(id) < unsigned(a.V)) atomicAdd(&cnt[id >> 8], 1);
  }
  __syncthreads();
  const int seg = (nvt + NT - 1) / NT;
  const int b0 = tid * seg;
  int loc = 0;
  for (int q = 0; q < seg; ++q)
    if (b0 + q < nvt) loc += cnt[b0 + q];
  part[tid] = loc;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {
    const int x = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += x;
    __syncthreads();
  }
  int run = part[tid] - loc;
  int32_t* bo = a.boff + int64_t(pt) * (nvt + 1);
  for (int q = 0; q < seg; ++q) {
    const int v = b0 + q;
    if (v < nvt) {
      const int c = cnt[v];
      bo[v] = run;
      cnt[v] = run;
      run += c;
    }
  }
  if (tid == NT - 1) bo[nvt] = part[NT - 1];
  __syncthreads();
  uint32_t* ent = a.ent + int64_t(pt) * kTile * K;
  for (int e = tid; e < ne; e += NT) {
    const int id = idx[e];
    if (unsigned(id) < unsigned(a.V)) {
      const int rr = e / K, k = e - rr * K;
      const int pos = atomicAdd(&cnt[id >> 8], 1);
      ent[pos] = (uint32_t(rr) << 16) | (uint32_t(id & (kTile - 1)) << 8) | uint32_t(k);
    }
  }
}

template <int MODE>  // 0: forward epilogue, 1: backward epilogue
__global__ __launch_bounds__(NT) void logits_kernel(LogitsArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM_ELEMS];
  const int total = a.nvt * a.npt;
  const int tile = xcd_remap(blockIdx.x, total);
  const int vt = tile / a.npt, pt = tile - vt * a.npt;
  const int v0 = vt * kTile, p0 = pt * kTile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16 acc[4][4];
  // A = W rows (vocab), B = H_c rows (positions); both K(=D)-contiguous.
  gemm_mainloop<LoadKC, LoadKC>(a.W, a.D, v0, a.V, a.D, a.Hc, a.D, p0, a.rows, a.D, 0, a.D, acc, smem);

  float* S = reinterpret_cast<float*>(smem);
  float* red = S + STAGE_FLOATS;  // [4][256]
  const bool vtail = v0 + kTile > a.V;
  const int ebeg = a.boff[int64_t(pt) * (a.nvt + 1) + vt];
  const int eend = a.boff[int64_t(pt) * (a.nvt + 1) + vt + 1];
  const uint32_t* ent = a.ent + int64_t(pt) * kTile * a.K;

  if (MODE == 0) {
    // z = acc / T; vocab rows past V do not exist
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float z = acc[i][j][r] * a.invT;
          if (vtail && v0 + acc_row(wm, i, r, lane) >= a.V) z = -INFINITY;
          acc[i][j][r] = z;
        }
    // per-position max and sum of exp over the tile's 256 vocab rows
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, acc[i][j][r]);
      float s = 0.f;
      if (m != -INFINITY) {
        const float mb = m * LOG2E;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) s += exp2_fast(fmaf(acc[i][j][r], LOG2E, -mb));
      }
      lse_merge(m, s, __shfl_xor(m, 32), __shfl_xor(s, 32));
      if (lane < 32) {
        const int pl = wn * 128 + j * 32 + lane;
        red[wm * kTile + pl] = m;
        red[(2 + wm) * kTile + pl] = s;
      }
    }
    __syncthreads();
    {
      float m = red[tid], s = red[2 * kTile + tid];
      lse_merge(m, s, red[kTile + tid], red[3 * kTile + tid]);
      const int prow = p0 + tid;
      if (prow < a.rows) {
        a.pm[int64_t(vt) * a.c_pad + prow] = m;
        a.ps[int64_t(vt) * a.c_pad + prow] = s;
      }
    }
    if (ebeg == eend) return;
    // logits at the cached ids that fall in this tile
    for (int h = 0; h < 2; ++h) {
      if (wn == h) stage_half(S, acc, wm, lane);
      __syncthreads();
      for (int e = ebeg + tid; e < eend; e += NT) {
        const uint32_t pk = ent[e];
        const int row = int(pk >> 16);
        if ((row >> 7) == h) {
          const int vl = int((pk >> 8) & 0xffu), k = int(pk & 0xffu);
          a.zsel[int64_t(p0 + row) * a.K + k] = S[(row & 127) * SLD + vl];
        }
      }
      __syncthreads();
    }
  } else {
    const float gs = a.g_scale * (a.grad_loss != nullptr ? a.grad_loss[0] : 1.f);
    float lse_l2[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int prow = p0 + wn * 128 + j * 32 + (lane & 31);
      lse_l2[j] = prow < a.rows ? a.lse[prow] * LOG2E : INFINITY;
    }
    // gs * softmax(z) over the full vocabulary, from the forward's lse
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float q = exp2_fast(fmaf(acc[i][j][r] * a.invT, LOG2E, -lse_l2[j]));
          if (vtail && v0 + acc_row(wm, i, r, lane) >= a.V) q = 0.f;
          acc[i][j][r] = gs * q;
        }
    for (int h = 0; h < 2; ++h) {
      if (wn == h) stage_half(S, acc, wm, lane);
      __syncthreads();
      // minus the teacher probability at each cached id (scatter-add)
      for (int e = ebeg + tid; e < eend; e += NT) {
        const uint32_t pk = ent[e];
        const int row = int(pk >> 16);
        if ((row >> 7) == h) {
          const int vl = int((pk >> 8) & 0xffu), k = int(pk & 0xffu);
          atomicAdd(S + (row & 127) * SLD + vl, -gs * a.p[int64_t(p0 + row) * a.K + k]);
        }
      }
      __syncthreads();
      // round to bf16 and write 128 rows x 256 vocab of G_c
#pragma unroll 4
      for (int it = 0; it < 16; ++it) {
        const int pl = it * 8 + (tid >> 5);
        const int c8 = (tid & 31) * 8;
        const int prow = p0 + h * 128 + pl;
        if (prow < a.rows) {
          const float4 x0 = *reinterpret_cast<const float4*>(S + pl * SLD + c8);
          const float4 x1 = *reinterpret_cast<const float4*>(S + pl * SLD + c8 + 4);
          uint4 o;
          o.x = bf16_rne(x0.x) | (bf16_rne(x0.y) << 16);
          o.y = bf16_rne(x0.z) | (bf16_rne(x0.w) << 16);
          o.z = bf16_rne(x1.x) | (bf16_rne(x1.y) << 16);
          o.w = bf16_rne(x1.z) | (bf16_rne(x1.w) << 16);
          *reinterpret_cast<uint4*>(a.G + int64_t(prow) * a.Vp + v0 + c8) = o;
        }
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(NT) void combine_kernel(CombineArgs a) {
  __shared__ float sm[8][32], ss[8][32], sg[8][32];
  const int tid = threadIdx.x, rl = tid & 31, g = tid >> 5;
  const int r = blockIdx.x * 32 + rl;
  float m = -INFINITY, s = 0.f, gz = 0.f;
  if (r < a.rows) {
    for (int vt = g; vt < a.nvt; vt += 8)
      lse_merge(m, s, a.pm[int64_t(vt) * a.c_pad + r], a.ps[int64_t(vt) * a.c_pad + r]);
    for (int k = g; k < a.K; k += 8)
      gz += a.p[int64_t(r) * a.K + k] * a.zsel[int64_t(r) * a.K + k];
  }
  sm[g][rl] = m;
  ss[g][rl] = s;
  sg[g][rl] = gz;
  __syncthreads();
  if (g == 0 && r < a.rows) {
    for (int q = 1; q < 8; ++q) {
      lse_merge(m, s, sm[q][rl], ss[q][rl]);
      gz += sg[q][rl];
    }
    const float lse = m + logf(s);
    a.lse[r] = lse;
    a.rowkl[r] = a.h[r] - gz + lse;
  }
}

__global__ __launch_bounds__(NT) void finalize_kernel(const float* __restrict__ rowkl, int64_t N,
                                                      float* __restrict__ loss) {
  __shared__ double red[NT];
  const int tid = threadIdx.x;
  double acc = 0.0;
  for (int64_t i = tid; i < N; i += NT) acc += double(rowkl[i]);
  red[tid] = acc;
  __syncthreads();
  for (int o = NT / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0) loss[0] = N > 0 ? float(red[0] / double(N)) : 0.f;
}

__global__ __launch_bounds__(NT) void dh_kernel(DhArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM_ELEMS];
  const int tiles_m = (a.rows + kTile - 1) / kTile;
  const int tiles_n = (a.D + kTile - 1) / kTile;
  const int tiles = tiles_m * tiles_n;
  const int tile = xcd_remap(blockIdx.x, tiles * a.split);
  const int sp = tile / tiles, rem = tile - sp * tiles;
  const int tm = rem % tiles_m, tn = rem / tiles_m;
  const int k_begin = sp * a.ktiles_per_split * BK;
  int k_end = k_begin + a.ktiles_per_split * BK;
  if (k_end > a.Vp) k_end = int(a.Vp);
  f32x16 acc[4][4];
  // A = G_c (positions x vocab, vocab-contiguous), B = W (vocab x D, D-contiguous)
  gemm_mainloop<LoadKC, LoadMC>(a.G, a.Vp, tm * kTile, a.rows, int(a.Vp), a.W, a.D, tn * kTile, a.D,
                                a.V, k_begin, k_end, acc, smem);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = tn * kTile + wn * 128 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int prow = tm * kTile + acc_row(wm, i, r, lane);
        if (prow < a.rows && d < a.D) {
          if (a.split > 1)
            a.part[(int64_t(sp) * a.c_pad + prow) * a.D + d] = acc[i][j][r];
          else
            a.dH[int64_t(prow) * a.D + d] = uint16_t(bf16_rne(acc[i][j][r]));
        }
      }
    }
}

__global__ __launch_bounds__(NT) void dh_reduce_kernel(const float* __restrict__ part, int split,
                                                       int64_t n4, int64_t split_stride4,
                                                       uint16_t* __restrict__ dH) {
  const int64_t i = int64_t(blockIdx.x) * NT + threadIdx.x;
  if (i >= n4) return;
  const float4* p4 = reinterpret_cast<const float4*>(part);
  float4 s = p4[i];
  for (int q = 1; q < split; ++q) {
    const float4 x = p4[q * split_stride4 + i];
    s.x += x.x;
    s.y += x.y;
    s.z += x.z;
    s.w += x.w;
  }
  uint2 o;
  o.x = bf16_rne(s.x) | (bf16_rne(s.y) << 16);
  o.y = bf16_rne(s.z) | (bf16_rne(s.w) << 16);
  reinterpret_cast<uint2*>(dH)[i] = o;
}

__global__ __launch_bounds__(NT) void dw_kernel(DwArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM_ELEMS];
  const int tiles_m = int((a.V + kTile - 1) / kTile);
  const int tiles_n = (a.D + kTile - 1) / kTile;
  const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
  f32x16 acc[4][4];
  // A[v][p] = G_c[p][v] (vocab-contiguous), B[p][d] = H_c[p][d] (D-contiguous)
  gemm_mainloop<LoadMC, LoadMC>(a.G, a.Vp, tm * kTile, int(a.Vp), a.rows, a.Hc, a.D, tn * kTile, a.D,
                                a.rows, 0, a.rows, acc, smem);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // Read-modify-write of the fp32 dW tile in four batches of 64 values per
  // lane: all loads of a batch are issued before its stores, so they overlap
  // instead of forming 256 dependent round trips.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float old[4][16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = tn * kTile + wn * 128 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = tm * kTile + acc_row(wm, i, r, lane);
        old[j][r] = (v < a.V && d < a.D) ? a.dW[int64_t(v) * a.D + d] : 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = tn * kTile + wn * 128 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = tm * kTile + acc_row(wm, i, r, lane);
        if (v < a.V && d < a.D) a.dW[int64_t(v) * a.D + d] = old[j][r] + acc[i][j][r];
      }
    }
  }
}

__global__ __launch_bounds__(NT) void validate_kernel(const int32_t* __restrict__ idx, int64_t N,
                                                      int K, int64_t V, int32_t* flags) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * (NT / 64) + (threadIdx.x >> 6);
  if (row >= N) return;
  const int32_t* r = idx + row * K;
  int f = 0;
  for (int k = lane; k < K; k += 64) {
    const int id = r[k];
    if (id < 0 || int64_t(id) >= V) f |= 1;
    for (int j = 0; j < K; ++j)
      if (j != k && r[j] == id) {
        f |= 2;
        break;
      }
  }
  if (f) atomicOr(flags, f);
}

__global__ __launch_bounds__(NT) void fill_f32_kernel(float* p, int64_t n, float v) {
  const int64_t i = int64_t(blockIdx.x) * NT + threadIdx.x;
  if (i < n) p[i] = v;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

hipError_t launch_prep(const PrepArgs& a, int npt, hipStream_t s) {
  hipLaunchKernelGGL(prep_kernel, dim3(npt), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_logits_fwd(const LogitsArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(logits_kernel<0>, dim3(a.nvt * a.npt), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_logits_bwd(const LogitsArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(logits_kernel<1>, dim3(a.nvt * a.npt), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3(unsigned(ceil_div(a.rows, 32))), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* rowkl, int64_t N, float* loss, hipStream_t s) {
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(NT), 0, s, rowkl, N, loss);
  return hipGetLastError();
}

hipError_t launch_dh(const DhArgs& a, hipStream_t s) {
  const int64_t tiles = ceil_div(a.rows, kTile) * ceil_div(a.D, kTile);
  hipLaunchKernelGGL(dh_kernel, dim3(unsigned(tiles * a.split)), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dh_reduce(const float* part, int split, int rows, int D, int64_t c_pad,
                            uint16_t* dH, hipStream_t s) {
  const int64_t n4 = int64_t(rows) * D / 4;
  const int64_t stride4 = c_pad * D / 4;
  hipLaunchKernelGGL(dh_reduce_kernel, dim3(unsigned(ceil_div(n4, NT))), dim3(NT), 0, s, part, split,
                     n4, stride4, dH);
  return hipGetLastError();
}

hipError_t launch_dw(const DwArgs& a, hipStream_t s) {
  const int64_t tiles = ceil_div(a.V, kTile) * ceil_div(a.D, kTile);
  hipLaunchKernelGGL(dw_kernel, dim3(unsigned(tiles)), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_validate(const int32_t* idx, int64_t N, int K, int64_t V, int32_t* flags,
                           hipStream_t s) {
  hipLaunchKernelGGL(fill_f32_kernel, dim3(1), dim3(NT), 0, s, reinterpret_cast<float*>(flags), 1, 0.f);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || N == 0) return e;
  hipLaunchKernelGGL(validate_kernel, dim3(unsigned(ceil_div(N, NT / 64))), dim3(NT), 0, s, idx, N, K, V,
                     flags);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  hipLaunchKernelGGL(fill_f32_kernel, dim3(unsigned(ceil_div(n, NT))), dim3(NT), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace kd
