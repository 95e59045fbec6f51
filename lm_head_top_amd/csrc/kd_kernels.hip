// gfx950 kernels of the fused chunked top-K KL distillation loss.
//
// The method ("Distilling an LLM on One GPU", section "The two changes"; "The
// $250GB Memory Spike That Killed Distillation Projects Is Now Optional",
// section "Fused Chunked KL: The Loss That Never Builds the Full Grid"): one chunk of positions
// at a time, project the hidden states to logits, fold them into the running
// loss and drop them; the backward recomputes each chunk's logits.  Here every
// chunk runs as
//
//   teacher   p = softmax_K(t/T) and h = sum p log p per position (one wave per row);
//   bucket    the chunk's (row, id, k) cache entries, counting-sorted by (position
//             tile, vocab tile) so each logits tile finds exactly its own entries;
//   logits    z^T = W H_c^T / T for 256 x 256 (vocab, position) tiles on bf16
//             MFMA (v_mfma_f32_32x32x16_bf16), one workgroup per compute unit
//             walking its tiles in bands of 4 position tiles, then per tile
//             forward: per-position tile max / sum-exp and the logits at the
//                      cached ids go to small buffers (never the tile itself);
//             backward: G = g/(N T) (exp(z - lse) - p scattered at the ids),
//                      rounded to bf16 into G_c[c, V];
//   combine   forward: merge the vocab-tile partials into lse and KL per row;
//   dh / dw   over the G rows of a group of chunks: dH = G W in blocks of up to
//             4096 rows (split over V into fp32 partials only when a block's
//             tiles cannot fill the chip) and dW += G^T H, reading G, W and H
//             as they are stored.
//
// GEMM core: a 256 x 256 output tile per workgroup, split over waves 2 (M) x
// WAVES/2 (N); each wave holds its (128 x 256/(WAVES/2)) part as 32x32 fp32
// MFMA accumulators.  Tiles of BK along K stream from HBM straight into LDS
// with buffer_load_dwordx4 ... lds (no register staging; out-of-range rows
// and columns read as zero), through a ring of STAGES buffers.  An operand
// is either K-contiguous (W and H_c in the logits GEMM, G in dH): its LDS
// tile is 256 rows of BK, 16-byte chunks XOR-swizzled by row, and a fragment
// is one ds_read_b128; or k-major (W in dH, G and H in dW): its LDS tile is
// BK rows of 256, 64-byte blocks XOR-swizzled by row, and a fragment is two
// ds_read_b64_tr_b16, gfx950's transposing LDS read.  A compute unit accepts
// one 1 KiB direct load about every 20 cycles for all its waves together, so
// the loads are spread between the MFMAs rather than issued in a burst.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "kd_kernels.h"

// Build knobs (defaults are the measured best on MI355X)
#ifndef KD_BK
#define KD_BK 64  // K depth of one pipeline stage
#endif
#ifndef KD_WAVES
#define KD_WAVES 8  // waves per GEMM workgroup: 8 (two per SIMD) or 4
#endif
#ifndef KD_LOAD_AUX
#define KD_LOAD_AUX 0  // cache-policy bits of the direct LDS loads
#endif
// Operand given a third LDS slot, so its loads run two stages ahead:
// 0 none, 1 A, 2 B (per GEMM kernel)
#ifndef KD_DEEP_LOGITS
#define KD_DEEP_LOGITS 1
#endif
#ifndef KD_DEEP_DH
#define KD_DEEP_DH 0
#endif
#ifndef KD_DEEP_DW
#define KD_DEEP_DW 0
#endif
// Ring loads of a stage: 0 = both operands' go out after the stage barrier
// in the last MFMA step; 1 = only the operand that must land first does, the
// other's go out in the next stage's first step (per GEMM kernel)
#ifndef KD_SPLIT_LOGITS
#define KD_SPLIT_LOGITS 1
#endif
#ifndef KD_SPLIT_DH
#define KD_SPLIT_DH 0
#endif
#ifndef KD_SPLIT_DW
#define KD_SPLIT_DW 0
#endif
// dW tile order: 0 = D tile fastest; b > 0 = bands of b vocab tiles, vocab
// tile fastest within a band
#ifndef KD_DW_BAND
#define KD_DW_BAND 4
#endif
// logits kernels: 0 = one workgroup per tile; 1 = one workgroup per compute
// unit looping over tiles
#ifndef KD_PERSIST_LOGITS
#define KD_PERSIST_LOGITS 1
#endif
// logits tile order: 0 = position tile fastest within a vocab tile; b > 0 =
// bands of b position tiles, position tile fastest within a band
#ifndef KD_LOGITS_BAND
#define KD_LOGITS_BAND 4
#endif
// dH tile order: bands of this many row tiles, row tile fastest
#ifndef KD_DH_BAND
#define KD_DH_BAND 4
#endif
// Debug builds (1) check the indices of the cache-entry scatters and gathers
// against the extents they address; a failed check skips the access and
// sets a bit of a device word that the entry points read back.
#ifndef KD_DEBUG_BOUNDS
#define KD_DEBUG_BOUNDS 0
#endif

namespace kd {
namespace {

constexpr int NT = 256;                          // threads of the small kernels
constexpr int WAVES = KD_WAVES;                  // 8: two waves per SIMD; 4: one
constexpr int GT = WAVES * 64;                   // threads per GEMM workgroup
constexpr int WAVES_M = 2;
constexpr int WAVES_N = WAVES / WAVES_M;
constexpr int WT_M = kTile / WAVES_M;            // wave tile rows (128)
constexpr int WT_N = kTile / WAVES_N;            // wave tile columns (64 or 128)
constexpr int MI = WT_M / 32;                    // 32-row MFMA blocks per wave
constexpr int NJ = WT_N / 32;                    // 32-column MFMA blocks per wave
constexpr int BK = KD_BK;                        // K columns per pipeline stage
constexpr int STAGES = 2;                        // LDS slots per operand (a deep operand has 3)
constexpr int CH = BK / 8;                       // 16-byte chunks per LDS row
constexpr int ROWB = BK * 2;                     // bytes per LDS row
constexpr int RPI = 64 / CH;                     // rows covered by one 1 KiB direct load
constexpr int NI = kTile * ROWB / 1024 / WAVES;  // direct loads per wave, per operand, per stage
constexpr int OPER_BYTES = kTile * ROWB;         // one operand tile in LDS
constexpr int STAGE_BYTES = 2 * OPER_BYTES;
constexpr int MAIN_BYTES = STAGES * STAGE_BYTES;
// LDS of the main loop when one operand has a third slot
constexpr int ring_bytes(int deep) { return deep ? MAIN_BYTES + OPER_BYTES : MAIN_BYTES; }
constexpr int NS = BK / 16;                      // 16-deep MFMA steps per stage
constexpr int SLD = kTile + 4;                   // fp32 row stride of the epilogue staging tile
constexpr int STAGE_FLOATS = 128 * SLD;          // half a tile: 128 positions x 256 vocab
constexpr int EPI_BYTES = (STAGE_FLOATS + 10 * kTile) * 4;
constexpr int SMEM_BYTES =
    ring_bytes(KD_DEEP_LOGITS) > EPI_BYTES ? ring_bytes(KD_DEEP_LOGITS) : EPI_BYTES;
constexpr uint32_t kOOB = 0xFFFFFFF0u;           // buffer offset past any operand: reads return 0

#if KD_DEBUG_BOUNDS
// bit 0: a bucketed entry's slot, bit 1: a forward gather, bit 2: a backward scatter
__device__ unsigned debug_fault;
#endif

// True when ok; in debug builds a false check also records bit.
__device__ __forceinline__ bool kd_check(bool ok, int bit) {
#if KD_DEBUG_BOUNDS
  if (!ok) atomicOr(&debug_fault, 1u << bit);
  return ok;
#else
  (void)ok;
  (void)bit;
  return true;
#endif
}
constexpr float LOG2E = 1.4426950408889634f;

static_assert(BK == 32 || BK == 64, "BK");
static_assert(WAVES == 4 || WAVES == 8, "WAVES");
static_assert(SMEM_BYTES <= 160 * 1024 && ring_bytes(1) <= 160 * 1024, "LDS budget of one gfx950 workgroup");

// GEMM kernels: one workgroup per compute unit; with 4 waves each wave may use
// the whole register file of its SIMD (accumulators in AGPRs).
#define KD_GEMM_KERNEL __global__ __launch_bounds__(GT) __attribute__((amdgpu_waves_per_eu(WAVES / 4, WAVES / 4)))

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> bf16, round to nearest even, by gfx950's v_cvt_pk_bf16_f32 (two
// values per instruction; denormals kept, NaN stays a NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

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

// s_waitcnt vmcnt(N) (gfx9 encoding; expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt vmcnt(N) lgkmcnt(0): this wave's loads but the newest N have
// landed and its LDS reads are done.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// Workgroup barrier that orders LDS accesses for the compiler but does not wait
// for outstanding loads (the LDS ring is managed with explicit vmcnt waits).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// XOR swizzle of the 16-byte chunks of LDS row r.  gfx950 serves a
// ds_read_b128 16 lanes at a time from 64 four-byte banks (a 256-byte
// window); the MFMA fragment read puts 16 consecutive rows at one logical
// chunk, and the swizzle gives those 16 rows 16 distinct 16-byte bank slots.
__device__ __forceinline__ int swz(int r) {
  return CH == 8 ? ((r & 7) ^ ((r >> 3) & 1)) : ((r >> 2) & 3);
}

// ------------------------------------------------------ direct LDS loads ---

// Streams a 256-row, K-contiguous operand X[row][k] (leading dimension ld,
// elements) into LDS tiles of 256 x BK.  Each wave issues NI direct loads of
// 1 KiB; lane l of load j fills LDS row r = (wave*NI + j)*RPI + l/CH,
// physical chunk l%CH, with logical chunk (l%CH) ^ swz(r).  Rows at or past
// row_lim and columns at or past k_lim read as zero.
struct DLoad {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff[NI];
  int kc[NI];  // first k of this lane's chunk within a tile, per load

  __device__ __forceinline__ void init(const uint16_t* base, uint64_t bytes, int64_t ld, int row0,
                                       int row_lim) {
    const uint32_t nrec = bytes < uint64_t(kOOB) ? uint32_t(bytes) : kOOB;
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, int(nrec), 0x00020000);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rib = lane / CH, phys = lane % CH;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int rt = (wave * NI + j) * RPI + rib;  // row within the tile (row0 % 256 == 0)
      kc[j] = (phys ^ swz(rt)) * 8;
      const int row = row0 + rt;
      voff[j] = row < row_lim ? uint32_t((int64_t(row) * ld + kc[j]) * 2) : kOOB;
    }
  }

  // Load j (of NI) of the 256 x BK tile at columns [k0, k0 + BK) into stage.
  __device__ __forceinline__ void issue_one(int j, char* stage, int k0, int k_lim) const {
    const int wave = threadIdx.x >> 6;
    const bool ok = (voff[j] != kOOB) & (k0 + kc[j] < k_lim);
    const uint32_t off = ok ? voff[j] + uint32_t(k0) * 2u : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(stage + (wave * NI + j) * 1024), 16, off,
                                             0, 0, KD_LOAD_AUX);
  }

  __device__ __forceinline__ void issue(char* stage, int k0, int k_lim) const {
#pragma unroll
    for (int j = 0; j < NI; ++j) issue_one(j, stage, k0, k_lim);
  }
};

// Streams an operand stored k-major, X[k][m] (m contiguous, leading dimension
// ld elements), into LDS tiles of BK rows (k) by 256 columns (m), 512 bytes a
// row.  Load j of wave w fills rows 2(w*NI + j) and 2(w*NI + j) + 1: lane l
// writes physical 16-byte chunk l%32 of row r = 2(w*NI + j) + l/32, which
// holds the logical 64-byte block ((l%32)/4) ^ (r & 3) of that row (32
// columns), so the transposing fragment reads below hit 64 distinct banks.
// Columns at or past m_lim and rows at or past k_lim read as zero.
struct MLoad {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff[NI];  // byte offset of (row, this lane's columns) for k0 = 0, or kOOB
  int kr[NI];         // tile row of this lane's chunk, per load
  uint32_t ldb;       // row stride in bytes

  __device__ __forceinline__ void init(const uint16_t* base, uint64_t bytes, int64_t ld, int m0,
                                       int m_lim) {
    const uint32_t nrec = bytes < uint64_t(kOOB) ? uint32_t(bytes) : kOOB;
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, int(nrec), 0x00020000);
    ldb = uint32_t(ld) * 2u;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane & 31;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int r = 2 * (wave * NI + j) + (lane >> 5);
      kr[j] = r;
      const int m = (((c >> 2) ^ (r & 3)) << 5) + (c & 3) * 8;
      voff[j] = m0 + m < m_lim ? uint32_t((int64_t(r) * ld + m0 + m) * 2) : kOOB;
    }
  }

  // Load j (of NI) of the BK x 256 tile at rows [k0, k0 + BK) into stage.
  __device__ __forceinline__ void issue_one(int j, char* stage, int k0, int k_lim) const {
    const int wave = threadIdx.x >> 6;
    // non-short-circuit test: a select, not a branch around the load
    const bool ok = (voff[j] != kOOB) & (k0 + kr[j] < k_lim);
    const uint32_t off = ok ? voff[j] + uint32_t(k0) * ldb : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(stage + (wave * NI + j) * 1024), 16, off,
                                             0, 0, KD_LOAD_AUX);
  }

  __device__ __forceinline__ void issue(char* stage, int k0, int k_lim) const {
#pragma unroll
    for (int j = 0; j < NI; ++j) issue_one(j, stage, k0, k_lim);
  }
};

static_assert(OPER_BYTES == BK * 512, "a k-major tile holds BK rows of 256 bf16");

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// MFMA 32x32x16 operand fragment (lane l: column l%32, k = 8(l/32) .. +7) from
// a k-major LDS tile: ds_read_b64_tr_b16 hands lane i of a 16-lane group the
// 16-bit element i%4 of the 8 bytes addressed by lanes 4s + i/4 (s = 0..3).
// Lane L of the group addresses row k0 + L/4, columns 4(L%4) .. +3, so lane i
// receives rows k0 .. k0+3 of column i; two reads (rows +0 and +4) give 8 k.
// `lane_off` is the lane's byte offset for block column 0 of step 0 without
// the block swizzle (see mn_lane_off).
__device__ __forceinline__ int mn_lane_off(int lane) {
  const int gq = lane >> 4, i16 = lane & 15;
  return (8 * (gq >> 1) + (i16 >> 2)) * 512 + (16 * (gq & 1) + 4 * (i16 & 3)) * 2;
}

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// One ds_read_b64_tr_b16.  The __restrict__ parameter gives the read alias
// scope information; without it the compiler waits for every direct LDS load
// in flight (vmcnt(0)) before a transposing read.  The GEMM loops order these
// reads against the direct loads with their own vmcnt waits and barriers.
__device__ __forceinline__ s16x4 ds_read_tr(const lds_s16x4* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_s16x4*>(p));
}

__device__ __forceinline__ bf16x8 frag_mn(const char* tile, int col0, int s, int lane, int lane_off) {
  // row & 3 of every row this lane addresses equals (lane & 15) >> 2
  const int blk = (col0 >> 5) ^ ((lane & 15) >> 2);
  const char* p = tile + s * (16 * 512) + lane_off + (blk << 6);
  const s16x4 lo = ds_read_tr((const lds_s16x4*)(p));
  const s16x4 hi = ds_read_tr((const lds_s16x4*)(p + 4 * 512));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// --------------------------------------------------------------- MFMA core ---

// MFMA 32x32x16 operands: lane l supplies row l % 32 and the 8 consecutive k
// of half l / 32; an operand tile is row-major with k contiguous (AMN / BMN
// false, one ds_read_b128 per fragment) or k-major (true, two transposing
// reads).
//
// One BK-deep stage with the barrier in its last step.  On entry fa[0] and
// fb[0] hold the stage's first-step fragments; steps read the next step's
// fragments while they multiply.  In the last step the wave waits for its own
// loads of the next stage (all but the newest VMW) and for its LDS reads, then
// passes the workgroup barrier: every wave has then finished reading this
// stage's slots and the next stage has landed.  It then reads the next
// stage's first-step fragments from nsA / nsB (into fa[0] / fb[0]) and
// refills this stage's slots (ring loads to ldA / ldB, the operand that must
// land first going out first) while the last step's MFMAs run.  With SPLIT
// only that operand goes out there; the other one's loads (to dd at dk) go
// out in the first step of the stage, for the slot the previous barrier
// freed.
template <bool AMN, bool BMN, bool B_FIRST, int VMW, bool SPLIT, class LA, class LB>
__device__ __forceinline__ void mma_stage_eb(const char* __restrict__ sA, const char* __restrict__ sB,
                                             const char* __restrict__ nsA, const char* __restrict__ nsB,
                                             bf16x8 (&fa)[2][MI], bf16x8 (&fb)[2][NJ], f32x16 (&acc)[MI][NJ],
                                             int wm, int wn, int lane, const LA& la, const LB& lb, char* ldA,
                                             int lka, char* ldB, int lkb, char* dd, int dk, int ka_lim,
                                             int kb_lim) {
  constexpr int NR = (AMN ? 2 : 1) * MI + (BMN ? 2 : 1) * NJ;  // fragment reads per step
  constexpr int NQ = MI * NJ;                                  // MFMAs per step
  constexpr int NL = 2 * NI;                                   // ring loads per stage
  static_assert(NS % 2 == 0, "the next stage's first fragments go to buffer 0");
  const int r31 = lane & 31, hi = lane >> 5, sw = swz(r31);
  const int mo = mn_lane_off(lane);
  auto read_a = [&](const char* t, int i, int st) -> bf16x8 {
    if constexpr (AMN) return frag_mn(t, wm * WT_M + i * 32, st, lane, mo);
    else
      return *reinterpret_cast<const bf16x8*>(t + (wm * WT_M + i * 32 + r31) * ROWB + (((2 * st + hi) ^ sw) * 16));
  };
  auto read_b = [&](const char* t, int j, int st) -> bf16x8 {
    if constexpr (BMN) return frag_mn(t, wn * WT_N + j * 32, st, lane, mo);
    else
      return *reinterpret_cast<const bf16x8*>(t + (wn * WT_N + j * 32 + r31) * ROWB + (((2 * st + hi) ^ sw) * 16));
  };
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) {
    const int cur = s & 1;
#pragma unroll
    for (int i = 0; i < MI; ++i) fa[cur ^ 1][i] = read_a(sA, i, s + 1);
#pragma unroll
    for (int j = 0; j < NJ; ++j) fb[cur ^ 1][j] = read_b(sB, j, s + 1);
    // deferred ring loads of the operand that lands second (SPLIT)
    if (SPLIT && s == 0) {
#pragma unroll
      for (int l = 0; l < NI; ++l) {
        if (B_FIRST) la.issue_one(l, dd, dk, ka_lim);
        else lb.issue_one(l, dd, dk, kb_lim);
      }
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
    const int nl = SPLIT && s == 0 ? NI : 0;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      const int rq = (NR * (q + 1)) / NQ - (NR * q) / NQ;
#pragma unroll
      for (int u = 0; u < rq; ++u) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      const int lq = (nl * (q + 1)) / NQ - (nl * q) / NQ;
#pragma unroll
      for (int u = 0; u < lq; ++u) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
  }
  constexpr int cur = (NS - 1) & 1;
  wait_vmcnt_lds<VMW>();
  lds_barrier();
#pragma unroll
  for (int i = 0; i < MI; ++i) fa[cur ^ 1][i] = read_a(nsA, i, 0);
#pragma unroll
  for (int j = 0; j < NJ; ++j) fb[cur ^ 1][j] = read_b(nsB, j, 0);
  constexpr int NLL = SPLIT ? NI : NL;  // ring loads in this step
#pragma unroll
  for (int l = 0; l < NLL; ++l) {
    if (l < NI) {
      if (B_FIRST) lb.issue_one(l, ldB, lkb, kb_lim);
      else la.issue_one(l, ldA, lka, ka_lim);
    } else {
      if (B_FIRST) la.issue_one(l - NI, ldA, lka, ka_lim);
      else lb.issue_one(l - NI, ldB, lkb, kb_lim);
    }
  }
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    const int rq = (NR * (q + 1)) / NQ - (NR * q) / NQ;
#pragma unroll
    for (int u = 0; u < rq; ++u) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    const int lq = (NLL * (q + 1)) / NQ - (NLL * q) / NQ;
#pragma unroll
    for (int u = 0; u < lq; ++u) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
}

// Multiplies the 256 x 256 tile over k in [k_begin, k_end) into acc.  The
// operands stream into an LDS ring, OPER_BYTES per slot: the A slots, then
// the B slots (ring_bytes(DEEP) in all).  Each operand has two slots, or
// three for the DEEP one (1: A, 2: B), whose loads then run two stages
// ahead.  The loads of an operand's stage s go to slot s % slots; stages past
// the end load zeros that nothing reads.
//
// Stage kt's barrier sits in its last MFMA step (mma_stage_eb).  After it,
// stage kt's slots take the operand stages kt + slots: the operand that must
// land first (B when A is deep, else A) goes out at once; the other one goes
// out there too, or with SPLIT in the next stage's first step.  The wave's
// wait before each barrier leaves in flight only the loads issued after the
// next stage's, so one wait and the barrier cover both operands of it.
template <bool AMN, bool BMN, int DEEP, bool SPLIT, class LA, class LB>
__device__ __forceinline__ void gemm_core(const LA& la, const LB& lb, int k_begin, int k_end,
                                          int ka_lim, int kb_lim, f32x16 (&acc)[MI][NJ], char* smem) {
  static_assert(DEEP >= 0 && DEEP <= 2, "DEEP");
  constexpr int SA = STAGES + (DEEP == 1 ? 1 : 0);  // A slots
  constexpr int SB = STAGES + (DEEP == 2 ? 1 : 0);  // B slots
  constexpr bool B_FIRST = DEEP == 1;
  char* const sa0 = smem;
  char* const sb0 = smem + SA * OPER_BYTES;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int nk = (k_end - k_begin + BK - 1) / BK;
  if (nk <= 0) return;
  // Prologue: A0 B0 A1 B1, then A2 (DEEP 1) or B2 (DEEP 2).  With SPLIT the
  // last of these (B1 when DEEP is 0) goes out in stage 0's first step
  // instead, as the second operand's loads of every later stage do.
  la.issue(sa0, k_begin, ka_lim);
  lb.issue(sb0, k_begin, kb_lim);
  la.issue(sa0 + OPER_BYTES, 1 < nk ? k_begin + BK : 0x3fffffff, ka_lim);
  if (!SPLIT || DEEP) lb.issue(sb0 + OPER_BYTES, 1 < nk ? k_begin + BK : 0x3fffffff, kb_lim);
  if (!SPLIT && DEEP == 1) la.issue(sa0 + 2 * OPER_BYTES, 2 < nk ? k_begin + 2 * BK : 0x3fffffff, ka_lim);
  if (!SPLIT && DEEP == 2) lb.issue(sb0 + 2 * OPER_BYTES, 2 < nk ? k_begin + 2 * BK : 0x3fffffff, kb_lim);
  // stage 0 of both operands has landed once only the loads issued after it remain
  wait_vmcnt<(DEEP ? 3 : 2) * NI - (SPLIT ? NI : 0)>();
  lds_barrier();
  bf16x8 fa[2][MI], fb[2][NJ];
  {
    const int r31 = lane & 31, hi = lane >> 5, sw = swz(r31), mo = mn_lane_off(lane);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      if constexpr (AMN) fa[0][i] = frag_mn(sa0, wm * WT_M + i * 32, 0, lane, mo);
      else fa[0][i] = *reinterpret_cast<const bf16x8*>(sa0 + (wm * WT_M + i * 32 + r31) * ROWB + ((hi ^ sw) * 16));
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if constexpr (BMN) fb[0][j] = frag_mn(sb0, wn * WT_N + j * 32, 0, lane, mo);
      else fb[0][j] = *reinterpret_cast<const bf16x8*>(sb0 + (wn * WT_N + j * 32 + r31) * ROWB + ((hi ^ sw) * 16));
    }
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int na = kt + SA, nb = kt + SB;
    const int lka = na < nk ? k_begin + na * BK : 0x3fffffff;
    const int lkb = nb < nk ? k_begin + nb * BK : 0x3fffffff;
    char* const cA = sa0 + (kt % SA) * OPER_BYTES;
    char* const cB = sb0 + (kt % SB) * OPER_BYTES;
    // SPLIT: the operand loaded second takes its stage kt + slots - 1 in this
    // stage's first step, into the slot freed by the previous barrier
    constexpr int SX = B_FIRST ? SA : SB;
    const int nd = kt + SX - 1;
    char* const dd = (B_FIRST ? sa0 : sb0) + (nd % SX) * OPER_BYTES;
    const int dk = nd < nk ? k_begin + nd * BK : 0x3fffffff;
    mma_stage_eb<AMN, BMN, B_FIRST, DEEP ? NI : 0, SPLIT>(cA, cB, sa0 + ((kt + 1) % SA) * OPER_BYTES,
                                                          sb0 + ((kt + 1) % SB) * OPER_BYTES, fa, fb, acc, wm, wn,
                                                          lane, la, lb, cA, lka, cB, lkb, dd, dk, ka_lim, kb_lim);
  }
  wait_vmcnt<0>();  // the trailing zero loads land before the epilogue reuses LDS
  lds_barrier();
}

// Row (within the 256-row tile) of accumulator register r of block i.
__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane) {
  return wm * WT_M + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Column (within the tile) of the accumulators of block j.
__device__ __forceinline__ int acc_col(int wn, int j, int lane) { return wn * WT_N + j * 32 + (lane & 31); }

// Writes the wave's columns that fall in half h (columns h*128 .. h*128+127)
// to the staging area S[column - h*128][row] (fp32, row stride SLD).
__device__ __forceinline__ void stage_half(float* S, const f32x16 (&acc)[MI][NJ], int wm, int wn, int lane,
                                           int h) {
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int col = acc_col(wn, j, lane);
    if ((wn * WT_N + j * 32) >> 7 != h) continue;  // uniform per wave
    const int pl = col & 127;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int vl = wm * WT_M + i * 32 + 8 * g + 4 * (lane >> 5);
        *reinterpret_cast<float4*>(S + pl * SLD + vl) =
            make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
      }
  }
}

// ---------------------------------------------------------- teacher side ---

// p = softmax over the K cached teacher logits at temperature T, and
// h = sum_k p log p (0 log 0 = 0); one wave per position.
__global__ __launch_bounds__(NT) void teacher_kernel(TeacherArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * (NT / 64) + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int K = a.K;
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

// Counting sort of one position tile's cache entries by vocab tile.  A row
// has KE entries: its K cached ids (k < K) and, with labels, the label (k =
// K).  Entry word: row-in-tile << 17 | id % 256 << 9 | k.  Ids outside
// [0, V) (and negative labels) are dropped.
//
// The cached ids are walked in their stored order (entry e of the tile is
// idx[r0 * K + e]); each thread loads all its entries at once (up to K = 128;
// more take further rounds) and keeps them in registers for the scatter.  The
// sorted list is built in LDS and copied out with coalesced stores when it
// fits (KE <= 118), else scattered straight to memory.  Cached ids crowd into
// the first vocab tiles (frequent tokens) and LDS atomics on one address
// serialize, so each tile gets bs counters (lane % bs picks one; bs = 16 down
// to 1 as the vocabulary grows, within the LDS left); the scan runs over
// (tile, counter) in order, so a tile's entries stay contiguous.
constexpr int BT = 1024;                   // threads of the bucketing kernel
constexpr int BU = 32;                     // entries per thread per round
constexpr int kBucketStage = 118 * kTile;  // entries of the LDS copy
constexpr int kBucketCnt = 10240;          // counters (>= kMaxVocabTiles)
static_assert(kBucketCnt >= kMaxVocabTiles, "one counter per vocab tile at least");

__global__ __launch_bounds__(BT) void bucket_kernel(BucketArgs a) {
  __shared__ int cnt[kBucketCnt];
  __shared__ int wsum[BT / 64];
  __shared__ uint32_t stage[kBucketStage];
  const int pt = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // this block's chunk: rows [crow0, crow0 + crows) of the run
  const int crow0 = int(blockIdx.y) * a.chunk;
  const int crows = min(a.chunk, a.rows - crow0);
  const int r0 = pt * kTile;  // within the chunk
  if (r0 >= crows) return;    // a tile past a short last chunk (the whole block)
  const int nr = min(kTile, crows - r0);
  const int nvt = a.nvt;
  const int32_t* labels = a.labels != nullptr ? a.labels + crow0 : nullptr;
  int bsh = 4;  // log2 of the counters per tile
  while (bsh > 0 && (nvt << bsh) > kBucketCnt) --bsh;
  const int nc = nvt << bsh;
  const int sub = lane & ((1 << bsh) - 1);
  const int nk = nr * a.K;  // cached entries of the tile
  const int32_t* idx = a.idx + (int64_t(crow0) + r0) * a.K;
  const float invK = 1.f / float(a.K);
  int id[BU];
  auto load = [&](int e0) {
#pragma unroll
    for (int u = 0; u < BU; ++u) {
      const int e = e0 + u * BT + tid;
      id[u] = e < nk ? idx[e] : -1;
    }
  };
  load(0);  // in flight while the counters are cleared
  for (int v = tid; v < nc; v += BT) cnt[v] = 0;
  __syncthreads();
  for (int e0 = 0;;) {
#pragma unroll
    for (int u = 0; u < BU; ++u)
      if (unsigned(id[u]) < unsigned(a.V)) atomicAdd(&cnt[((id[u] >> 8) << bsh) | sub], 1);
    e0 += BU * BT;
    if (e0 >= nk) break;
    load(e0);
  }
  if (labels != nullptr)
    for (int rr = tid; rr < nr; rr += BT) {
      const int y = labels[r0 + rr];
      if (unsigned(y) < unsigned(a.V)) atomicAdd(&cnt[((y >> 8) << bsh) | sub], 1);
    }
  __syncthreads();
  // exclusive scan of the counters: each thread owns seg consecutive ones;
  // shuffles scan within a wave, then the 16 wave totals
  const int seg = (nc + BT - 1) / BT;
  const int b0 = tid * seg;
  int loc = 0;
  for (int q = 0; q < seg; ++q)
    if (b0 + q < nc) loc += cnt[b0 + q];
  int x = loc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = lane < BT / 64 ? wsum[lane] : 0;
#pragma unroll
    for (int o = 1; o < BT / 64; o <<= 1) {
      const int y = __shfl_up(w, o);
      if (lane >= o) w += y;
    }
    if (lane < BT / 64) wsum[lane] = w;
  }
  __syncthreads();
  int run = (wave > 0 ? wsum[wave - 1] : 0) + x - loc;
  const int total = wsum[BT / 64 - 1];
  int32_t* bo = a.boff + int64_t(blockIdx.y) * a.boff_stride + int64_t(pt) * (nvt + 1);
  for (int q = 0; q < seg; ++q) {
    const int v = b0 + q;
    if (v < nc) {
      const int c = cnt[v];
      if ((v & ((1 << bsh) - 1)) == 0) bo[v >> bsh] = run;
      cnt[v] = run;
      run += c;
    }
  }
  if (tid == BT - 1) bo[nvt] = total;
  __syncthreads();
  uint32_t* ent = a.ent + int64_t(blockIdx.y) * a.ent_stride + int64_t(pt) * kTile * a.KE;
  const bool in_lds = nr * a.KE <= kBucketStage;  // uniform
  uint32_t* dst = in_lds ? stage : ent;
  const bool multi = nk > BU * BT;  // else the ids are still in registers
  for (int e0 = 0; e0 < nk; e0 += BU * BT) {
    if (multi) load(e0);
#pragma unroll
    for (int u = 0; u < BU; ++u)
      if (unsigned(id[u]) < unsigned(a.V)) {
        const int e = e0 + u * BT + tid;
        // e / K through the float reciprocal: (e + 0.5) / K < 256 misses every
        // integer by at least 1/(2K) >= 2^-9, and the two roundings err by less
        // than 2^-15 (checked exhaustively for every K and e on the host)
        const int rr = int((float(e) + 0.5f) * invK);
        const int k = e - rr * a.K;
        const int pos = atomicAdd(&cnt[((id[u] >> 8) << bsh) | sub], 1);
        if (kd_check(pos >= 0 && pos < nr * a.KE && rr < nr && k < a.K, 0))
          dst[pos] = (uint32_t(rr) << 17) | (uint32_t(id[u] & (kTile - 1)) << 9) | uint32_t(k);
      }
  }
  if (labels != nullptr)
    for (int rr = tid; rr < nr; rr += BT) {
      const int y = labels[r0 + rr];
      if (unsigned(y) < unsigned(a.V)) {
        const int pos = atomicAdd(&cnt[((y >> 8) << bsh) | sub], 1);
        if (kd_check(pos >= 0 && pos < nr * a.KE && a.K < a.KE, 0))
          dst[pos] = (uint32_t(rr) << 17) | (uint32_t(y & (kTile - 1)) << 9) | uint32_t(a.K);
      }
    }
  if (in_lds) {
    __syncthreads();
    for (int i = tid; i < total; i += BT) ent[i] = stage[i];
  }
}

// ----------------------------------------------------------- logits tile ---

// (m, S0, S1) <- merge of two teacher triples (max of a, sum exp(a - max),
// sum exp(a - max) (a - b)).
__device__ __forceinline__ void tri_merge(float& m, float& s0, float& s1, float m2, float t0, float t1) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) {
    m = M;
    s0 = s1 = 0.f;
    return;
  }
  const float e1 = exp2_fast((m - M) * LOG2E), e2 = exp2_fast((m2 - M) * LOG2E);
  s0 = s0 * e1 + t0 * e2;
  s1 = s1 * e1 + t1 * e2;
  m = M;
}

// Four consecutive teacher logits t[p][v .. v+3] (fp32 or bf16) as loaded:
// 16 bytes of fp32, or 8 bytes of bf16 in .x / .y.
__device__ __forceinline__ uint4 teacher_raw(const void* t, int dtype, int64_t off) {
  if (dtype == 0) return *reinterpret_cast<const uint4*>(static_cast<const float*>(t) + off);
  const uint2 h = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(t) + off);
  return make_uint4(h.x, h.y, 0u, 0u);
}

// The four logits of teacher_raw times 1/T.
__device__ __forceinline__ float4 teacher_cvt(uint4 r, int dtype, float invT) {
  if (dtype == 0)
    return make_float4(__uint_as_float(r.x) * invT, __uint_as_float(r.y) * invT, __uint_as_float(r.z) * invT,
                       __uint_as_float(r.w) * invT);
  return make_float4(__uint_as_float(r.x << 16) * invT, __uint_as_float(r.x & 0xffff0000u) * invT,
                     __uint_as_float(r.y << 16) * invT, __uint_as_float(r.y & 0xffff0000u) * invT);
}

// Loads the teacher logits of one accumulator column (position p0 + pl) for
// all MI x 4 register groups of the wave, every load in flight at once;
// groups past V or past the chunk read element 0 and are marked invalid.
__device__ __forceinline__ void teacher_column(const void* t, int dtype, int64_t V, int rows, int p0, int pl,
                                               int v0, int wm, int lane, uint4 (&raw)[MI][4],
                                               bool (&ok)[MI][4]) {
  const bool pok = p0 + pl < rows;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int vr = v0 + acc_row(wm, i, 4 * g, lane);
      ok[i][g] = pok && vr < V;  // V % 4 == 0: vr < V covers vr .. vr + 3
      raw[i][g] = teacher_raw(t, dtype, ok[i][g] ? int64_t(p0 + pl) * V + vr : 0);
    }
}

// 0: forward epilogue, 1: backward epilogue, 2: forward epilogue that also
// stores z, 3: dense-teacher forward epilogue, 4: dense-teacher backward epilogue
template <int MODE>
__device__ __forceinline__ void logits_tile(const LogitsArgs& a, int t, char* smem) {
  const int total = a.nvt * a.npt;
  const int tile = xcd_remap(t, total);
#if KD_LOGITS_BAND > 0
  // bands of up to KD_LOGITS_BAND position tiles, position tile fastest: the
  // 32 tiles an XCD runs at once cover 32 / band vocab tiles x band position
  // tiles, whose operand strips its L2 shares
  constexpr int LB = KD_LOGITS_BAND;
  const int band = tile / (LB * a.nvt), bw = min(LB, a.npt - LB * band);
  const int bi = tile - band * LB * a.nvt;
  const int pt = LB * band + bi % bw, vt = bi / bw;
#else
  const int vt = tile / a.npt, pt = tile - vt * a.npt;
#endif
  const int v0 = vt * kTile, p0 = pt * kTile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  f32x16 acc[MI][NJ];
  {
    // A = W rows (vocab), B = H_c rows (positions); both D-contiguous
    DLoad la, lb;
    la.init(a.W, uint64_t(a.V) * a.D * 2, a.D, v0, a.V);
    lb.init(a.Hc, uint64_t(a.rows) * a.D * 2, a.D, p0, a.rows);
    gemm_core<false, false, KD_DEEP_LOGITS, KD_SPLIT_LOGITS != 0>(la, lb, 0, a.D, a.D, a.D, acc, smem);
  }

  float* S = reinterpret_cast<float*>(smem);
  float* red = S + STAGE_FLOATS;  // [4][256]
  const bool vtail = v0 + kTile > a.V;
  constexpr bool CACHE = MODE <= 2;  // top-K cache entries (the dense-teacher modes have none)
  const int ebeg = CACHE ? a.boff[int64_t(pt) * (a.nvt + 1) + vt] : 0;
  const int eend = CACHE ? a.boff[int64_t(pt) * (a.nvt + 1) + vt + 1] : 0;
  const uint32_t* ent = CACHE ? a.ent + int64_t(pt) * kTile * a.KE : nullptr;

  if (MODE == 0 || MODE == 2 || MODE == 3) {
    // vocab rows past V do not exist (a uniform branch: only the last vocab tile)
    if (vtail) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (v0 + acc_row(wm, i, r, lane) >= a.V) acc[i][j][r] = -INFINITY;
    }
    // the top-K mode keeps acc = T z (T > 0, so the order and the max carry
    // over) and folds 1/T into the exponent and the gathered values; the
    // others need z = acc / T in the registers
    constexpr bool SCALED = MODE != 0;
    if (SCALED) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] *= a.invT;
    }
    const float ez = SCALED ? LOG2E : a.invT * LOG2E;  // exp(z - m) = exp2(acc ez - m_acc ez)
    if (MODE == 2) {
      // keep z[position][vocab] (fp32, row stride Vp): registers 4g .. 4g+3
      // of a block are 4 consecutive vocab rows at one position
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int prow = p0 + acc_col(wn, j, lane);
        if (prow < a.rows) {
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g)
              *reinterpret_cast<float4*>(a.zkeep + int64_t(prow) * a.Vp + v0 + acc_row(wm, i, 4 * g, lane)) =
                  make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                              acc[i][j][4 * g + 3]);
        }
      }
    }
    // per-position max and sum of exp over the tile's 256 vocab rows
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, acc[i][j][r]);
      float s = 0.f;
      if (m != -INFINITY) {
        const float mb = m * ez;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) s += exp2_fast(fmaf(acc[i][j][r], ez, -mb));
      }
      if (!SCALED) m *= a.invT;  // the max in logit units
      lse_merge(m, s, __shfl_xor(m, 32), __shfl_xor(s, 32));
      if (lane < 32) {
        const int pl = acc_col(wn, j, lane);
        red[wm * kTile + pl] = m;
        red[(2 + wm) * kTile + pl] = s;
      }
    }
    if (MODE == 3) {
      // teacher: a = t / T over the same (vocab, position) tile; per position
      // max of a, sum exp(a - max) and sum exp(a - max) (a - z)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int pl = acc_col(wn, j, lane);
        uint4 raw[MI][4];
        bool ok[MI][4];
        teacher_column(a.tlog, a.t_dtype, a.V, a.rows, p0, pl, v0, wm, lane, raw, ok);
        float tm = -INFINITY;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            if (ok[i][g]) {
              const float4 t4 = teacher_cvt(raw[i][g], a.t_dtype, a.invT);
              tm = fmaxf(tm, fmaxf(fmaxf(t4.x, t4.y), fmaxf(t4.z, t4.w)));
            }
        float t0 = 0.f, t1 = 0.f;
        if (tm != -INFINITY) {
          const float tmb = tm * LOG2E;
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g)
              if (ok[i][g]) {
                const float4 t4 = teacher_cvt(raw[i][g], a.t_dtype, a.invT);
                const float tq[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
                for (int q = 0; q < 4; ++q)
                  if (tq[q] != -INFINITY) {
                    const float e = exp2_fast(fmaf(tq[q], LOG2E, -tmb));
                    t0 += e;
                    t1 += e * (tq[q] - acc[i][j][4 * g + q]);
                  }
              }
        }
        tri_merge(tm, t0, t1, __shfl_xor(tm, 32), __shfl_xor(t0, 32), __shfl_xor(t1, 32));
        if (lane < 32) {
          red[(4 + wm) * kTile + pl] = tm;
          red[(6 + wm) * kTile + pl] = t0;
          red[(8 + wm) * kTile + pl] = t1;
        }
        __builtin_amdgcn_sched_barrier(0);  // one column's loads in flight at a time
      }
    }
    __syncthreads();
    if (tid < kTile) {
      float m = red[tid], s = red[2 * kTile + tid];
      lse_merge(m, s, red[kTile + tid], red[3 * kTile + tid]);
      const int prow = p0 + tid;
      if (prow < a.rows) {
        a.pm[int64_t(vt) * a.c_pad + prow] = m;
        a.ps[int64_t(vt) * a.c_pad + prow] = s;
      }
      if (MODE == 3) {
        float tm = red[4 * kTile + tid], t0 = red[6 * kTile + tid], t1 = red[8 * kTile + tid];
        tri_merge(tm, t0, t1, red[5 * kTile + tid], red[7 * kTile + tid], red[9 * kTile + tid]);
        if (prow < a.rows) {
          a.tm[int64_t(vt) * a.c_pad + prow] = tm;
          a.ts0[int64_t(vt) * a.c_pad + prow] = t0;
          a.ts1[int64_t(vt) * a.c_pad + prow] = t1;
        }
      }
    }
    if (MODE == 3 || ebeg == eend) return;
    if (!kd_check(0 <= ebeg && ebeg <= eend && eend <= kTile * a.KE, 1)) return;
    // logits at the cached ids that fall in this tile
    for (int h = 0; h < 2; ++h) {
      stage_half(S, acc, wm, wn, lane, h);
      __syncthreads();
      for (int e = ebeg + tid; e < eend; e += GT) {
        const uint32_t pk = ent[e];
        const int row = int(pk >> 17);
        if ((row >> 7) == h) {
          const int vl = int((pk >> 9) & 0xffu), k = int(pk & 0x1ffu);
          const float zv = S[(row & 127) * SLD + vl];
          if (kd_check(k < a.KE && p0 + row < a.rows, 1))
            a.zsel[int64_t(p0 + row) * a.KE + k] = SCALED ? zv : zv * a.invT;
        }
      }
      __syncthreads();
    }
  } else {
    const float gs = a.g_scale * (a.grad_loss != nullptr ? a.grad_loss[0] : 1.f);
    const float iws = a.row_w != nullptr ? a.inv_wsum[0] : 1.f;
    // per position: lse, and gs * w_n / sum w * (alpha + beta [label]) on the softmax
    float lse_l2[NJ], qs[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int prow = p0 + acc_col(wn, j, lane);
      const bool ok = prow < a.rows;
      lse_l2[j] = ok ? a.lse[prow] * LOG2E : INFINITY;
      const float rs = ok && a.row_w != nullptr ? a.row_w[prow] * iws : 1.f;
      const bool lab = ok && a.labels != nullptr && unsigned(a.labels[prow]) < unsigned(a.V);
      qs[j] = gs * rs * (lab ? a.alpha + a.beta : a.alpha);
    }
    // gs * softmax(z) over the full vocabulary, from the forward's lse:
    // exp(acc / T - lse) = exp2(acc ez - lse log2 e)
    const float ez = a.invT * LOG2E;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = qs[j] * exp2_fast(fmaf(acc[i][j][r], ez, -lse_l2[j]));
    // vocab rows past V do not exist (a uniform branch: only the last vocab tile)
    if (vtail) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (v0 + acc_row(wm, i, r, lane) >= a.V) acc[i][j][r] = 0.f;
    }
    if (MODE == 4) {
      // minus gs * softmax(t / T) over the full vocabulary, from the teacher's lse
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int pl = acc_col(wn, j, lane);
        uint4 raw[MI][4];
        bool ok[MI][4];
        teacher_column(a.tlog, a.t_dtype, a.V, a.rows, p0, pl, v0, wm, lane, raw, ok);
        const float tl2 = p0 + pl < a.rows ? a.lse_t[p0 + pl] * LOG2E : 0.f;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            if (!ok[i][g]) continue;
            const float4 t4 = teacher_cvt(raw[i][g], a.t_dtype, a.invT);
            acc[i][j][4 * g] -= gs * exp2_fast(fmaf(t4.x, LOG2E, -tl2));
            acc[i][j][4 * g + 1] -= gs * exp2_fast(fmaf(t4.y, LOG2E, -tl2));
            acc[i][j][4 * g + 2] -= gs * exp2_fast(fmaf(t4.z, LOG2E, -tl2));
            acc[i][j][4 * g + 3] -= gs * exp2_fast(fmaf(t4.w, LOG2E, -tl2));
          }
        __builtin_amdgcn_sched_barrier(0);  // one column's loads in flight at a time
      }
    }
    const bool ents_ok = !CACHE || kd_check(0 <= ebeg && ebeg <= eend && eend <= kTile * a.KE, 2);
    for (int h = 0; h < 2; ++h) {
      stage_half(S, acc, wm, wn, lane, h);
      __syncthreads();
      // minus alpha p at each cached id and beta at the label (scatter-add),
      // times gs w_n / sum w
      for (int e = ebeg + tid; ents_ok && e < eend; e += GT) {
        const uint32_t pk = ent[e];
        const int row = int(pk >> 17);
        if ((row >> 7) == h) {
          const int vl = int((pk >> 9) & 0xffu), k = int(pk & 0x1ffu);
          const int prow = p0 + row;
          if (!kd_check(k < a.KE && prow < a.rows, 2)) continue;
          const float rs = a.row_w != nullptr ? a.row_w[prow] * iws : 1.f;
          const float mass = k < a.K ? a.alpha * a.p[int64_t(prow) * a.K + k] : a.beta;
          atomicAdd(S + (row & 127) * SLD + vl, -(gs * rs) * mass);
        }
      }
      __syncthreads();
      // G_c rows: 128 positions x 256 vocab, bf16 (the dH and dW GEMMs both
      // read this one copy)
#pragma unroll 4
      for (int it = 0; it < 128 * 32 / GT; ++it) {
        const int pl = it * (GT / 32) + (tid >> 5);
        const int c8 = (tid & 31) * 8;
        const int prow = p0 + h * 128 + pl;
        if (prow < a.rows) {
          const float4 x0 = *reinterpret_cast<const float4*>(S + pl * SLD + c8);
          const float4 x1 = *reinterpret_cast<const float4*>(S + pl * SLD + c8 + 4);
          uint4 o;
          o.x = bf16x2_rne(x0.x, x0.y);
          o.y = bf16x2_rne(x0.z, x0.w);
          o.z = bf16x2_rne(x1.x, x1.y);
          o.w = bf16x2_rne(x1.z, x1.w);
          *reinterpret_cast<uint4*>(a.G + int64_t(prow) * a.Vp + v0 + c8) = o;
        }
      }
      __syncthreads();
    }
  }
}

template <int MODE>
KD_GEMM_KERNEL void logits_kernel(LogitsArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[SMEM_BYTES];
#if KD_PERSIST_LOGITS
  // one workgroup per compute unit walks the tiles b, b + grid, ...: the
  // tiles an XCD runs at a time stay those of the one-tile-per-workgroup grid
  // (the grid is a multiple of 8), without a workgroup launch between them
  const int total = a.nvt * a.npt;
  for (int t = blockIdx.x; t < total; t += gridDim.x) {
    logits_tile<MODE>(a, t, smem);
    __syncthreads();  // the next tile's loads refill the LDS this epilogue read
  }
#else
  logits_tile<MODE>(a, blockIdx.x, smem);
#endif
}

// ----------------------------------------------------------------- combine ---

// One block per CR positions; its CG thread groups each merge every CG-th
// vocabulary tile's (max, sum exp) partial and every CG-th cached entry, then
// two LDS rounds merge the groups (8 groups each, then the 8 results), so each
// thread's chain of dependent merges is short.  Blocks are dealt so that the
// blocks reading one 128-byte line of partials share an XCD's L2.
constexpr int CR = 4;        // positions per combine block
constexpr int CG = NT / CR;  // thread groups per position
static_assert(CG == 64, "two merge rounds of 8");

__global__ __launch_bounds__(NT) void combine_kernel(CombineArgs a) {
  __shared__ float sm[CG][CR], ss[CG][CR], sg[CG][CR];
  const int tid = threadIdx.x, rl = tid % CR, g = tid / CR;
  const int r = xcd_remap(blockIdx.x, gridDim.x) * CR + rl;
  float m = -INFINITY, s = 0.f, gz = 0.f;
  if (r < a.rows) {
    for (int vt = g; vt < a.nvt; vt += CG)
      lse_merge(m, s, a.pm[int64_t(vt) * a.c_pad + r], a.ps[int64_t(vt) * a.c_pad + r]);
    for (int k = g; k < a.K; k += CG)
      gz += a.p[int64_t(r) * a.K + k] * a.zsel[int64_t(r) * a.KE + k];
  }
  sm[g][rl] = m;
  ss[g][rl] = s;
  sg[g][rl] = gz;
  __syncthreads();
  if (g < 8) {
#pragma unroll
    for (int q = 1; q < 8; ++q) {
      lse_merge(m, s, sm[g + 8 * q][rl], ss[g + 8 * q][rl]);
      gz += sg[g + 8 * q][rl];
    }
    sm[g][rl] = m;
    ss[g][rl] = s;
    sg[g][rl] = gz;
  }
  __syncthreads();
  if (g == 0 && r < a.rows) {
#pragma unroll
    for (int q = 1; q < 8; ++q) {
      lse_merge(m, s, sm[q][rl], ss[q][rl]);
      gz += sg[q][rl];
    }
    const float lse = m + logf(s);
    a.lse[r] = lse;
    float l = a.h[r] - gz + lse;  // KL_n
    if (a.labels != nullptr) {    // the loss terms: scale (alpha KL_n + beta CE_n)
      const int y = a.labels[r];
      const float ce = unsigned(y) < unsigned(a.V) ? lse - a.zsel[int64_t(r) * a.KE + a.K] : 0.f;
      l = a.scale * (a.alpha * l + a.beta * ce);
    } else if (a.alpha != 1.f || a.scale != 1.f) {
      l = a.scale * (a.alpha * l);
    }
    a.rowkl[r] = l;
  }
}

// Dense teacher: lse of the student and of the teacher from the vocab-tile
// partials, and KL_n = sum_v p (a - z) - lse_a + lse_z with
// sum_v p (a - z) = S1 / S0.  Laid out like combine_kernel: CR positions per
// block, CG groups each merging every CG-th vocab tile, then two LDS rounds.
__global__ __launch_bounds__(NT) void dense_combine_kernel(DenseCombineArgs a) {
  __shared__ float sm[CG][CR], ss[CG][CR], stm[CG][CR], st0[CG][CR], st1[CG][CR];
  const int tid = threadIdx.x, rl = tid % CR, g = tid / CR;
  const int r = xcd_remap(blockIdx.x, gridDim.x) * CR + rl;
  float m = -INFINITY, s = 0.f, tm = -INFINITY, t0 = 0.f, t1 = 0.f;
  if (r < a.rows)
    for (int vt = g; vt < a.nvt; vt += CG) {
      const int64_t o = int64_t(vt) * a.c_pad + r;
      lse_merge(m, s, a.pm[o], a.ps[o]);
      tri_merge(tm, t0, t1, a.tm[o], a.ts0[o], a.ts1[o]);
    }
  sm[g][rl] = m;
  ss[g][rl] = s;
  stm[g][rl] = tm;
  st0[g][rl] = t0;
  st1[g][rl] = t1;
  __syncthreads();
  if (g < 8) {
#pragma unroll
    for (int q = 1; q < 8; ++q) {
      lse_merge(m, s, sm[g + 8 * q][rl], ss[g + 8 * q][rl]);
      tri_merge(tm, t0, t1, stm[g + 8 * q][rl], st0[g + 8 * q][rl], st1[g + 8 * q][rl]);
    }
    sm[g][rl] = m;
    ss[g][rl] = s;
    stm[g][rl] = tm;
    st0[g][rl] = t0;
    st1[g][rl] = t1;
  }
  __syncthreads();
  if (g == 0 && r < a.rows) {
#pragma unroll
    for (int q = 1; q < 8; ++q) {
      lse_merge(m, s, sm[q][rl], ss[q][rl]);
      tri_merge(tm, t0, t1, stm[q][rl], st0[q][rl], st1[q][rl]);
    }
    const float lse = m + logf(s);
    const float lse_t = tm + logf(t0);
    a.lse[r] = lse;
    a.lse_t[r] = lse_t;
    a.rowkl[r] = t1 / t0 - lse_t + lse;
  }
}

// loss = sum_n w_n l_n / sum_n w_n (w_n = 1 without weights; 0 for an empty
// or all-zero weight), summed in fp64 in a fixed order.  Also leaves
// 1 / sum_n w_n in *inv_wsum when asked (the backward's per-row factor).
constexpr int FT = 1024;  // threads of the finalize kernel
__global__ __launch_bounds__(FT) void finalize_kernel(const float* __restrict__ rowl, const float* __restrict__ w,
                                                      int64_t N, float* __restrict__ loss, float* inv_wsum) {
  __shared__ double red[FT], redw[FT];
  const int tid = threadIdx.x;
  double acc = 0.0, aw = 0.0;
  for (int64_t i = tid; i < N; i += FT) {
    const double wi = w != nullptr ? double(w[i]) : 1.0;
    if (rowl != nullptr && wi != 0.0) acc += wi * double(rowl[i]);
    aw += wi;
  }
  red[tid] = acc;
  redw[tid] = aw;
  __syncthreads();
  for (int o = FT / 2; o > 0; o >>= 1) {
    if (tid < o) {
      red[tid] += red[tid + o];
      redw[tid] += redw[tid + o];
    }
    __syncthreads();
  }
  if (tid == 0) {
    if (loss != nullptr) loss[0] = redw[0] != 0.0 ? float(red[0] / redw[0]) : 0.f;
    if (inv_wsum != nullptr) inv_wsum[0] = redw[0] != 0.0 ? float(1.0 / redw[0]) : 0.f;
  }
}

// --------------------------------------------------------------- dH and dW ---

KD_GEMM_KERNEL void dh_kernel(DhArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[ring_bytes(KD_DEEP_DH)];
  const int tiles_m = (a.rows + kTile - 1) / kTile;
  const int tiles_n = (a.D + kTile - 1) / kTile;
  const int tiles = tiles_m * tiles_n;
  const int tile = xcd_remap(blockIdx.x, tiles * a.split);
  const int sp = tile / tiles, rem = tile - sp * tiles;
  // bands of up to 4 row tiles, row tile fastest: the 32 tiles an XCD runs at
  // once cover 4 row tiles x 8 column tiles, whose operand strips its L2 shares
  constexpr int HB = KD_DH_BAND;
  const int band = rem / (HB * tiles_n), bh = min(HB, tiles_m - HB * band);
  const int bi = rem - band * HB * tiles_n;
  const int tm = HB * band + bi % bh, tn = bi / bh;
  const int k_begin = sp * a.ktiles_per_split * BK;
  int k_end = k_begin + a.ktiles_per_split * BK;
  if (k_end > a.Vp) k_end = int(a.Vp);
  f32x16 acc[MI][NJ];
  {
    // A = G (positions x vocab, vocab-contiguous); B = W read k-major
    // (vocab rows, D contiguous) through the transposing fragment reads
    DLoad la;
    MLoad lb;
    la.init(a.G, uint64_t(a.rows) * a.Vp * 2, a.Vp, tm * kTile, a.rows);
    lb.init(a.W, uint64_t(a.V) * a.D * 2, a.D, tn * kTile, a.D);
    gemm_core<false, true, KD_DEEP_DH, KD_SPLIT_DH != 0>(la, lb, k_begin, k_end, int(a.Vp), a.V, acc, smem);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  // uniform: one scalar register, so later stores never wait on its load
  const float sc = a.scale != nullptr ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.scale[0])))
                                      : 1.f;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int d = tn * kTile + acc_col(wn, j, lane);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int prow = tm * kTile + acc_row(wm, i, r, lane);
        if (prow < a.rows && d < a.D) {
          if (a.split > 1)
            a.part[(int64_t(sp) * a.c_pad + prow) * a.D + d] = sc * acc[i][j][r];
          else
            a.dH[int64_t(prow) * a.D + d] = uint16_t(bf16_rne(sc * acc[i][j][r]));
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
  o.x = bf16x2_rne(s.x, s.y);
  o.y = bf16x2_rne(s.z, s.w);
  reinterpret_cast<uint2*>(dH)[i] = o;
}

KD_GEMM_KERNEL void dw_kernel(DwArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[ring_bytes(KD_DEEP_DW)];
  const int tiles_m = int((a.V + kTile - 1) / kTile);
  const int tiles_n = (a.D + kTile - 1) / kTile;
  const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  int tm, tn;
  if (KD_DW_BAND > 0) {
    constexpr int B = KD_DW_BAND > 0 ? KD_DW_BAND : 1;
    const int band = tile / (B * tiles_n), bh = min(B, tiles_m - B * band);
    const int bi = tile - band * B * tiles_n;
    tm = B * band + bi % bh;
    tn = bi / bh;
  } else {
    tm = tile / tiles_n;
    tn = tile - tm * tiles_n;
  }
  f32x16 acc[MI][NJ];
  {
    // A = G^T and B = H^T of the chunk group, both read k-major from G
    // (positions x vocab) and H (positions x D) as they are stored
    MLoad la, lb;
    la.init(a.G, uint64_t(a.rows) * a.Vp * 2, a.Vp, tm * kTile, int(a.Vp));
    lb.init(a.H, uint64_t(a.rows) * a.D * 2, a.D, tn * kTile, a.D);
    gemm_core<true, true, KD_DEEP_DW, KD_SPLIT_DW != 0>(la, lb, 0, a.rows, a.rows, a.rows, acc, smem);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  // uniform: one scalar register, so later stores never wait on its load
  const float sc = a.scale != nullptr ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.scale[0])))
                                      : 1.f;
  // dW += tile with one fp32 atomic add per element (no value returned): the
  // read-modify-write happens in L2, so the workgroup does not wait for the
  // old values.  Each element gets exactly one add per launch, so the result
  // equals a plain read-modify-write and does not depend on timing.
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int d = tn * kTile + acc_col(wn, j, lane);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = tm * kTile + acc_row(wm, i, r, lane);
        if (v < a.V && d < a.D) unsafeAtomicAdd(a.dW + int64_t(v) * a.D + d, sc * acc[i][j][r]);
      }
    }
}

// ------------------------------------------------- kept-gradient (comparator) ---

// z[p][v] <- exp(z[p][v] - lse[p]) in place, for p < rows, v < Vp (the kept
// logits of one chunk; v >= V hold -inf and become 0).
__global__ __launch_bounds__(NT) void keep_softmax_kernel(float* __restrict__ z, const float* __restrict__ lse,
                                                          int rows, int64_t Vp) {
  const int64_t q = int64_t(blockIdx.x) * NT + threadIdx.x;  // float4 index
  const int64_t per_row = Vp / 4;
  if (q >= int64_t(rows) * per_row) return;
  const int64_t p = q / per_row;
  const float l2 = lse[p] * LOG2E;
  float4 v = reinterpret_cast<float4*>(z)[q];
  v.x = exp2_fast(fmaf(v.x, LOG2E, -l2));
  v.y = exp2_fast(fmaf(v.y, LOG2E, -l2));
  v.z = exp2_fast(fmaf(v.z, LOG2E, -l2));
  v.w = exp2_fast(fmaf(v.w, LOG2E, -l2));
  reinterpret_cast<float4*>(z)[q] = v;
}

// z[p][idx[p][k]] -= p[p][k] (duplicates add up; ids outside [0, V) skipped).
__global__ __launch_bounds__(NT) void keep_scatter_kernel(float* __restrict__ z, const int32_t* __restrict__ idx,
                                                          const float* __restrict__ pk, int rows, int K, int V,
                                                          int64_t Vp) {
  const int64_t e = int64_t(blockIdx.x) * NT + threadIdx.x;
  if (e >= int64_t(rows) * K) return;
  const int64_t p = e / K;
  const int id = idx[e];
  if (unsigned(id) < unsigned(V)) atomicAdd(z + p * Vp + id, -pk[e]);
}

// G[p][v] = bf16(gs * z[p][v]) for p < rows, v < Vp (16 bytes of G per thread).
__global__ __launch_bounds__(NT) void keep_convert_kernel(const float* __restrict__ z, float gs, int rows,
                                                          int64_t Vp, uint16_t* __restrict__ G) {
  const int64_t q = int64_t(blockIdx.x) * NT + threadIdx.x;  // 8-element index
  if (q >= int64_t(rows) * (Vp / 8)) return;
  const float4 x0 = reinterpret_cast<const float4*>(z)[2 * q];
  const float4 x1 = reinterpret_cast<const float4*>(z)[2 * q + 1];
  uint4 o;
  o.x = bf16x2_rne(gs * x0.x, gs * x0.y);
  o.y = bf16x2_rne(gs * x0.z, gs * x0.w);
  o.z = bf16x2_rne(gs * x1.x, gs * x1.y);
  o.w = bf16x2_rne(gs * x1.z, gs * x1.w);
  reinterpret_cast<uint4*>(G)[q] = o;
}

// ---------------------------------------------------------------- utility ---

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

int gemm_bk() { return BK; }

hipError_t launch_teacher(const TeacherArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(teacher_kernel, dim3(unsigned(ceil_div(a.rows, NT / 64))), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bucket(const BucketArgs& a, int npt, int nchunks, hipStream_t s) {
  hipLaunchKernelGGL(bucket_kernel, dim3(npt, nchunks), dim3(BT), 0, s, a);
  return hipGetLastError();
}

// Workgroups of a logits launch: one per tile, or with KD_PERSIST_LOGITS one
// per compute unit of the current device (a multiple of 8), at most one per tile.
unsigned logits_grid(const LogitsArgs& a) {
  const unsigned tiles = unsigned(a.nvt) * unsigned(a.npt);
  if (!KD_PERSIST_LOGITS) return tiles;
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return tiles;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return tiles;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  const unsigned g = unsigned(n) / 8 * 8;
  return g == 0 || tiles <= g ? tiles : g;
}

hipError_t launch_logits_fwd(const LogitsArgs& a, hipStream_t s) {
  const dim3 grid(logits_grid(a));
  if (a.tlog != nullptr)
    hipLaunchKernelGGL(logits_kernel<3>, grid, dim3(GT), 0, s, a);
  else if (a.zkeep != nullptr)
    hipLaunchKernelGGL(logits_kernel<2>, grid, dim3(GT), 0, s, a);
  else
    hipLaunchKernelGGL(logits_kernel<0>, grid, dim3(GT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_keep_grad(float* z, const float* lse, const int32_t* idx, const float* p, int rows, int K,
                            int V, int64_t Vp, float gs, uint16_t* G, hipStream_t s) {
  const int64_t n4 = int64_t(rows) * (Vp / 4);
  hipLaunchKernelGGL(keep_softmax_kernel, dim3(unsigned(ceil_div(n4, NT))), dim3(NT), 0, s, z, lse, rows, Vp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t ne = int64_t(rows) * K;
  hipLaunchKernelGGL(keep_scatter_kernel, dim3(unsigned(ceil_div(ne, NT))), dim3(NT), 0, s, z, idx, p, rows, K,
                     V, Vp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n8 = int64_t(rows) * (Vp / 8);
  hipLaunchKernelGGL(keep_convert_kernel, dim3(unsigned(ceil_div(n8, NT))), dim3(NT), 0, s, z, gs, rows, Vp, G);
  return hipGetLastError();
}

hipError_t launch_logits_bwd(const LogitsArgs& a, hipStream_t s) {
  const dim3 grid(logits_grid(a));
  if (a.tlog != nullptr)
    hipLaunchKernelGGL(logits_kernel<4>, grid, dim3(GT), 0, s, a);
  else
    hipLaunchKernelGGL(logits_kernel<1>, grid, dim3(GT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3(unsigned(ceil_div(a.rows, CR))), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dense_combine(const DenseCombineArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(dense_combine_kernel, dim3(unsigned(ceil_div(a.rows, CR))), dim3(NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* rowl, const float* w, int64_t N, float* loss, float* inv_wsum,
                           hipStream_t s) {
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(FT), 0, s, rowl, w, N, loss, inv_wsum);
  return hipGetLastError();
}

hipError_t launch_dh(const DhArgs& a, hipStream_t s) {
  const int64_t tiles = ceil_div(a.rows, kTile) * ceil_div(a.D, kTile);
  hipLaunchKernelGGL(dh_kernel, dim3(unsigned(tiles * a.split)), dim3(GT), 0, s, a);
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
  hipLaunchKernelGGL(dw_kernel, dim3(unsigned(tiles)), dim3(GT), 0, s, a);
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

hipError_t debug_fault_take(unsigned* bits, hipStream_t s) {
  *bits = 0;
#if KD_DEBUG_BOUNDS
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemcpyFromSymbol(bits, HIP_SYMBOL(debug_fault), sizeof(unsigned));
  if (e == hipSuccess && *bits != 0) {
    const unsigned zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(debug_fault), &zero, sizeof(unsigned));
  }
  return e;
#else
  (void)s;
  return hipSuccess;
#endif
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  hipLaunchKernelGGL(fill_f32_kernel, dim3(unsigned(ceil_div(n, NT))), dim3(NT), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace kd
