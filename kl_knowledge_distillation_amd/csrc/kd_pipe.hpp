// bf16 main loop with direct global -> LDS copies and a 3-stage pipeline (gfx950).
//
// Workgroup: 512 threads = 8 wave64 as 4 (A rows) x 2 (B rows). Output tile
// BM x BN (A rows x B rows), each wave TM x TN = (BM/4) x (BN/2), made of 32x32
// blocks of v_mfma_f32_32x32x16_bf16. One K step moves 32 bf16 (64 bytes) of
// every operand row.
//
// Copies. global_load_lds_dwordx4 writes lane l's 16 bytes at LDS base + 16 l,
// whatever the source address, so a wave fills 1 KB of LDS per instruction and
// never touches a VGPR. An operand tile is stored as rows of 64 bytes (4 chunks
// of 16 bytes); one copy instruction fills 16 whole rows, so each row's 64
// bytes come from one contiguous global segment. The chunk index is XOR-
// swizzled by swz(r) = (r >> 2) & 3: the lane that owns LDS slot (row, p)
// fetches logical chunk p ^ swz(row). On gfx950 the fragment reads (32 rows,
// one 16-byte chunk each, ds_read_b128) are then free of bank conflicts; the
// swizzles measured for this were 4-way (r & 3), 2-way (several others) or
// conflict-free (this one among them). A fragment-native layout (32 rows x 32
// bytes per copy) is conflict-free too but doubles the cache lines each copy
// touches, and measured slower.

// Ragged edges. A row past the operand's end is clamped to its last row: the
// duplicated values feed only output rows/columns the callers mask out. The K
// extent must be a multiple of 32 (checked on the host).
//
// Pipeline. Stages s = 0, 1 are issued up front; iteration kt waits until its
// own stage has landed (vmcnt counts this thread's copies, a barrier makes all
// threads' copies visible), issues stage kt + 2 into the buffer iteration
// kt - 1 just finished with, and runs the MFMAs of stage kt.
#pragma once

#include "kd_device.hpp"

namespace kd {

constexpr int kPipeBK = 32;  // bf16 elements per K step

__device__ __forceinline__ int pipe_swz(int r) { return (r >> 2) & 3; }

// Workgroup barrier without the implicit wait for every outstanding memory
// operation that __syncthreads() carries: the pipeline has already waited for
// exactly the copies it needs. The empty asm statements keep the compiler from
// moving LDS accesses across the barrier.
__device__ __forceinline__ void pipe_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // gfx9 s_waitcnt: vmcnt in bits [3:0] and [15:14]; expcnt (7) and lgkmcnt (15) left open.
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// A K-contiguous bf16 operand: element (row, k) at ptr[row * ld + k], rows < `rows`.
struct PipeOperand {
  const bf16_t* ptr;
  int64_t ld;
  int64_t rows;
};

// Tile configuration: BM x BN output tile, NB B operands sharing the A tile,
// WM x 2 waves, S pipeline stages; AKC / BKC: whether A / B are K-contiguous
// (else row-contiguous, see pipe_copy_mn).
template <int BM, int BN, int NB, int WM = 4, int S = 3, bool AKC = true, bool BKC = true>
struct PipeCfg {
  static constexpr int WN = 2;
  static constexpr bool kAKC = AKC, kBKC = BKC;
  static constexpr int kWaves = WM * WN, kThreads = 64 * kWaves, kStages = S;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int MBLK = TM / 32, NBLK = TN / 32;
  static constexpr int kABytes = BM * 64, kBBytes = BN * 64;
  static constexpr int kStageBytes = kABytes + NB * kBBytes;
  static constexpr int kLdsBytes = S * kStageBytes;
  // copy instructions per thread per stage: R rows / 16 rows per instruction / waves
  static constexpr int kCopiesA = BM / (16 * kWaves), kCopiesB = BN / (16 * kWaves);
  static constexpr int kCopies = kCopiesA + NB * kCopiesB;
  static_assert(BM % (16 * kWaves) == 0 && BN % (16 * kWaves) == 0, "copies must split evenly");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 blocks");
  static_assert(S >= 2 && kCopies * (S - 2) < 64, "pipeline depth");
};

// Issue the copies of one R-row operand tile for K step k0 into `dst`.
template <int R, int NWAVES>
__device__ __forceinline__ void pipe_copy(const PipeOperand& op, int64_t row0, int64_t k0,
                                          uint8_t* dst, int lane, int w) {
  constexpr int kPerWave = R / (16 * NWAVES);
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int inst = w * kPerWave + j;           // 16 rows per instruction
    const int row = inst * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ pipe_swz(row);
    int64_t grow = row0 + row;
    grow = grow < op.rows ? grow : op.rows - 1;
    const bf16_t* src = op.ptr + grow * op.ld + k0 + chunk * 8;
    __builtin_amdgcn_global_load_lds(
        (const void*)src, (__attribute__((address_space(3))) void*)(dst + inst * 1024), 16, 0, 0);
  }
}

// A row-contiguous bf16 operand: element (row, k) at ptr[k * ld + row]; rows < `rows`
// (a multiple of 8), k-rows < `kdim`. A k-row past `kdim` is clamped to the last
// one, so the other operand must be zero there (callers guarantee it).
struct PipeOperandMN {
  const bf16_t* ptr;
  int64_t ld;
  int64_t rows;
  int64_t kdim;
};

// Row-contiguous tile image: 32 k-rows of R bf16 each (2R bytes per k-row), the
// 16-byte chunk index XOR-ed with (k & 3) << 2. Copies move whole k-row segments
// (R/8 lanes per k-row, fully coalesced); fragments are read with
// ds_read_b64_tr_b16, which returns lane i of each 16-lane group the 4 values
// (k0 + e, m0 + i), e = 0..3, when lane 4e + q reads 8 bytes at (k0 + e, m0 + 4q).
// With the swizzle, the 4 k-rows a half-wave reads land in distinct bank quarters.
template <int R>
__device__ __forceinline__ int mn_offset(int k, int m) {
  return k * (2 * R) + (((m >> 3) ^ ((k & 3) << 2)) << 4) + 2 * (m & 7);
}

template <int R, int NWAVES>
__device__ __forceinline__ void pipe_copy_mn(const PipeOperandMN& op, int64_t row0, int64_t k0,
                                             uint8_t* dst, int lane, int w) {
  static_assert(R >= 128 && R % 128 == 0, "row-contiguous tiles are 128 or 256 wide");
  constexpr int kCpr = R / 8;               // 16-byte chunks per k-row
  constexpr int kRowsPerInst = 64 / kCpr;   // k-rows per copy instruction
  constexpr int kPerWave = R / (16 * NWAVES);
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int inst = w * kPerWave + j;
    const int krow = inst * kRowsPerInst + lane / kCpr;
    const int chunk = (lane % kCpr) ^ ((krow & 3) << 2);
    int64_t k = k0 + krow;
    k = k < op.kdim ? k : op.kdim - 1;
    int64_t m = row0 + chunk * 8;
    m = m < op.rows ? m : op.rows - 8;
    const bf16_t* src = op.ptr + k * op.ld + m;
    __builtin_amdgcn_global_load_lds(
        (const void*)src, (__attribute__((address_space(3))) void*)(dst + inst * 1024), 16, 0, 0);
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16 through inline asm: issued this way the compiler does not
// add a wait for every in-flight LDS copy in front of it (it cannot tell the
// intrinsic form apart from the slots those copies fill). Its results are only
// ready after an lgkmcnt wait, which the main loop issues explicitly before the
// fragments are used.
__device__ __forceinline__ uint2 lds_read_tr16(const uint8_t* p) {
  uint2 v;
  const uint32_t addr = (uint32_t)(uintptr_t)p;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}

// Fragment of rows [m0, m0 + 32) at k16 step kk from a row-contiguous tile.
template <int R>
__device__ __forceinline__ bf16x8 mn_frag(const uint8_t* tile, int m0, int kk, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int m = m0 + 16 * (g & 1) + 4 * (i & 3);
  const int kb = 16 * kk + 8 * (g >> 1) + (i >> 2);
  const uint2 lo = lds_read_tr16(tile + mn_offset<R>(kb, m));
  const uint2 hi = lds_read_tr16(tile + mn_offset<R>(kb + 4, m));
  return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// K-contiguous fragment of rows [row0, row0 + 32) at k16 step kk.
__device__ __forceinline__ bf16x8 kc_frag(const uint8_t* tile, int row0, int kk, int lane) {
  const int row = row0 + (lane & 31);
  const int c = 2 * kk + (lane >> 5);
  return *reinterpret_cast<const bf16x8*>(tile + row * 64 + ((c ^ pipe_swz(row)) << 4));
}

// The A-group (waves 0..3) copies the A tile, the B-group (waves 4..7) the B tiles.
template <class C, class OA>
__device__ __forceinline__ void pipe_issue_a(const OA& A, int64_t a_row0, int64_t k0, uint8_t* stage,
                                             int lane, int gw) {
  if constexpr (C::kAKC) pipe_copy<C::kABytes / 64, 4>(A, a_row0, k0, stage, lane, gw);
  else pipe_copy_mn<C::kABytes / 64, 4>(A, a_row0, k0, stage, lane, gw);
}
template <class C, int NB, class OB>
__device__ __forceinline__ void pipe_issue_b(const OB* B, int64_t b_row0, int64_t k0, uint8_t* stage,
                                             int lane, int gw) {
#pragma unroll
  for (int g = 0; g < NB; ++g) {
    uint8_t* dst = stage + C::kABytes + g * C::kBBytes;
    if constexpr (C::kBKC) pipe_copy<C::kBBytes / 64, 4>(B[g], b_row0, k0, dst, lane, gw);
    else pipe_copy_mn<C::kBBytes / 64, 4>(B[g], b_row0, k0, dst, lane, gw);
  }
}

// Fragments of one K step (both 16-wide halves) for this wave's sub-tile.
template <class C, int NB>
struct PipeFrags {
  bf16x8 a[2][C::MBLK];
  bf16x8 b[2][NB][C::NBLK];
};

template <class C, int NB>
__device__ __forceinline__ void pipe_read(const uint8_t* stage, PipeFrags<C, NB>& f, int wm, int wn,
                                          int lane) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int mb = 0; mb < C::MBLK; ++mb) {
      const int row0 = wm * C::TM + mb * 32;
      if constexpr (C::kAKC) f.a[kk][mb] = kc_frag(stage, row0, kk, lane);
      else f.a[kk][mb] = mn_frag<C::kABytes / 64>(stage, row0, kk, lane);
    }
#pragma unroll
    for (int g = 0; g < NB; ++g)
#pragma unroll
      for (int nb = 0; nb < C::NBLK; ++nb) {
        const uint8_t* tile = stage + C::kABytes + g * C::kBBytes;
        const int row0 = wn * C::TN + nb * 32;
        if constexpr (C::kBKC) f.b[kk][g][nb] = kc_frag(tile, row0, kk, lane);
        else f.b[kk][g][nb] = mn_frag<C::kBBytes / 64>(tile, row0, kk, lane);
      }
  }
}

template <class C, int NB>
__device__ __forceinline__ void pipe_mma(const PipeFrags<C, NB>& f, f32x16 (&acc)[NB][C::MBLK][C::NBLK]) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int g = 0; g < NB; ++g)
#pragma unroll
      for (int mb = 0; mb < C::MBLK; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::NBLK; ++nb)
          acc[g][mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[kk][mb], f.b[kk][g][nb],
                                                                   acc[g][mb][nb], 0, 0, 0);
}

// Wait until at most `n` copy instructions of this thread are still in flight.
template <int PER, int MAXN>
__device__ __forceinline__ void wait_stages(int n) {
  if constexpr (MAXN >= 3) { if (n >= 3) { wait_vmcnt<3 * PER>(); return; } }
  if constexpr (MAXN >= 2) { if (n == 2) { wait_vmcnt<2 * PER>(); return; } }
  if constexpr (MAXN >= 1) { if (n == 1) { wait_vmcnt<PER>(); return; } }
  wait_vmcnt<0>();
}

// acc[g] = A[a_row0 : +BM, 0:K] * B[g][b_row0 : +BN, 0:K]^T, K a multiple of 32.
//
// Ping-pong schedule. Waves 0..3 (group A, one per SIMD) and waves 4..7
// (group B) run half an iteration apart, with two barriers per K step:
//
//   part 1:  A: MFMAs of step i           B: read fragments of step i,
//                                            copy B tiles of step i+S-1
//   barrier 1 (step i+1 visible: every wave first waits for its own copies)
//   part 2:  A: read fragments of step i+1 B: MFMAs of step i
//               copy A tile of step i+S-1
//   barrier 2
//
// While one group's wave issues MFMAs, the other group's wave on the same SIMD
// does its LDS reads and copies, so the matrix pipe does not drain at the
// barriers. Slot reuse: step i+S-1 goes into the slot of step i-1, whose reads
// finished before barrier 1 of step i-1 (group B waits for its reads before
// that barrier; group A's were consumed by its MFMAs of step i-1).
// Ends with a full barrier, so the caller may reuse `lds` right after.
template <class C, int NB, class OA, class OB>
__device__ __forceinline__ void pipe_mainloop(const OA& A, const OB* B, int64_t a_row0, int64_t b_row0,
                                              int64_t K, uint8_t* lds,
                                              f32x16 (&acc)[NB][C::MBLK][C::NBLK], int tid) {
  constexpr int S = C::kStages;
  static_assert(S >= 3, "the ping-pong schedule needs at least 3 slots");
  static_assert(C::kWaves == 8, "two groups of four waves");
  constexpr int kCopiesA = C::kABytes / 1024 / 4;        // per A-group wave per step
  constexpr int kCopiesB = NB * C::kBBytes / 1024 / 4;   // per B-group wave per step
  // The wave index is the same for all lanes of a wave; readfirstlane makes that
  // visible to the compiler, so the group branches below are scalar branches.
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;
  const bool grp_b = w >= 4;
  const int gw = w & 3;
#pragma unroll
  for (int g = 0; g < NB; ++g)
#pragma unroll
    for (int mb = 0; mb < C::MBLK; ++mb)
#pragma unroll
      for (int nb = 0; nb < C::NBLK; ++nb)
#pragma unroll
        for (int x = 0; x < 16; ++x) acc[g][mb][nb][x] = 0.f;

  const int nk = (int)(K / kPipeBK);
  // Prologue: steps 0 .. S-2, each group its own operand.
#pragma unroll
  for (int st = 0; st < S - 1; ++st)
    if (st < nk) {
      uint8_t* slot = lds + st * C::kStageBytes;
      if (grp_b) pipe_issue_b<C, NB, OB>(B, b_row0, (int64_t)st * kPipeBK, slot, lane, gw);
      else pipe_issue_a<C, OA>(A, a_row0, (int64_t)st * kPipeBK, slot, lane, gw);
    }
  // Step 0 visible: at most steps 1 .. min(S-2, nk-1) still in flight.
  {
    const int later = min(S - 2, nk - 1);
    if (grp_b) wait_stages<kCopiesB, S - 2>(later);
    else wait_stages<kCopiesA, S - 2>(later);
  }
  pipe_barrier();
  PipeFrags<C, NB> f;
  if (!grp_b) {
    // Group A: MFMAs in part 1, reads and A-tile copies in part 2.
    pipe_read<C, NB>(lds, f, wm, wn, lane);
    int cur = 0;  // slot of step i
    for (int i = 0; i < nk; ++i) {
      const int nxt = (cur + 1 == S) ? 0 : cur + 1;     // slot of step i+1
      const int fill = (cur == 0) ? S - 1 : cur - 1;    // slot of step i+S-1
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // fragments of step i ready
      __builtin_amdgcn_s_setprio(1);
      pipe_mma<C, NB>(f, acc);
      __builtin_amdgcn_s_setprio(0);
      // step i+1 must have landed; steps i+2 .. i+S-2 may stay in flight
      wait_stages<kCopiesA, S - 2>(max(0, min(S - 3, nk - 2 - i)));
      pipe_barrier();
      if (i + 1 < nk) pipe_read<C, NB>(lds + nxt * C::kStageBytes, f, wm, wn, lane);
      if (i + S - 1 < nk)
        pipe_issue_a<C, OA>(A, a_row0, (int64_t)(i + S - 1) * kPipeBK, lds + fill * C::kStageBytes,
                            lane, gw);
      pipe_barrier();
      cur = nxt;
    }
  } else {
    // Group B: reads and B-tile copies in part 1, MFMAs in part 2.
    int cur = 0;
    for (int i = 0; i < nk; ++i) {
      const int nxt = (cur + 1 == S) ? 0 : cur + 1;
      const int fill = (cur == 0) ? S - 1 : cur - 1;
      pipe_read<C, NB>(lds + cur * C::kStageBytes, f, wm, wn, lane);
      if (i + S - 1 < nk)
        pipe_issue_b<C, NB, OB>(B, b_row0, (int64_t)(i + S - 1) * kPipeBK, lds + fill * C::kStageBytes,
                                lane, gw);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads of slot `cur` done
      // step i+1 must have landed; steps i+2 .. i+S-1 may stay in flight
      wait_stages<kCopiesB, S - 2>(max(0, min(S - 2, nk - 2 - i)));
      pipe_barrier();
      __builtin_amdgcn_s_setprio(1);
      pipe_mma<C, NB>(f, acc);
      __builtin_amdgcn_s_setprio(0);
      pipe_barrier();
      cur = nxt;
    }
  }
  __syncthreads();
}

// Row of the BM-row tile held by accumulator register x of block mb (wave row wm).
template <int TM>
__device__ __forceinline__ int pipe_row(int wm, int mb, int x, int lane) {
  return wm * TM + mb * 32 + 8 * (x >> 2) + 4 * (lane >> 5) + (x & 3);
}
template <int TN>
__device__ __forceinline__ int pipe_col(int wn, int nb, int lane) { return wn * TN + nb * 32 + (lane & 31); }

}  // namespace kd
