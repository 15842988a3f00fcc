// bf16 main loop with buffer loads straight into LDS (three A-operand slots,
// two or four B-operand slots), ping-pong scheduling and
// v_mfma_f32_16x16x32_bf16 (gfx950).
//
// Workgroup: 512 threads = 8 wave64 as 4 (A rows) x 2 (B rows). Output tile
// BM x BN (A rows x B rows); each wave owns TM x TN = (BM/4) x (BN/2), made of
// 16x16 blocks. One K step moves 64 bf16 (128 bytes, one cache line) of every
// operand row.
//
// Output layout of the 16x16x32 MFMA: lane l holds column l % 16 and rows
// 4 (l / 16) + r, r in [0, 4), of its block. The A fragment of lane l is row
// l % 16 with 8 k values; the B fragment is column l % 16 with the same 8 k
// values (any k order shared by both operands gives the same sum).
//
// Why this shape. With random bf16 operands the chip is power limited well
// below its nominal MFMA peak, and the 16x16x32 form sustains a higher clock
// than 32x32x16 for the same work. Moving a full 128-byte line per row and step
// halves the cache-line traffic per byte against 64-byte row segments.
//
// Copies. buffer_load_dwordx4 ... lds writes lane l's 16 bytes at LDS base +
// 16 l and never touches a VGPR; a wave fills 1 KB per instruction. The buffer
// descriptor bounds every copy: a lane past the end of the operand reads zero,
// so ragged tiles need no clamping and padded rows / k-rows hold zeros. The
// wave-uniform part of each address (row block, K offset) goes into soffset,
// so all copies of an operand share one or two offset VGPRs.
//
// K-contiguous tiles are rows of 128 bytes (8 chunks of 16 bytes); one copy
// fills 8 whole rows, each from one cache line. Chunk c of row r sits at
// position c ^ swz(r), swz(r) = (r >> 1) & 7: the 16 rows a fragment read
// touches at one chunk then fall in 16 distinct 16-byte bank groups.
//
// Row-contiguous tiles (the dW / dH operands) are 64 k-rows of R bf16; their
// fragments are read with ds_read_b64_tr_b16 (see mn_offset).
//
// Schedule. Waves 0..3 (group A) and 4..7 (group B), one of each per SIMD, run
// half a step apart:
//   part 1:  A: MFMAs of step i, copying    B: read fragments of step i
//               the A operand of step i+2
//   barrier 1 (step i+1 has landed: each group waited for its own copies)
//   part 2:  A: read fragments of step i+1  B: MFMAs of step i, copying the
//                                              B operands of step i+SB
//   barrier 2
// While one wave of a SIMD issues MFMAs the other does its LDS reads, so the
// matrix pipe keeps running across the barriers. The copies are spread over
// both parts, each half of them between one group's MFMAs; bunched in one
// part they stall the MFMAs behind them. (The copies set the loop's pace, but
// not by the rate a CU can be served: with every copy hitting L2 the loop is
// only a few percent faster.) Step s has its A operand in
// A-slot s % 3 and its B operands in B-slot s % SB (SB = 4 where the LDS holds
// four, one 128-row B operand; else 2); the A-slot of step i-1 and the B-slot
// of step i are free after barrier 1 of those steps.
#pragma once

#include "kd_device.hpp"

namespace kd {

constexpr int kPipeBK = 64;  // bf16 elements per K step

__device__ __forceinline__ int pipe_swz(int r) { return (r >> 1) & 7; }

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

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer descriptor over [base, base + bytes); sizes of 4 GiB and more are
// cut to 4 GiB - 1 (every offset a tile uses stays far below it).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0xffffffffll ? 0xffffffffu : (uint32_t)bytes);
  // dword 3: 32-bit data format, the setting raw buffer loads use on gfx9.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

// 16 bytes per lane from descriptor r at voff + soff into dst + 16 lane; lanes
// whose offset falls outside the descriptor write zeros.
__device__ __forceinline__ void buffer_copy(rsrc_t r, uint8_t* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff,
                                           soff, 0, 0);
}

// A K-contiguous bf16 operand: element (row, k) at ptr[row * ld + k], rows < `rows`.
struct PipeOperand {
  const bf16_t* ptr;
  int64_t ld;
  int64_t rows;
};

// A row-contiguous bf16 operand: element (row, k) at ptr[k * ld + row], k < `kdim`.
// Rows past `rows` read neighbouring (finite) data or zeros; they only feed
// outputs the callers drop.
struct PipeOperandMN {
  const bf16_t* ptr;
  int64_t ld;
  int64_t rows;
  int64_t kdim;
};

// Row-contiguous tile image: 64 k-rows of R bf16 each (2R bytes per k-row), the
// 16-byte chunk index XOR-ed with mn_swz(k). Fragments are read with
// ds_read_b64_tr_b16: in each 16-lane group, lane 4e + q reads 8 bytes at
// (k0 + e, m0 + 4q) and lane i receives the 4 values (k0 + e, m0 + i), e = 0..3.
// Lane groups 0 and 1 (served together) read k-rows k0 + e and k0 + 8 + e: bits
// 2-3 of the swizzle spread the four k-rows of a group over distinct banks, bit
// 1 (from k-row bit 3) separates the two groups.
__device__ __forceinline__ int mn_swz(int k) { return ((k & 3) << 2) | (((k >> 3) & 1) << 1); }
template <int R>
__device__ __forceinline__ int mn_offset(int k, int m) {
  return k * (2 * R) + (((m >> 3) ^ mn_swz(k)) << 4) + 2 * (m & 7);
}

// Copy source of one operand tile. issue(k0, dst, local) moves 1 KB block
// `local` of the tile for the K step starting at k0 into dst + 1024 local.
template <bool KC, int R>
struct TileSrc;

// K-contiguous: block `local` is rows 8 local .. 8 local + 7.
template <int R>
struct TileSrc<true, R> {
  rsrc_t rsrc;
  uint32_t voff[2];  // lane offset for even / odd blocks (the swizzle depends on row bit 3)
  uint32_t stride;   // bytes per row

  __device__ __forceinline__ void init(const PipeOperand& op, int64_t row0, int lane) {
    rsrc = make_rsrc(op.ptr + row0 * op.ld, (op.rows - row0) * op.ld * 2);
    stride = (uint32_t)(op.ld * 2);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int row = p * 8 + (lane >> 3);  // row within a pair of blocks
      const int chunk = (lane & 7) ^ pipe_swz(row);
      voff[p] = (uint32_t)(lane >> 3) * stride + (uint32_t)chunk * 16u;
    }
  }
  __device__ __forceinline__ void issue(int64_t k0, uint8_t* dst, int local) const {
    const uint32_t soff = (uint32_t)local * 8u * stride + (uint32_t)(k0 * 2);
    buffer_copy(rsrc, dst + local * 1024, voff[local & 1], soff);
  }
};

// Row-contiguous: block `local` is k-rows kKpi local .. kKpi (local + 1) - 1.
template <int R>
struct TileSrc<false, R> {
  static_assert(R == 128 || R == 256, "row-contiguous tiles are 128 or 256 wide");
  static constexpr int kCpr = R / 8;      // 16-byte chunks per k-row
  static constexpr int kKpi = 64 / kCpr;  // k-rows per block (4 or 2)
  const bf16_t* base;                     // element (row0, k = 0)
  int64_t ld, kdim, row0;
  // lane offsets by the swizzle-relevant bits of the block's first k-row
  // (bit 1 and bit 3; k-rows within a block only differ below those)
  uint32_t voff[4];

  __device__ __forceinline__ static int variant(int local) {
    const int k = local * kKpi;
    return ((k >> 1) & 1) | (((k >> 3) & 1) << 1);
  }
  __device__ __forceinline__ void init(const PipeOperandMN& op, int64_t r0, int lane) {
    base = op.ptr + r0;
    ld = op.ld;
    kdim = op.kdim;
    row0 = r0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int kr = lane / kCpr;                      // k-row within the block
      const int k = ((v & 1) << 1) + ((v >> 1) << 3) + kr;
      const int chunk = (lane % kCpr) ^ mn_swz(k);
      voff[v] = (uint32_t)kr * (uint32_t)(ld * 2) + (uint32_t)chunk * 16u;
    }
  }
  __device__ __forceinline__ void issue(int64_t k0, uint8_t* dst, int local) const {
    // descriptor from k-row k0 on, so offsets stay small whatever K * ld is
    const rsrc_t r = make_rsrc(base + k0 * ld, ((kdim - k0) * ld - row0) * 2);
    const uint32_t soff = (uint32_t)(local * kKpi) * (uint32_t)(ld * 2);
    buffer_copy(r, dst + local * 1024, voff[variant(local)], soff);
  }
};

// Tile configuration: BM x BN output tile, NB B operands sharing the A tile;
// AKC / BKC: whether A / B are K-contiguous.
template <int BM, int BN, int NB, bool AKC = true, bool BKC = true>
struct PipeCfg {
  static constexpr int WM = 4, WN = 2;
  static constexpr bool kAKC = AKC, kBKC = BKC;
  static constexpr int kWaves = WM * WN, kThreads = 64 * kWaves;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int MB = TM / 16, NBK = TN / 16;
  static constexpr int kABytes = BM * 128, kBBytes = BN * 128;
  // LDS: three A-operand slots, then slots of the NB B operands: four where
  // the rest of the LDS holds them (one 128-row B operand), else two
  static constexpr int kBFit = (160 * 1024 - 3 * kABytes) / (NB * kBBytes);
  static constexpr int kBSlots = kBFit >= 4 ? 4 : 2;
  static constexpr int kBBase = 3 * kABytes;
  static constexpr int kLdsBytes = 3 * kABytes + kBSlots * NB * kBBytes;
  // copy instructions per wave and step: group A copies the A operand, group
  // B the B operands, a quarter each per wave
  static constexpr int kAPer = kABytes / 1024 / 4, kBPer = kBBytes / 1024 / 4;
  static constexpr int kACopies = kAPer, kBCopies = NB * kBPer;
  static constexpr int kMfma = 2 * NB * MB * NBK;  // per wave per step
  static_assert(BM % 256 == 0 && BN % 128 == 0, "copies must split evenly over 4 waves");
  static_assert(kACopies <= kMfma && kBCopies <= kMfma, "copies must fit between the MFMAs");
  static_assert(kACopies < 32 && kBCopies < 32, "vmcnt range");
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
};

// K-contiguous fragment of rows [row0, row0 + 16) at k32 step kk.
__device__ __forceinline__ bf16x8 kc_frag(const uint8_t* tile, int row0, int kk, int lane) {
  const int row = row0 + (lane & 15);
  const int c = 4 * kk + (lane >> 4);
  return *reinterpret_cast<const bf16x8*>(tile + row * 128 + ((c ^ pipe_swz(row)) << 4));
}

// ds_read_b64_tr_b16 through inline asm: issued this way the compiler does not
// add a wait for every in-flight LDS copy in front of it (it cannot tell the
// intrinsic form apart from the slots those copies fill). Its results are only
// ready after an lgkmcnt wait, which the main loop issues explicitly, and
// pipe_frags_ready ties every use to that wait.
__device__ __forceinline__ uint2 lds_read_tr16(const uint8_t* p) {
  uint2 v;
  const uint32_t addr = (uint32_t)(uintptr_t)p;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}

// Per-lane part of the transposed-read addresses of NF fragments of rows
// [m_first + 16 f, m_first + 16 f + 16), f = 0 .. NF-1, at k32 step 0 of a
// tile. Lane l = 16 g + 4 e + q reads k-row 8 g + e and rows m + 4 q; its
// swizzle mn_swz(8 g + e) does not change with the k32 step (32 kk) or the
// second half (+4), which only add a constant. Keeping one base per fragment
// (instead of every final address) keeps the register count down.
template <int R, int NF>
struct MnLane {
  uint32_t base[NF];
  __device__ __forceinline__ void init(int m_first, int lane) {
    const int g = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
    const int k = 8 * g + e;
#pragma unroll
    for (int f = 0; f < NF; ++f) base[f] = (uint32_t)mn_offset<R>(k, m_first + 16 * f + 4 * q);
  }
};

// Row-contiguous fragment f at k32 step kk: lane l gets row l % 16 at
// k = 32 kk + 8 (l / 16) + e, e = 0..7 (the K-contiguous order).
template <int R, int NF>
__device__ __forceinline__ bf16x8 mn_frag(const uint8_t* tile, const MnLane<R, NF>& ml, int f, int kk) {
  const uint8_t* p = tile + ml.base[f] + kk * 32 * (2 * R);
  const uint2 lo = lds_read_tr16(p);
  const uint2 hi = lds_read_tr16(p + 4 * (2 * R));
  return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Fragments of one K step (two k32 halves) for this wave's sub-tile.
template <class C, int NB>
struct PipeFrags {
  bf16x8 a[2][C::MB];
  bf16x8 b[2][NB][C::NBK];
};

// Waits for this wave's LDS reads, then makes every fragment register that a
// transposed read (inline asm, whose latency the compiler does not see) filled
// the result of an asm statement placed after the wait. Volatile asm keeps its
// order, so no MFMA using such a fragment can be scheduled above the wait; the
// compiler itself waits for the K-contiguous fragments (ordinary LDS loads).
template <class C, int NB>
__device__ __forceinline__ void pipe_frags_ready(PipeFrags<C, NB>& f) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if constexpr (!C::kAKC) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) asm volatile("" : "+v"(f.a[kk][mb]));
  }
  if constexpr (!C::kBKC) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int g = 0; g < NB; ++g)
#pragma unroll
        for (int nb = 0; nb < C::NBK; ++nb) asm volatile("" : "+v"(f.b[kk][g][nb]));
  }
}

// Transposed-read lane bases of this wave's A and B fragments (unused for
// K-contiguous operands).
template <class C>
struct PipeLanes {
  MnLane<C::kABytes / 128, C::MB> a;
  MnLane<C::kBBytes / 128, C::NBK> b;
  __device__ __forceinline__ void init(int wm, int wn, int lane) {
    if constexpr (!C::kAKC) a.init(wm * C::TM, lane);
    if constexpr (!C::kBKC) b.init(wn * C::TN, lane);
  }
};

// Fragments of one K step from its A-operand slot and its B-operand slot (the
// NB B operands one after another).
template <class C, int NB>
__device__ __forceinline__ void pipe_read(const uint8_t* aslot, const uint8_t* bslot, PipeFrags<C, NB>& f,
                                          const PipeLanes<C>& pl, int wm, int wn, int lane) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      if constexpr (C::kAKC) f.a[kk][mb] = kc_frag(aslot, wm * C::TM + mb * 16, kk, lane);
      else f.a[kk][mb] = mn_frag(aslot, pl.a, mb, kk);
    }
#pragma unroll
    for (int g = 0; g < NB; ++g)
#pragma unroll
      for (int nb = 0; nb < C::NBK; ++nb) {
        const uint8_t* tile = bslot + g * C::kBBytes;
        if constexpr (C::kBKC) f.b[kk][g][nb] = kc_frag(tile, wn * C::TN + nb * 16, kk, lane);
        else f.b[kk][g][nb] = mn_frag(tile, pl.b, nb, kk);
      }
  }
}

template <class C, int NB>
__device__ __forceinline__ void pipe_mma(const PipeFrags<C, NB>& f, f32x4 (&acc)[NB][C::MB][C::NBK]) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int g = 0; g < NB; ++g)
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::NBK; ++nb)
          acc[g][mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[kk][mb], f.b[kk][g][nb],
                                                                   acc[g][mb][nb], 0, 0, 0);
}

// The same MFMAs with copy(j), j = 0 .. N-1, spread evenly: copy j after MFMA
// IL (j + 1) - 1, IL = kMfma / N (sched_group_barrier keeps the interleave).
// With 256-row operands IL is 8: four waves each issuing 1 KB per 8 MFMAs (16
// cycles each) ask for ~32 B/clk per CU, about half of what the L2 delivers to
// a CU; issued faster, copies queue and stall the MFMAs behind them.
template <class C, int NB, int N, class F>
__device__ __forceinline__ void pipe_mma_copies(const PipeFrags<C, NB>& f,
                                                f32x4 (&acc)[NB][C::MB][C::NBK], F&& copy) {
  constexpr int IL = C::kMfma / N;
  static_assert(IL >= 1 && N * IL <= C::kMfma, "copies fit between the MFMAs");
  int m = 0;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int g = 0; g < NB; ++g)
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::NBK; ++nb) {
          acc[g][mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[kk][mb], f.b[kk][g][nb],
                                                                   acc[g][mb][nb], 0, 0, 0);
          if (m % IL == IL - 1 && m / IL < N) copy(m / IL);
          ++m;
        }
#pragma unroll
  for (int j = 0; j < N; ++j) {
    __builtin_amdgcn_sched_group_barrier(0x008, IL, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
  }
  if constexpr (C::kMfma - N * IL > 0) __builtin_amdgcn_sched_group_barrier(0x008, C::kMfma - N * IL, 0);
}

// acc[g] = A[a_row0 : +BM, 0:K] * B[g][b_row0 : +BN, 0:K]^T, K a multiple of 64.
// Ends with a full barrier, so the caller may reuse `lds` right after.
//
// Step s (64 of K) has its A operand in A-slot s % 3 and its B operands in
// B-slot s % SB (SB = C::kBSlots, 2 or 4). Group A (waves 0-3) runs its MFMAs
// of step i while group B reads its fragments of step i; after barrier 1 group
// B runs its MFMAs while group A reads step i+1; barrier 2 ends the step. Each
// group copies its own operand between its own MFMAs of step i: group A the A
// operand of step i+2 into the A-slot of step i-1 (both groups read it before
// barrier 1 of step i-1), group B the B operands of step i+SB into the B-slot
// of step i (read before barrier 1 of step i). The A operand so leads by
// 1.5-2 steps, the B operands by SB-1. Each group waits for its own copies of
// step i+1 before barrier 1 of step i.
template <class C, int NB, class OA, class OB>
__device__ __forceinline__ void pipe_mainloop(const OA& A, const OB* B, int64_t a_row0, int64_t b_row0,
                                              int64_t K, uint8_t* lds,
                                              f32x4 (&acc)[NB][C::MB][C::NBK], int tid) {
  static_assert(C::kWaves == 8, "two groups of four waves");
  static_assert(NB == 1 || NB == 2, "one or two B operands (copy_b picks between the first and the last)");
  static_assert(C::kBSlots == 2 || C::kBSlots == 4, "B-slot index by mask; the tail's waits cover up to four");
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
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < C::NBK; ++nb)
#pragma unroll
        for (int x = 0; x < 4; ++x) acc[g][mb][nb][x] = 0.f;

  const int nk = (int)(K / kPipeBK);
  PipeFrags<C, NB> f;
  PipeLanes<C> pl;
  pl.init(wm, wn, lane);
  auto aslot = [&](int st) { return lds + (st % 3) * C::kABytes; };
  constexpr int SB = C::kBSlots;
  auto bslot = [&](int st) { return lds + C::kBBase + (st & (SB - 1)) * (NB * C::kBBytes); };
  constexpr int kNA = C::kACopies, kNB = C::kBCopies;
  // (copy-and-MFMA steps and the last two steps are separate loops: one loop
  // with a branch between the two MFMA bodies made the compiler spill)
  if (!grp_b) {
    TileSrc<C::kAKC, C::kABytes / 128> sa;
    sa.init(A, a_row0, lane);
    auto copy_a = [&](int st, int j) { sa.issue((int64_t)st * kPipeBK, aslot(st), gw * kNA + j); };
    // Prologue: the A operand of steps 0 and 1; step 0 visible at the first barrier.
#pragma unroll
    for (int j = 0; j < kNA; ++j) copy_a(0, j);
    if (nk > 1) {
#pragma unroll
      for (int j = 0; j < kNA; ++j) copy_a(1, j);
      wait_vmcnt<kNA>();
    } else {
      wait_vmcnt<0>();
    }
    pipe_barrier();
    pipe_read<C, NB>(aslot(0), bslot(0), f, pl, wm, wn, lane);
    int i = 0;
    for (; i + 2 < nk; ++i) {
      pipe_frags_ready<C, NB>(f);  // fragments of step i ready
      __builtin_amdgcn_s_setprio(1);
      pipe_mma_copies<C, NB, kNA>(f, acc, [&](int j) { copy_a(i + 2, j); });
      __builtin_amdgcn_s_setprio(0);
      wait_vmcnt<kNA>();  // the A operand of step i+1 has landed
      pipe_barrier();     // 1
      pipe_read<C, NB>(aslot(i + 1), bslot(i + 1), f, pl, wm, wn, lane);
      pipe_barrier();  // 2
    }
    for (; i < nk; ++i) {
      pipe_frags_ready<C, NB>(f);
      __builtin_amdgcn_s_setprio(1);
      pipe_mma<C, NB>(f, acc);
      __builtin_amdgcn_s_setprio(0);
      wait_vmcnt<0>();
      pipe_barrier();  // 1
      if (i + 1 < nk) pipe_read<C, NB>(aslot(i + 1), bslot(i + 1), f, pl, wm, wn, lane);
      pipe_barrier();  // 2
    }
  } else {
    TileSrc<C::kBKC, C::kBBytes / 128> sb[NB];
#pragma unroll
    for (int g = 0; g < NB; ++g) sb[g].init(B[g], b_row0, lane);
    auto copy_b = [&](int st, int j) {
      const int g = j / C::kBPer, jj = j % C::kBPer;
      uint8_t* dst = bslot(st) + g * C::kBBytes;
      // (a branch, not an index: an indexed sb would live in scratch)
      if (g == 0) sb[0].issue((int64_t)st * kPipeBK, dst, gw * C::kBPer + jj);
      else sb[NB - 1].issue((int64_t)st * kPipeBK, dst, gw * C::kBPer + jj);
    };
    // Prologue: the B operands of steps 0 .. SB-1; step 0 visible at the first barrier.
#pragma unroll
    for (int st = 0; st < SB; ++st)
      if (st < nk) {
#pragma unroll
        for (int j = 0; j < kNB; ++j) copy_b(st, j);
      }
    if (nk >= SB) wait_vmcnt<(SB - 1) * kNB>();
    else wait_vmcnt<0>();
    pipe_barrier();
    int i = 0;
    for (; i + SB < nk; ++i) {
      pipe_read<C, NB>(aslot(i), bslot(i), f, pl, wm, wn, lane);
      pipe_frags_ready<C, NB>(f);  // reads of step i done
      wait_vmcnt<(SB - 2) * kNB>();  // the B operands of step i+1 have landed (those of i+2 .. i+SB-1 may not)
      pipe_barrier();  // 1
      __builtin_amdgcn_s_setprio(1);
      pipe_mma_copies<C, NB, kNB>(f, acc, [&](int j) { copy_b(i + SB, j); });
      __builtin_amdgcn_s_setprio(0);
      pipe_barrier();  // 2
    }
    for (; i < nk; ++i) {
      pipe_read<C, NB>(aslot(i), bslot(i), f, pl, wm, wn, lane);
      pipe_frags_ready<C, NB>(f);
      // step i+1 landed; the copies of steps i+2 .. nk-1 may still be in flight
      if constexpr (SB == 4) {
        const int later = nk - 2 - i;
        if (later >= 2) wait_vmcnt<2 * kNB>();
        else if (later == 1) wait_vmcnt<kNB>();
        else wait_vmcnt<0>();
      } else {
        wait_vmcnt<0>();
      }
      pipe_barrier();  // 1
      __builtin_amdgcn_s_setprio(1);
      pipe_mma<C, NB>(f, acc);
      __builtin_amdgcn_s_setprio(0);
      pipe_barrier();  // 2
    }
  }
  __syncthreads();
}

// Row (A side) and column (B side) within the BM x BN tile of accumulator
// register r of block (mb, nb).
template <class C>
__device__ __forceinline__ int pipe_row(int wm, int mb, int r, int lane) {
  return wm * C::TM + mb * 16 + 4 * (lane >> 4) + r;
}
template <class C>
__device__ __forceinline__ int pipe_col(int wn, int nb, int lane) {
  return wn * C::TN + nb * 16 + (lane & 15);
}

}  // namespace kd
