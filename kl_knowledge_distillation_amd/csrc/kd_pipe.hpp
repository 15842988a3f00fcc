// bf16 main loop with buffer loads straight into LDS, two slots, ping-pong
// scheduling and v_mfma_f32_16x16x32_bf16 (gfx950).
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
// Schedule (two slots). Waves 0..3 (group A) and 4..7 (group B), one of each
// per SIMD, run half a step apart:
//   part 1:  A: MFMAs of step i            B: read fragments of step i
//   barrier 1 (step i+1 has landed: group B waited for its copies)
//   part 2:  A: read fragments of step i+1 B: MFMAs of step i, issuing the
//                                             copies of step i+2 into the slot
//                                             of step i between them
//   barrier 2
// While one wave of a SIMD issues MFMAs the other does its LDS reads, so the
// matrix pipe keeps running across the barriers. The slot of step i is free at
// barrier 1: group B read it in part 1, group A in part 2 of step i-1. Copies
// of step i+2 have the rest of part 2 and part 1 of step i+1 to land.
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
  static constexpr int kStageBytes = kABytes + NB * kBBytes;
  static constexpr int kLdsBytes = 2 * kStageBytes;
  // copy instructions per group-B wave per step: A blocks first, then each B
  static constexpr int kAPer = kABytes / 1024 / 4, kBPer = kBBytes / 1024 / 4;
  static constexpr int kCopies = kAPer + NB * kBPer;
  static constexpr int kMfma = 2 * NB * MB * NBK;  // per wave per step
  // MFMAs per copy: the copies spread evenly over the whole MFMA phase. Four
  // waves each issuing 1 KB per kIL MFMAs (16 cycles each) ask for 64 B/clk
  // per CU at kIL = 4, the rate the L2 delivers to a CU; issued faster, they
  // queue and stall the MFMAs behind them.
  static constexpr int kIL = kMfma / kCopies > 0 ? kMfma / kCopies : 1;
  static_assert(BM % 256 == 0 && BN % 128 == 0, "copies must split evenly over 4 waves");
  static_assert(kCopies * kIL <= kMfma, "copies must fit between the MFMAs");
  static_assert(kCopies < 64, "vmcnt range");
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
// ready after an lgkmcnt wait, which the main loop issues explicitly before the
// fragments are used.
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

template <class C, int NB>
__device__ __forceinline__ void pipe_read(const uint8_t* stage, PipeFrags<C, NB>& f, const PipeLanes<C>& pl,
                                          int wm, int wn, int lane) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      if constexpr (C::kAKC) f.a[kk][mb] = kc_frag(stage, wm * C::TM + mb * 16, kk, lane);
      else f.a[kk][mb] = mn_frag(stage, pl.a, mb, kk);
    }
#pragma unroll
    for (int g = 0; g < NB; ++g)
#pragma unroll
      for (int nb = 0; nb < C::NBK; ++nb) {
        const uint8_t* tile = stage + C::kABytes + g * C::kBBytes;
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

// The same MFMAs with copy(j), j = 0 .. C::kCopies-1, issued after MFMA
// kIL (j + 1) - 1, in that order (sched_group_barrier keeps the interleave).
template <class C, int NB, class F>
__device__ __forceinline__ void pipe_mma_copies(const PipeFrags<C, NB>& f,
                                                f32x4 (&acc)[NB][C::MB][C::NBK], F&& copy) {
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
          if (m % C::kIL == C::kIL - 1 && m / C::kIL < C::kCopies) copy(m / C::kIL);
          ++m;
        }
#pragma unroll
  for (int j = 0; j < C::kCopies; ++j) {
    __builtin_amdgcn_sched_group_barrier(0x008, C::kIL, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);       // VMEM read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, C::kMfma - C::kCopies * C::kIL, 0);
}

// Copy j of group-B wave gw for the K step at k0 into `stage`: the wave takes a
// quarter of the A blocks, then a quarter of each B operand's blocks.
template <class C, int NB, class SA, class SB>
__device__ __forceinline__ void pipe_copy(const SA& sa, const SB (&sb)[NB], int64_t k0, uint8_t* stage,
                                          int gw, int j) {
  if (j < C::kAPer) {
    sa.issue(k0, stage, gw * C::kAPer + j);
  } else {
    const int g = (j - C::kAPer) / C::kBPer, jj = (j - C::kAPer) % C::kBPer;
    sb[g].issue(k0, stage + C::kABytes + g * C::kBBytes, gw * C::kBPer + jj);
  }
}

// Cooperative L2 prefetch of the fused tiles. The 32 tiles an XCD runs at
// once are 4 vocabulary tiles x 8 token tiles in the grouped order, so each A
// row (256 per tile) is read by 8 of them and each B row (NB x 128) by 4. Tile
// (a, b) reads, kPipeAhead K steps early, one 16-byte piece of each 128-byte
// line of its share: A rows 32 (b % 8) .. + 31 and B rows NB 32 (a % 4) ..
// + NB 32 - 1, so each line of the group comes into L2 once, before the tiles
// copy it (measured: fused kernels 3-5% faster at the quickstart shape).
#ifndef KD_PIPE_AHEAD
#define KD_PIPE_AHEAD 4
#endif
constexpr int kPipeAhead = KD_PIPE_AHEAD;
struct PipePrefetch {
  int on;         // 0: no prefetch
  int a_share;    // 0..7
  int b_share;    // 0..3
  uint8_t* dump;  // 1 KB of LDS that the prefetch reads land in (never read)
};

// Prefetch lines of a row-contiguous tile (R columns, R / 64 lines per k-row)
// read by `sharers` tiles side by side: share s takes 64 / sharers of the 64
// k-rows of every K step, half per wave (`half` 0 or 1); the other lanes repeat
// those lines. Left off (on stays false) when the operand spans 4 GiB or more,
// where the per-step offsets would not fit 32 bits.
template <int R>
__device__ __forceinline__ void mn_prefetch_lines(const TileSrc<false, R>& s, int sharers, int share, int half,
                                                  int lane, rsrc_t& r, uint32_t& voff, uint32_t& step_bytes,
                                                  bool& on) {
  constexpr int kLines = R / 64;
  const int kper = 64 / sharers / 2;  // k-rows per wave
  if (s.kdim * s.ld * 2 >= 0xffffffffll) return;
  r = make_rsrc(s.base, (s.kdim * s.ld - s.row0) * 2);
  const int kr = share * 2 * kper + half * kper + (lane / kLines) % kper;
  voff = (uint32_t)kr * (uint32_t)(s.ld * 2) + (uint32_t)(lane % kLines) * 128u;
  step_bytes = (uint32_t)(kPipeBK * s.ld * 2);
  on = true;
}

// acc[g] = A[a_row0 : +BM, 0:K] * B[g][b_row0 : +BN, 0:K]^T, K a multiple of 64.
// Ends with a full barrier, so the caller may reuse `lds` right after. With a
// prefetch share (K-contiguous operands, two B operands of 128 rows) group B
// also reads its share of the lines kPipeAhead steps ahead: one buffer read
// per wave after a batch of copies (while that step exists); a wait for the
// copies then leaves that one younger read outstanding.
template <class C, int NB, class OA, class OB>
__device__ __forceinline__ void pipe_mainloop(const OA& A, const OB* B, int64_t a_row0, int64_t b_row0,
                                              int64_t K, uint8_t* lds,
                                              f32x4 (&acc)[NB][C::MB][C::NBK], int tid,
                                              PipePrefetch pf = PipePrefetch{0, 0, 0, nullptr}) {
  static_assert(C::kWaves == 8, "two groups of four waves");
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
  if (!grp_b) {
    pipe_barrier();  // pairs with the prologue barrier of group B: step 0 visible
    pipe_read<C, NB>(lds, f, pl, wm, wn, lane);
    for (int i = 0; i < nk; ++i) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // fragments of step i ready
      __builtin_amdgcn_s_setprio(1);
      pipe_mma<C, NB>(f, acc);
      __builtin_amdgcn_s_setprio(0);
      pipe_barrier();  // 1: step i+1 has landed
      if (i + 1 < nk) pipe_read<C, NB>(lds + ((i + 1) & 1) * C::kStageBytes, f, pl, wm, wn, lane);
      pipe_barrier();  // 2
    }
  } else {
    TileSrc<C::kAKC, C::kABytes / 128> sa;
    TileSrc<C::kBKC, C::kBBytes / 128> sb[NB];
    sa.init(A, a_row0, lane);
#pragma unroll
    for (int g = 0; g < NB; ++g) sb[g].init(B[g], b_row0, lane);
    // This wave's prefetch lines: waves 0-1 take the A operand's share (read by
    // the 8 tiles along B), waves 2-3 the B operands' share (read by the 4
    // tiles along A), half each. K-contiguous rows are one line per K step;
    // row-contiguous tiles are k-rows of R / 64 lines. Lines past the operand
    // read out of range (nothing).
    bool pf_on = false;
    rsrc_t pf_r = make_rsrc(nullptr, 0);  // no records: reads nothing
    uint32_t pf_voff = 0, pf_step = kPipeBK * 2;
    constexpr int kRowsB = C::kBBytes / 128;  // rows of one B operand
    constexpr bool kPfB = C::kBKC ? (NB * kRowsB == 128 || NB * kRowsB == 256) : NB == 1;
    if constexpr (kPfB) {
      if (pf.on) {
        if (gw < 2) {
          if constexpr (C::kAKC) {
            pf_on = true;
            pf_r = sa.rsrc;
            pf_voff = (uint32_t)(pf.a_share * 32 + gw * 16 + (lane & 15)) * sa.stride;
          } else {
            mn_prefetch_lines(sa, 8, pf.a_share, gw, lane, pf_r, pf_voff, pf_step, pf_on);
          }
        } else if constexpr (C::kBKC) {
          // NB x kRowsB B rows in all (one operand of 128 or 256, or two of
          // 128): each of the 4 tiles along A prefetches a quarter of them
          pf_on = true;
          constexpr int kHalf = NB * kRowsB / 8;  // B rows per wave
          const int first = pf.b_share * 2 * kHalf + (gw - 2) * kHalf;  // of the NB x kRowsB B rows
          // (a branch, not an index: an indexed sb would live in scratch)
          const TileSrc<C::kBKC, kRowsB>& src = (first >= kRowsB) ? sb[NB - 1] : sb[0];
          pf_r = src.rsrc;
          pf_voff = (uint32_t)((first % kRowsB) + (lane & (kHalf - 1))) * src.stride;
        } else {
          mn_prefetch_lines(sb[0], 4, pf.b_share, gw - 2, lane, pf_r, pf_voff, pf_step, pf_on);
        }
      }
    }
    // the lines of K step `step` if it exists; true if a read was issued
    auto prefetch = [&](int step) -> bool {
      if (!pf_on || step >= nk) return false;
      buffer_copy(pf_r, pf.dump, pf_voff, (uint32_t)step * pf_step);
      return true;
    };
    bool pf_last = false;  // the youngest vector memory operation is a prefetch
    // Prologue: steps 0 and 1; step 0 visible at the first barrier.
#pragma unroll
    for (int j = 0; j < C::kCopies; ++j) pipe_copy<C, NB>(sa, sb, 0, lds, gw, j);
    if (nk > 1) {
#pragma unroll
      for (int j = 0; j < C::kCopies; ++j)
        pipe_copy<C, NB>(sa, sb, kPipeBK, lds + C::kStageBytes, gw, j);
      pf_last = prefetch(kPipeAhead - 1);
      if (pf_last) wait_vmcnt<C::kCopies + 1>();
      else wait_vmcnt<C::kCopies>();
    } else {
      wait_vmcnt<0>();
    }
    pipe_barrier();
    // Steps that still copy step i+2, then the last two without copies: two
    // branch-free loop bodies.
    int i = 0;
    for (; i + 2 < nk; ++i) {
      pipe_read<C, NB>(lds + (i & 1) * C::kStageBytes, f, pl, wm, wn, lane);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads of step i done
      if (pf_last) wait_vmcnt<1>();                          // step i+1 has landed
      else wait_vmcnt<0>();
      pipe_barrier();  // 1
      __builtin_amdgcn_s_setprio(1);
      uint8_t* stage = lds + (i & 1) * C::kStageBytes;
      const int64_t k0 = (int64_t)(i + 2) * kPipeBK;
      pipe_mma_copies<C, NB>(f, acc, [&](int j) { pipe_copy<C, NB>(sa, sb, k0, stage, gw, j); });
      pf_last = prefetch(i + kPipeAhead);
      __builtin_amdgcn_s_setprio(0);
      pipe_barrier();  // 2
    }
    for (; i < nk; ++i) {
      pipe_read<C, NB>(lds + (i & 1) * C::kStageBytes, f, pl, wm, wn, lane);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (pf_last) wait_vmcnt<1>();
      else wait_vmcnt<0>();
      pf_last = false;
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
