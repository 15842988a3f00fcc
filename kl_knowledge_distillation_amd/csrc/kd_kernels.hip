// HIP kernels of the fused LM-head + CE + KL distillation loss, gfx950.
//
// Forward  (kd_loss_fwd):
//   prep      one wave per token: label logits z[y], t[y] by a D-long dot
//             product, validity flags; top-K: M = sum p, E = sum p log p and
//             S = sum p z[idx] from the cached entries.
//   fwd       grid = (vocabulary tile) x (128-token tile). A workgroup runs the
//             MFMA main loop (logit tiles z = W H_s^T and t = W H_t^T or
//             W_t H_t^T) and reduces its tile to per-token statistics: the
//             tile maxima of z and t, the sums of 2^(x log2e / T - max) for z,
//             z/T, t/T, t, and the cross term sum 2^(t~ - m) (t - z). The
//             logits never leave registers (flash_kd, module description:
//             online softmax over vocabulary chunks is exact).
//   merge     combines the per-tile records of each token (the online-softmax
//             merge) into lse values, per-token CE / KL / top-K objective, the
//             saved statistics and a per-block partial loss.
//   finalize  one workgroup sums the partials in a fixed order.
// Backward (kd_loss_bwd), per vocabulary chunk (CompactifAI/Full-Chunked-KL-
// Loss, Full Chunked KL: recompute each chunk, apply the closed-form gradient):
//   bwd_dz    recompute the chunk's logit tiles, form dz in registers from the
//             saved lse values (top-K: minus (g/den) w_kl p at the row's cached
//             indices in the tile), round once and store the (n x chunk) slab.
//   gemm_dw   dW[chunk] = dz^T H_s       (K = n)
//   gemm_dh   dH += dz W[chunk]          (K = chunk)
#include <limits.h>
#include <math.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <vector>

#include "kd_device.hpp"
#include "kd_internal.hpp"
#include "kd_pipe.hpp"

namespace kd {

// ---------------------------------------------------------------------------
// Online statistics
// ---------------------------------------------------------------------------

struct RowStats {
  float mz1, sz1;      // z at T = 1 (base-2 units of z log2e)
  float mzT, szT, ar;  // z / T and the cross term sum 2^(z~ - mzT) (z - t) (reverse KL)
  float mtT, stT, a;   // t / T and the cross term sum 2^(t~ - mtT) (t - z)
  float mt1, st1;      // t at T = 1 (teacher CE when T != 1)
};

__device__ __forceinline__ void stats_init(RowStats& s) {
  s.mz1 = s.mzT = s.mtT = s.mt1 = -INFINITY;
  s.sz1 = s.szT = s.stT = s.st1 = s.a = s.ar = 0.f;
}

// 2^(m_old - m_new), with an empty record (m_new = -inf) scaling to 0.
__device__ __forceinline__ float rescale(float m_old, float m_new) {
  return (m_new == -INFINITY) ? 0.f : exp2_fast(m_old - m_new);
}

__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  s = s * rescale(m, mn) + s2 * rescale(m2, mn);
  m = mn;
}

__device__ __forceinline__ void merge_msa(float& m, float& s, float& a, float m2, float s2, float a2) {
  const float mn = fmaxf(m, m2);
  const float f1 = rescale(m, mn), f2 = rescale(m2, mn);
  s = s * f1 + s2 * f2;
  a = a * f1 + a2 * f2;
  m = mn;
}

__device__ __forceinline__ void stats_merge(RowStats& s, const RowStats& o) {
  merge_ms(s.mz1, s.sz1, o.mz1, o.sz1);
  merge_msa(s.mzT, s.szT, s.ar, o.mzT, o.szT, o.ar);
  merge_msa(s.mtT, s.stT, s.a, o.mtT, o.stT, o.a);
  merge_ms(s.mt1, s.st1, o.mt1, o.st1);
}

// A record's ten fields, `stride` floats apart (SoA records).
__device__ __forceinline__ void rec_load(const float* r, int64_t stride, RowStats& o) {
  o.mz1 = r[0 * stride]; o.sz1 = r[1 * stride]; o.mzT = r[2 * stride];
  o.szT = r[3 * stride]; o.mtT = r[4 * stride]; o.stT = r[5 * stride];
  o.a = r[6 * stride];   o.mt1 = r[7 * stride]; o.st1 = r[8 * stride];
  o.ar = r[9 * stride];
}
__device__ __forceinline__ void rec_store(float* r, int64_t stride, const RowStats& o) {
  r[0 * stride] = o.mz1; r[1 * stride] = o.sz1; r[2 * stride] = o.mzT;
  r[3 * stride] = o.szT; r[4 * stride] = o.mtT; r[5 * stride] = o.stT;
  r[6 * stride] = o.a;   r[7 * stride] = o.mt1; r[8 * stride] = o.st1;
  r[9 * stride] = o.ar;
}

// Read access to a wave's tile values, value (mb, nb, r) = register r of
// block (mb, nb): fp32 accumulators, or given bf16 logits still packed two to
// a register (bf16 -> fp32 is exact, so unpacking at each use loses nothing
// and halves the registers the tile holds).
template <int NBT>
struct AccView {
  const f32x4 (&x)[kMB][NBT];
  __device__ __forceinline__ float operator()(int mb, int nb, int r) const { return x[mb][nb][r]; }
};
template <int NBT>
struct PackedView {
  const uint2 (&u)[kMB][NBT];
  __device__ __forceinline__ float operator()(int mb, int nb, int r) const {
    const uint32_t w = (r < 2) ? u[mb][nb].x : u[mb][nb].y;
    return __uint_as_float((r & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <int NBT>
__device__ __forceinline__ AccView<NBT> view(const f32x4 (&x)[kMB][NBT]) { return AccView<NBT>{x}; }
template <int NBT>
__device__ __forceinline__ PackedView<NBT> view(const uint2 (&u)[kMB][NBT]) { return PackedView<NBT>{u}; }

// Bit 4 mb + r of `ok`: register r of row block mb is a real vocabulary row.
__device__ __forceinline__ bool ok_bit(uint32_t ok, int mb, int r) { return (ok >> (mb * 4 + r)) & 1u; }

// Largest of the 16 values a lane holds for token block nb (masked rows skipped).
template <bool TAIL, class XV>
__device__ __forceinline__ float tile_max(const XV& x, int nb, uint32_t ok) {
  float m = -INFINITY;
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (!TAIL || ok_bit(ok, mb, r)) m = fmaxf(m, x(mb, nb, r));
  return m;
}

// sum over the lane's 16 values of 2^(x c - mc); mc = c * (token max), so every
// term is at most 1 and all partial sums of a token share one reference.
template <bool TAIL, class XV>
__device__ __forceinline__ float tile_sum(const XV& x, int nb, float c, float mc, uint32_t ok) {
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int mb = 0; mb < kMB; mb += 2)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float e0 = exp2_fast(fmaf(x(mb, nb, r), c, -mc));
      float e1 = exp2_fast(fmaf(x(mb + 1, nb, r), c, -mc));
      if (TAIL) {
        e0 = ok_bit(ok, mb, r) ? e0 : 0.f;
        e1 = ok_bit(ok, mb + 1, r) ? e1 : 0.f;
      }
      s0 += e0;
      s1 += e1;
    }
  return s0 + s1;
}

// Sum of x at scale c and the cross term. Teacher-weighted (TEACHER_W):
// x = t, y = z, e = 2^(t c - mc), a = sum e (t rho - z); student-weighted:
// x = z, y = t, a = sum e (z - t rho); rho = T_s / T_t, so a / T_s is the
// weighted sum of t / T_t - z / T_s (or its negative). ZERO_SAFE: an e of 0
// adds 0 even where the difference is infinite (a teacher logit of -inf).
template <bool TAIL, bool TEACHER_W, bool ZERO_SAFE = false, class XV, class YV>
__device__ __forceinline__ void tile_sum_cross(const XV& x, const YV& y, int nb, float c, float mc,
                                               float rho, uint32_t ok, float& s, float& a) {
  float s0 = 0.f, s1 = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int mb = 0; mb < kMB; mb += 2)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float e0 = exp2_fast(fmaf(x(mb, nb, r), c, -mc));
      float e1 = exp2_fast(fmaf(x(mb + 1, nb, r), c, -mc));
      if (TAIL) {
        e0 = ok_bit(ok, mb, r) ? e0 : 0.f;
        e1 = ok_bit(ok, mb + 1, r) ? e1 : 0.f;
      }
      s0 += e0;
      s1 += e1;
      float d0, d1;
      if constexpr (TEACHER_W) {
        d0 = fmaf(x(mb, nb, r), rho, -y(mb, nb, r));
        d1 = fmaf(x(mb + 1, nb, r), rho, -y(mb + 1, nb, r));
      } else {
        d0 = fmaf(y(mb, nb, r), -rho, x(mb, nb, r));
        d1 = fmaf(y(mb + 1, nb, r), -rho, x(mb + 1, nb, r));
      }
      if constexpr (ZERO_SAFE) {
        d0 = (e0 > 0.f) ? d0 : 0.f;
        d1 = (e1 > 0.f) ? d1 : 0.f;
      }
      a0 = fmaf(e0, d0, a0);
      a1 = fmaf(e1, d1, a1);
    }
  s = s0 + s1;
  a = a0 + a1;
}

// tile_sum_cross with q = sum e^2 besides: the sum at twice the scale against
// twice the reference. At T = 2 that is the T = 1 sum, so one exponential per
// element serves both temperatures (the square rounds once more, well inside
// fp32). STUDENT_W: the student-weighted cross term (e of z, d = z - t rho);
// CROSS = false: no cross term (a is left alone).
template <bool TAIL, bool CROSS, bool TEACHER_W, bool ZERO_SAFE = false, class XV, class YV>
__device__ __forceinline__ void tile_sums_sq(const XV& x, const YV& y, int nb, float c, float mc,
                                             float rho, uint32_t ok, float& s, float& q, float& a) {
  float s0 = 0.f, s1 = 0.f, q0 = 0.f, q1 = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int mb = 0; mb < kMB; mb += 2)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float e0 = exp2_fast(fmaf(x(mb, nb, r), c, -mc));
      float e1 = exp2_fast(fmaf(x(mb + 1, nb, r), c, -mc));
      if (TAIL) {
        e0 = ok_bit(ok, mb, r) ? e0 : 0.f;
        e1 = ok_bit(ok, mb + 1, r) ? e1 : 0.f;
      }
      s0 += e0;
      s1 += e1;
      q0 = fmaf(e0, e0, q0);
      q1 = fmaf(e1, e1, q1);
      if constexpr (CROSS) {
        float d0, d1;
        if constexpr (TEACHER_W) {
          d0 = fmaf(x(mb, nb, r), rho, -y(mb, nb, r));
          d1 = fmaf(x(mb + 1, nb, r), rho, -y(mb + 1, nb, r));
        } else {
          d0 = fmaf(y(mb, nb, r), -rho, x(mb, nb, r));
          d1 = fmaf(y(mb + 1, nb, r), -rho, x(mb + 1, nb, r));
        }
        if constexpr (ZERO_SAFE) {
          d0 = (e0 > 0.f) ? d0 : 0.f;
          d1 = (e1 > 0.f) ? d1 : 0.f;
        }
        a0 = fmaf(e0, d0, a0);
        a1 = fmaf(e1, d1, a1);
      }
    }
  s = s0 + s1;
  q = q0 + q1;
  if constexpr (CROSS) a = a0 + a1;
}

// ---------------------------------------------------------------------------
// Tile geometry of the fused kernels
// ---------------------------------------------------------------------------

// Staged: 128 vocabulary rows x 128 tokens, 4 waves (2 x 2), registers carry
// the copies; any element type, any hidden size that is a multiple of 8.
// Every geometry: a wave holds kMB x kNB blocks of 16 x 16 (vocabulary rows x
// tokens); col() is the token column (within the tile) of block nb.
struct GeoStaged {
  static constexpr bool kPipe = false;
  static constexpr int kThreads = 256, kVT = 128, kTT = 128, kWM = 2, kNB = 4;
  template <int NB> static constexpr int lds_bytes() { return 2 * (1 + NB) * kTileBytes; }
  __device__ static int col(int wn, int nb, int lane) { return acc_col(wn, nb, lane); }
};
// Pipelined: 256 vocabulary rows x TT tokens, 8 waves (4 x 2, two ping-pong
// groups), buffer-load copies into 3 A slots and 2 or 4 B slots; bf16 with hidden sizes multiple of
// 64. TT = 128 for two B operands (tied teacher) and for the separate teacher's
// two products in turn; TT = 256 for one B operand (top-K, and the tiles that
// hold a given logits tile in registers), which halves the operand bytes
// copied per MFMA against 256 x 128.
template <int TT>
struct GeoPipeT {
  static constexpr bool kPipe = true;
  static constexpr int kThreads = 512, kVT = 256, kTT = TT, kWM = 4, kNB = TT / 32;
  template <int NB> using Cfg = PipeCfg<256, TT, NB>;
  template <int NB> static constexpr int lds_bytes() { return Cfg<NB>::kLdsBytes; }
  __device__ static int col(int wn, int nb, int lane) { return wn * (TT / 2) + nb * 16 + (lane & 15); }
};
using GeoPipe = GeoPipeT<128>;
using GeoWide = GeoPipeT<256>;
using GeoFused = GeoPipe;
static_assert(GeoPipe::kNB == kNB, "the 128-token tiles keep the staged block layout");

// acc[g] = A[a_row0 : +VT, 0:K] * B_g[b_row0 : +TT, 0:K]^T for K-contiguous operands.
template <typename T, class G, int NB>
__device__ __forceinline__ void tile_product(const T* a, int64_t lda, int64_t arows,
                                             const T* const (&b)[NB], int64_t ldb, int64_t brows,
                                             int64_t a_row0, int64_t b_row0, int64_t K,
                                             uint8_t* lds, f32x4 (&acc)[NB][kMB][G::kNB], int tid) {
  if constexpr (G::kPipe) {
    static_assert(sizeof(T) == 2, "the pipelined geometry is bf16 only");
    const PipeOperand A{a, lda, arows};
    PipeOperand B[NB];
#pragma unroll
    for (int g = 0; g < NB; ++g) B[g] = PipeOperand{b[g], ldb, brows};
    pipe_mainloop<typename G::template Cfg<NB>, NB>(A, B, a_row0, b_row0, K, lds, acc, tid);
  } else {
    const Operand<T, true> A{a, lda, arows, K};
    Operand<T, true> B[NB];
#pragma unroll
    for (int g = 0; g < NB; ++g) B[g] = Operand<T, true>{b[g], ldb, brows, K};
    mainloop<T, true, true, NB>(A, B, a_row0, b_row0, K, lds, acc, tid);
  }
}

// Kept products of the last chunk, in register order: tile `tile` (token
// tile x tiles of the chunk + vocabulary tile) holds its waves' accumulators
// one after another, block (mb, nb) of wave w as 64 lanes x 16 bytes, so every
// store and load of a wave is one contiguous 1 KB and a tile one contiguous
// [kVT x kTT] block. Only the library reads the layout back, with the same
// tile geometry.
template <int NBT>
__device__ __forceinline__ int64_t kept_block(int64_t tile, int waves, int w, int lane) {
  return ((tile * waves + w) * (kMB * NBT)) * 256 + lane * 4;
}
// Stores are nontemporal: the backward reads them back only after the rest of
// the forward and a whole recomputed chunk (equal or 0.3% faster per step).
template <int NBT>
__device__ __forceinline__ void kept_store(float* m, int64_t tile, int waves, int w, int lane,
                                           const f32x4 (&x)[kMB][NBT]) {
  float* p = m + kept_block<NBT>(tile, waves, w, lane);
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBT; ++nb)
      __builtin_nontemporal_store(x[mb][nb], reinterpret_cast<f32x4*>(p + (mb * NBT + nb) * 256));
}
// Token block nb of that part read back (streaming loads: each byte is read
// once); a token that is not live reads as zero.
template <int NBT>
__device__ __forceinline__ void kept_load(const float* m, int64_t tile, int waves, int w, int lane, int nb,
                                          bool live, f32x4 (&x)[kMB]) {
  const float* p = m + kept_block<NBT>(tile, waves, w, lane);
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) {
    const uint4 u = load_stream(p + (mb * NBT + nb) * 256);
    x[mb] = live ? f32x4{__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w)}
                 : f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// The [kVT x kTT] tile of a row-major [n x v] logits matrix (tokens are rows)
// in the accumulator layout: register r of row block mb, token block nb holds
// vocabulary row v0 + acc_row(wm, mb, r, lane) of token t0 + acc_col(wn, nb, lane).
// A lane's four rows are consecutive in memory and load as one 8-byte (bf16) or
// 16-byte (fp32) vector when `vec` (v a multiple of 4, base aligned to the
// vector). Rows past v and tokens past n read 0; the epilogue masks them.
template <typename T>
__device__ __forceinline__ void load_logits_tile(const T* L, int64_t n, int64_t v, int64_t t0, int64_t v0,
                                                 int wm, int wn, int lane, bool vec, WaveAcc& out) {
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int64_t tok = t0 + acc_col(wn, nb, lane);
    const bool live = tok < n;
    const int64_t base = live ? tok * v : 0;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      const int64_t vv = v0 + acc_row(wm, mb, 0, lane);
      if (live && vec && vv + 4 <= v) {
        if constexpr (sizeof(T) == 2) {
          const uint2 u = *reinterpret_cast<const uint2*>(L + base + vv);
          out[mb][nb][0] = __uint_as_float(u.x << 16);
          out[mb][nb][1] = __uint_as_float(u.x & 0xffff0000u);
          out[mb][nb][2] = __uint_as_float(u.y << 16);
          out[mb][nb][3] = __uint_as_float(u.y & 0xffff0000u);
        } else {
          const float4 f = *reinterpret_cast<const float4*>(L + base + vv);
          out[mb][nb][0] = f.x;
          out[mb][nb][1] = f.y;
          out[mb][nb][2] = f.z;
          out[mb][nb][3] = f.w;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          out[mb][nb][r] = (live && vv + r < v) ? to_f32(L[base + vv + r]) : 0.f;
      }
    }
  }
}

// Given bf16 logits in registers (pipelined geometry, 256-token tiles): every
// wave loads its own part of the tile, still packed (two bf16 per register,
// unpacked at each use; bf16 -> fp32 is exact), after the main loop, whose
// registers it would not fit beside. `vec`: v a multiple of 4 and the matrix
// 8-byte aligned (one 8-byte load per lane and block); otherwise element
// loads. Tokens past n and rows past v read 0. (Staging the tile through LDS
// with buffer loads instead measured 2-4% slower.)
template <int NBT>
using GivenRawT = uint2[kMB][NBT];
typedef GivenRawT<kNB> GivenRaw;
// G: the tile geometry (its token column map and token blocks per wave);
// token blocks nb0 .. nb0 + count - 1 (default: all of them).
template <class G>
__device__ __forceinline__ void given_raw_load(const bf16_t* L, int64_t n, int64_t v, int64_t t0,
                                               int64_t v0, int wm, int wn, int lane, bool vec,
                                               GivenRawT<G::kNB>& raw, int nb0 = 0, int count = G::kNB) {
#pragma unroll
  for (int nb = nb0; nb < nb0 + count; ++nb) {
    const int64_t tok = t0 + G::col(wn, nb, lane);
    const bool live = tok < n;
    const int64_t base = live ? tok * v : 0;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      const int64_t vv = v0 + acc_row(wm, mb, 0, lane);
      if (live && vec && vv + 4 <= v) {
        raw[mb][nb] = *reinterpret_cast<const uint2*>(L + base + vv);
      } else {
        uint32_t e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) e[r] = (live && vv + r < v) ? (uint32_t)L[base + vv + r] : 0u;
        raw[mb][nb] = make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
      }
    }
  }
}

// Given logits of this tile in the staged geometry, loaded after the main
// loop (flag 1: 4-element vectors, 0: elements).
template <typename T>
__device__ __forceinline__ void given_tile(const T* L, int64_t n, int64_t v, int64_t t0, int64_t v0,
                                           int flag, int wm, int wn, int lane, WaveAcc& out) {
  load_logits_tile<T>(L, n, v, t0, v0, wm, wn, lane, flag != 0, out);
}

// ---------------------------------------------------------------------------
// Forward tile kernel
// ---------------------------------------------------------------------------

struct FwdArgs {
  const void* hs;
  const void* w;
  const void* ht;
  const void* wt;
  const void* logits;   // student logits (LOGITS)
  const void* tlogits;  // teacher logits (TLOGITS)
  int64_t n, d, dt, v;
  int n_ttiles, n_vtiles, tps, n_slices;
  float cT, cTt, rho;   // log2(e) / T_s, log2(e) / T_t, T_s / T_t
  int need_zT, need_t1;
  int kl;      // KD_KL_*: the reverse direction also needs sum 2^(z~ - m) (z - t)
  int vec;     // given logits: given_mode (3 / 4 registers, 1 vector loads, 0 element loads)
  int sqz;     // T_s == 2: the T = 1 student sums are the squares of those at T
  float* rec;  // [kRecFields][n_slices][n]
  const int32_t* nv;  // compacted rows: their number (tiles past it exit); null = n
  // top-K teacher: each row's k entries sorted by index and where each
  // vocabulary tile's entries start (prep_kernel)
  const int32_t* topk_sidx;  // [n, k]
  const float* topk_sprob;   // [n, k]
  const int32_t* topk_off;   // [n, n_slices + 1]: this launch's tiles
  int k;
  int slice0;                // first vocabulary tile of this launch (n_slices tiles from it)
  // non-null: this launch's products kept for the backward in register order
  // (student, then the teacher's keep_t elements later)
  float* keep;
  int64_t keep_t;
};

template <typename T, int MODE, class G>
__global__ __launch_bounds__(G::kThreads, 2) void fwd_tiles_kernel(FwdArgs a) {
  constexpr int NB = (MODE == MODE_TIED) ? 2 : 1;
  constexpr int NBT = G::kNB;  // token blocks of 16 per wave
  using Acc = f32x4[kMB][NBT];
  constexpr bool kGiven = MODE == MODE_TLOGITS || MODE == MODE_LOGITS;  // one logits tile is given
  constexpr int kMainBytes = G::template lds_bytes<NB>();
  // pipelined tiles hold a given logits tile in registers
  constexpr bool kGivenRegs = kGiven && G::kPipe;
  constexpr int kLdsMain = kMainBytes;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsMain];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  // Compacted rows: only the token tiles below nv have work; they are mapped
  // onto the first blocks of every XCD and the rest of the grid exits.
  const int n_tt = a.nv ? (int)((*a.nv + G::kTT - 1) / G::kTT) : a.n_ttiles;
  int t;
  if (!xcd_live_tile(blockIdx.x, a.n_slices * n_tt, t)) return;
  int slice, tt;  // slice = the vocabulary tile of this workgroup
  grouped_tile(t, a.n_slices, n_tt, tile_group(G::kVT, G::kTT), slice, tt);
  const int64_t t0 = (int64_t)tt * G::kTT;
  const int64_t v0 = (int64_t)(a.slice0 + slice) * G::kVT;

  const T* hs = static_cast<const T*>(a.hs);
  const T* W = static_cast<const T*>(a.w);
  const T* ht = static_cast<const T*>(a.ht);
  const T* Wt = static_cast<const T*>(a.wt);

  f32x4 acc[NB][kMB][NBT];
  f32x4 tacc[1][kMB][NBT];  // teacher accumulator of the separate / logits modes
  // a given logits tile (the scorer's student logits, LOGITS; a cached dense
  // teacher, TLOGITS): on the pipelined path always a 256-token tile, kept
  // packed beside the 128 accumulator registers and unpacked at each use
  static_assert(!kGivenRegs || G::kTT > 128, "pipelined given tiles are 256-token tiles");
  constexpr bool kPacked = kGiven && kGivenRegs;
  constexpr bool kPackedZ = kPacked && MODE == MODE_LOGITS;
  constexpr bool kPackedT = kPacked && MODE == MODE_TLOGITS;
  Acc zl;
  GivenRawT<NBT> zraw;  // the packed given tile (student or teacher)

  if constexpr (MODE == MODE_TIED) {
    const T* const b[2] = {hs, ht};
    tile_product<T, G, 2>(W, a.d, a.v, b, a.d, a.n, v0, t0, a.d, lds, acc, tid);
  } else if constexpr (MODE == MODE_SEPARATE) {
    const T* const b[1] = {hs};
    tile_product<T, G, 1>(W, a.d, a.v, b, a.d, a.n, v0, t0, a.d, lds, acc, tid);
    const T* const bt[1] = {ht};
    tile_product<T, G, 1>(Wt, a.dt, a.v, bt, a.dt, a.n, v0, t0, a.dt, lds, tacc, tid);
  } else if constexpr (MODE == MODE_TOPK) {
    const T* const b[1] = {hs};
    tile_product<T, G, 1>(W, a.d, a.v, b, a.d, a.n, v0, t0, a.d, lds, acc, tid);
  } else if constexpr (MODE == MODE_TLOGITS) {
    const T* L = static_cast<const T*>(a.tlogits);
    const T* const b[1] = {hs};
    if constexpr (kPackedT) {  // the teacher tile is loaded in the epilogue, half at a time
      tile_product<T, G, 1>(W, a.d, a.v, b, a.d, a.n, v0, t0, a.d, lds, acc, tid);
    } else {
      tile_product<T, G, 1>(W, a.d, a.v, b, a.d, a.n, v0, t0, a.d, lds, acc, tid);
      given_tile<T>(L, a.n, a.v, t0, v0, a.vec, wm, wn, lane, tacc[0]);
    }
  } else {  // MODE_LOGITS
    const T* L = static_cast<const T*>(a.logits);
    const T* const bt[1] = {ht};
    if constexpr (kPackedZ) {
      // the given tile (64 registers) would not fit beside the main loop's; it
      // is loaded in the epilogue (its latency is a few percent of the tile's)
      tile_product<T, G, 1>(Wt, a.dt, a.v, bt, a.dt, a.n, v0, t0, a.dt, lds, tacc, tid);
    } else {
      tile_product<T, G, 1>(Wt, a.dt, a.v, bt, a.dt, a.n, v0, t0, a.dt, lds, tacc, tid);
      given_tile<T>(L, a.n, a.v, t0, v0, a.vec, wm, wn, lane, zl);
    }
  }
  // The products of the last chunk, stored for the backward before the
  // epilogue so that the stores drain under its arithmetic.
  if constexpr (MODE != MODE_LOGITS) {
    if (a.keep) {
      const int64_t tile = (int64_t)tt * a.n_slices + slice;
      constexpr int kWaves = G::kThreads / 64;
      kept_store<NBT>(a.keep, tile, kWaves, w, lane, acc[0]);
      if constexpr (MODE == MODE_TIED || MODE == MODE_SEPARATE)
        kept_store<NBT>(a.keep + a.keep_t, tile, kWaves, w, lane, MODE == MODE_TIED ? acc[NB - 1] : tacc[0]);
    }
  }

  // Epilogue: this tile's statistics of every token, in two passes over the
  // registers. (1) Token maxima of z and t over the tile's vocabulary rows:
  // lane maxima, then the four lanes l % 16 + 16 q, then the kWM waves of the
  // token block (LDS). (2) Sums of 2^(x c - c max) against those maxima, so the
  // partial sums of lanes and waves simply add. The main loop ended with a
  // barrier, so its LDS is free.
  uint32_t ok = 0xffffu;
  const bool tail = v0 + G::kVT > a.v;
  if (tail) {
    ok = 0u;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (v0 + acc_row(wm, mb, r, lane) < a.v) ok |= 1u << (mb * 4 + r);
  }
  const Acc& z_acc = (MODE == MODE_LOGITS) ? zl : acc[0];
  const Acc& tl_acc = (MODE == MODE_TIED) ? acc[NB - 1] : tacc[0];
  const auto z = [&]() {
    if constexpr (kPackedZ) return view(zraw);
    else return view(z_acc);
  }();
  const auto tl = [&]() {
    if constexpr (kPackedT) return view(zraw);
    else return view(tl_acc);
  }();
  constexpr bool kTeacher = MODE != MODE_TOPK;
  constexpr bool kInfT = MODE == MODE_TLOGITS;  // given teacher logits may be -inf
  constexpr int kSums = 6;  // sz1, szT, stT, a (top-K: sum p z[idx]), st1, ar
  static_assert(G::kWM * 2 * NBT * (2 + kSums) * 16 * 4 <= kLdsMain, "epilogue exchange fits the LDS");
  constexpr int kNBX = kPacked ? NBT / 2 : NBT;                   // token blocks per exchange
  float* xmax = reinterpret_cast<float*>(lds);                    // [kWM][2][kNBX][2][16]
  float* xsum = xmax + G::kWM * 2 * kNBX * 2 * 16;                // [kWM][2][kNBX][kSums][16]
  const int rb = acc_row(wm, 0, 0, lane);  // this lane's rows: v0 + rb + 16 mb + r
  const int l16 = lane & 15;

  // Top-K: each token block's run of index-sorted entries in this tile, read
  // for all token blocks before any is used (a row past n reads row 0's bounds
  // and gets an empty run), so that the loads' latencies overlap.
  int kj0[MODE == MODE_TOPK ? NBT : 1], kj1[MODE == MODE_TOPK ? NBT : 1];
  if constexpr (MODE == MODE_TOPK) {
#pragma unroll
    for (int nb = 0; nb < NBT; ++nb) {
      const int64_t tok = t0 + G::col(wn, nb, lane);
      const bool live = tok < a.n;
      const int32_t* off = a.topk_off + (live ? tok : 0) * (a.n_slices + 1) + slice;
      const int o0 = off[0], o1 = off[1];
      kj0[nb] = live ? o0 : 0;
      kj1[nb] = live ? o1 : 0;
    }
  }
  // 256-token tiles with packed given logits run the epilogue in two halves of
  // token blocks, each loading its half of the given tile just before it, so
  // only half of it is held beside the teacher accumulators.
  constexpr int kHalves = kPacked ? 2 : 1;
  constexpr int NBH = NBT / kHalves;
  auto half = [&](auto h_tag) {
  constexpr int h = decltype(h_tag)::value;  // compile-time, so every register index is too
  if constexpr (kPacked) {
    const T* L = static_cast<const T*>(kPackedZ ? a.logits : a.tlogits);
    given_raw_load<G>(reinterpret_cast<const bf16_t*>(L), a.n, a.v, t0, v0, wm, wn, lane, a.vec == 3, zraw,
                      h * NBH, NBH);
  }
  float mz[NBH], mt[NBH];
#pragma unroll
  for (int jb = 0; jb < NBH; ++jb) {
    const int nb = h * NBH + jb;
    mz[jb] = tail ? tile_max<true>(z, nb, ok) : tile_max<false>(z, nb, ok);
    mt[jb] = !kTeacher ? 0.f : (tail ? tile_max<true>(tl, nb, ok) : tile_max<false>(tl, nb, ok));
#pragma unroll
    for (int off = 16; off <= 32; off *= 2) {
      mz[jb] = fmaxf(mz[jb], __shfl_xor(mz[jb], off));
      if (kTeacher) mt[jb] = fmaxf(mt[jb], __shfl_xor(mt[jb], off));
    }
    if (lane < 16) {
      float* p = xmax + (((wm * 2 + wn) * NBH + jb) * 2) * 16 + l16;
      p[0] = mz[jb];
      p[16] = mt[jb];
    }
  }
  __syncthreads();
#pragma unroll
  for (int jb = 0; jb < NBH; ++jb) {
    // every wave reads the same kWM values (fmax is exact, so the order is free)
    float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
    for (int src = 0; src < G::kWM; ++src) {
      const float* p = xmax + (((src * 2 + wn) * NBH + jb) * 2) * 16 + l16;
      m0 = fmaxf(m0, p[0]);
      m1 = fmaxf(m1, p[16]);
    }
    mz[jb] = m0;
    mt[jb] = m1;
  }
#pragma unroll
  for (int jb = 0; jb < NBH; ++jb) {
    const int nb = h * NBH + jb;
    float v[kSums] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const bool rev = a.kl != KD_KL_FORWARD;
    if constexpr (MODE == MODE_TOPK) {
      // sum of p z[idx] over the token's cached entries in this tile (orda-kernel,
      // Teacher descriptors: TopKTeacher), from the tile's own z values: the
      // token's run of index-sorted entries, each added by the lane that holds
      // its row; the lane and wave partials add up like the sums below.
      const int64_t tok = t0 + G::col(wn, nb, lane);
      float cr = 0.f;
      {
        const int j0 = kj0[nb], j1 = kj1[nb];  // sorted entries with index in [v0, v0 + kVT) and < v
        const int32_t* ix = a.topk_sidx + tok * a.k;
        const float* pr = a.topk_sprob + tok * a.k;
        const int base = (int)(v0 + rb);
        for (int j = j0; j < j1; ++j) {
          const int d = ix[j] - base;
          float zz = 0.f;
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) zz = (d == 16 * mb + r) ? z(mb, nb, r) : zz;
          cr = fmaf(pr[j], zz, cr);
        }
      }
      v[3] = cr;
    }
    const float mz1 = mz[jb] * kLog2e, mzT = mz[jb] * a.cT;
    // A teacher tile with no finite logit (all -inf) sums 2^-inf = 0 against a
    // finite reference; its record keeps the -inf maximum, which the merge
    // treats as empty.
    const float mtb = (kInfT && mt[jb] == -INFINITY) ? 0.f : mt[jb];
    const float mtT = mtb * a.cTt, mt1 = mtb * kLog2e;
    auto sums = [&](auto tail_tag) {
      constexpr bool TL = decltype(tail_tag)::value;
      if (kTeacher && a.sqz) {
        // T_s = 2: the sums at z/T and at z from one exponential per element
        if (rev) tile_sums_sq<TL, true, false>(z, tl, nb, a.cT, mzT, a.rho, ok, v[1], v[0], v[5]);
        else tile_sums_sq<TL, false, false>(z, z, nb, a.cT, mzT, 0.f, ok, v[1], v[0], v[5]);
      } else {
        v[0] = tile_sum<TL>(z, nb, kLog2e, mz1, ok);
        if (kTeacher) {
          if (rev) tile_sum_cross<TL, false>(z, tl, nb, a.cT, mzT, a.rho, ok, v[1], v[5]);
          else if (a.need_zT) v[1] = tile_sum<TL>(z, nb, a.cT, mzT, ok);
        }
      }
      if (kTeacher) {
        tile_sum_cross<TL, true, kInfT>(tl, z, nb, a.cTt, mtT, a.rho, ok, v[2], v[3]);
        if (a.need_t1) v[4] = tile_sum<TL>(tl, nb, kLog2e, mt1, ok);
      }
    };
    if (tail) sums(std::true_type{});
    else sums(std::false_type{});
#pragma unroll
    for (int j = 0; j < kSums; ++j) {
      v[j] += __shfl_xor(v[j], 16);
      v[j] += __shfl_xor(v[j], 32);
    }
    if (lane < 16) {
      float* p = xsum + (((wm * 2 + wn) * NBH + jb) * kSums) * 16 + l16;
#pragma unroll
      for (int j = 0; j < kSums; ++j) p[j * 16] = v[j];
    }
  }
  __syncthreads();
  if (wm == 0 && lane < 16) {
#pragma unroll
    for (int jb = 0; jb < NBH; ++jb) {
      const int nb = h * NBH + jb;
      float v[kSums] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int src = 0; src < G::kWM; ++src) {  // fixed order
        const float* p = xsum + (((src * 2 + wn) * NBH + jb) * kSums) * 16 + l16;
#pragma unroll
        for (int j = 0; j < kSums; ++j) v[j] += p[j * 16];
      }
      const int64_t tok = t0 + G::col(wn, nb, lane);
      if (tok < a.n) {
        const int64_t stride = (int64_t)a.n_slices * a.n;
        float* r = a.rec + (int64_t)slice * a.n + tok;
        r[0 * stride] = mz[jb] * kLog2e; r[1 * stride] = v[0];
        r[2 * stride] = mz[jb] * a.cT;   r[3 * stride] = v[1];
        r[4 * stride] = mt[jb] * a.cTt;  r[5 * stride] = v[2];
        // top-K: field 6 carries the tile's cross term sum p z[idx]
        r[6 * stride] = v[3];
        r[7 * stride] = mt[jb] * kLog2e; r[8 * stride] = v[4];
        r[9 * stride] = v[5];
      }
    }
  }
  };
  half(std::integral_constant<int, 0>{});
  if constexpr (kHalves == 2) half(std::integral_constant<int, 1>{});
}

// ---------------------------------------------------------------------------
// Prep: label logits, validity, top-K sums (one wave per token)
// ---------------------------------------------------------------------------

struct PrepArgs {
  const void* hs;
  const void* w;
  const void* ht;
  const void* wt;
  const void* logits;   // student logits (LOGITS)
  const void* tlogits;  // teacher logits (TLOGITS)
  const int64_t* labels;
  const int32_t* idx;
  const float* prob;
  int64_t n, d, dt, v, ignore;
  int k;
  int want_teacher;  // teacher label logit needed (teacher CE weight or output)
  float* prep;       // [4][n]: z[y] | S, t[y] | E, M, flag; null: not written
  // top-K: the row's entries sorted by index (an index outside [0, v) as v,
  // last)
  int32_t* sidx;
  float* sprob;
};

template <typename T>
__device__ __forceinline__ float wave_dot(const T* x, const T* y, int64_t len, int lane) {
  constexpr int PC = Elem<T>::kPerChunk;
  float s = 0.f;
  for (int64_t e = (int64_t)lane * PC; e < len; e += 64 * PC) {
    const uint4 ux = *reinterpret_cast<const uint4*>(x + e);
    const uint4 uy = *reinterpret_cast<const uint4*>(y + e);
    const T* px = reinterpret_cast<const T*>(&ux);
    const T* py = reinterpret_cast<const T*>(&uy);
#pragma unroll
    for (int j = 0; j < PC; ++j) s = fmaf(to_f32(px[j]), to_f32(py[j]), s);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  return s;
}

template <typename T, int MODE>
__global__ __launch_bounds__(kThreads) void prep_kernel(PrepArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (i >= a.n) return;
  const T* hs = static_cast<const T*>(a.hs);
  const T* W = static_cast<const T*>(a.w);
  float f0 = 0.f, f1 = 0.f, f2 = 0.f, flag = 1.f;
  if constexpr (MODE == MODE_TOPK) {
    // the mass and sum p log p of the row (its cross term comes from the
    // tiles), and its entries sorted by index for them: entry j goes to its
    // rank (ties in entry order), O(k^2) compares per row
    const int32_t* ix = a.idx + i * a.k;
    const float* pr = a.prob + i * a.k;
    auto key = [&](int j) -> int64_t {
      const int64_t x = ix[j];
      return (x < 0 || x >= a.v) ? a.v : x;  // never used as an address
    };
    float mass = 0.f, ent = 0.f;
    bool bad = false;
    for (int j = lane; j < a.k; j += 64) {
      const float p = pr[j];
      mass += p;
      ent += (p > 0.f) ? p * logf(p) : 0.f;
      const int64_t kj = key(j);
      bad = bad || kj == a.v;
      int rank = 0;
      for (int jj = 0; jj < a.k; ++jj) {
        const int64_t kk = key(jj);
        rank += (kk < kj || (kk == kj && jj < j)) ? 1 : 0;
      }
      a.sidx[i * a.k + rank] = (int32_t)kj;
      a.sprob[i * a.k + rank] = p;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      mass += __shfl_xor(mass, off);
      ent += __shfl_xor(ent, off);
    }
    bad = __any(bad);
    f1 = ent;
    f2 = mass;
    flag = bad ? 2.f : 1.f;
  } else {
    const int64_t y = a.labels ? a.labels[i] : a.ignore;
    const bool in_range = y >= 0 && y < a.v;
    const bool valid = a.labels == nullptr || (y != a.ignore && in_range);
    flag = valid ? 1.f : ((y != a.ignore && !in_range) ? 2.f : 0.f);
    if (a.labels != nullptr && valid) {
      if constexpr (MODE == MODE_LOGITS || MODE == MODE_BOTH) {
        f0 = to_f32(static_cast<const T*>(a.logits)[i * a.v + y]);
      } else {
        f0 = wave_dot<T>(hs + i * a.d, W + y * a.d, a.d, lane);
      }
      if (a.want_teacher) {
        if constexpr (MODE == MODE_TLOGITS || MODE == MODE_BOTH) {
          f1 = to_f32(static_cast<const T*>(a.tlogits)[i * a.v + y]);
        } else {
          const T* ht = static_cast<const T*>(a.ht);
          const T* Wt = static_cast<const T*>(a.wt);
          f1 = wave_dot<T>(ht + i * a.dt, Wt + y * a.dt, a.dt, lane);
        }
      }
    }
  }
  if (lane == 0 && a.prep) {  // (the backward only wants the sorted entries)
    a.prep[i] = f0;
    a.prep[a.n + i] = f1;
    a.prep[2 * a.n + i] = f2;
    a.prep[3 * a.n + i] = flag;
  }
}

// Top-K, one forward launch (vocabulary tiles slice0 .. slice0 + n_slices):
// where each tile's run of a row's index-sorted entries starts, by binary
// search, off[i][j] = #{entries of row i with index < min((slice0 + j) vt, v)},
// j = 0 .. n_slices (the last one closes the last tile's run).
struct TileStartArgs {
  const int32_t* sidx;  // [n, k] sorted; an index outside [0, v) stored as v
  int64_t n, v;
  int k, vt_rows, slice0, n_slices;
  int32_t* off;         // [n, n_slices + 1]
};

__global__ __launch_bounds__(kThreads) void topk_tile_starts_kernel(TileStartArgs a) {
  const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t per = a.n_slices + 1;
  if (e >= a.n * per) return;
  const int64_t i = e / per;
  const int j = (int)(e - i * per);
  const int64_t lo = min((int64_t)(a.slice0 + j) * a.vt_rows, a.v);
  const int32_t* sk = a.sidx + i * a.k;
  int l = 0, h = a.k;  // the first position with index >= lo
  while (l < h) {
    const int m = (l + h) >> 1;
    if ((int64_t)sk[m] < lo) l = m + 1;
    else h = m;
  }
  a.off[e] = l;
}

// ---------------------------------------------------------------------------
// Student and teacher logits both given (nemo kd_loss, KDLoss.forward): no
// projection, so the path is HBM-bound and runs as row kernels: one wave per
// slice of a token row streams that part of both [n x v] matrices once, with
// 16-byte loads; each slice leaves one record for the merge.
// ---------------------------------------------------------------------------

struct RowArgs {
  const void* zl;       // student logits [n, v]
  const void* tl;       // teacher logits [n, v]
  int64_t n, v;
  int64_t slice;        // elements per slice of a row, a whole number of steps
  int n_slices;         // slices per row (one wave each)
  float cT, cTt, rho;   // log2(e) / T_s, log2(e) / T_t, T_s / T_t
  int vec;              // rows (and the output) 16-byte aligned: chunk loads and stores
  float* rec;           // [kRecFields][n_slices][n] (forward)
  // backward
  const int64_t* labels;
  int64_t ignore;
  const float* saved;
  const float* grad;
  float ws, wkl, T;
  int kl, accumulate;
  void* dz;             // [n, v] student dtype
};

// The (row, slice) of this wave and the slice's element range [b0, b1);
// false for a wave past the last row.
__device__ __forceinline__ bool row_wave(const RowArgs& a, int64_t& i, int& sl, int64_t& b0,
                                         int64_t& b1) {
  const int64_t w = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  i = w / a.n_slices;
  sl = (int)(w - i * a.n_slices);
  b0 = (int64_t)sl * a.slice;
  b1 = min(a.v, b0 + a.slice);
  return i < a.n;
}

// The 16 bytes of elements [e0, e0 + PC) of a row, still packed, for a step
// that may cross `end`: elements at or past it read as -inf (weight 0).
template <typename T>
__device__ __forceinline__ uint4 row_fetch(const T* row, int64_t e0, int64_t end, bool vec) {
  constexpr int PC = Elem<T>::kPerChunk;
  if (vec && e0 + PC <= end) return load_stream(row + e0);
  uint4 u;
  T* p = reinterpret_cast<T*>(&u);
#pragma unroll
  for (int j = 0; j < PC; ++j) {
    if (e0 + j < end) {
      p[j] = row[e0 + j];
    } else if constexpr (sizeof(T) == 2) {
      p[j] = (T)0xff80u;  // bf16 -inf
    } else {
      p[j] = -INFINITY;
    }
  }
  return u;
}

template <typename T>
__device__ __forceinline__ void row_unpack(const uint4& u, float (&x)[Elem<T>::kPerChunk]) {
  const T* p = reinterpret_cast<const T*>(&u);
#pragma unroll
  for (int j = 0; j < Elem<T>::kPerChunk; ++j) x[j] = to_f32(p[j]);
}

// Running statistics of one lane: maxima of z and t (raw units) and the sums
// of record fields 1, 3, 5, 6, 8, 9 against them.
struct RowRun {
  float mz, mt;
  float sz1, szT, ar, stT, at, st1;
};

__device__ __forceinline__ float run_scale(float m_old, float m_new, float c) {
  // the sums against m_old re-expressed against m_new >= m_old (0 while empty)
  return (m_old == m_new) ? 1.f : ((m_old == -INFINITY) ? 0.f : exp2_fast((m_old - m_new) * c));
}

__device__ __forceinline__ void row_fold(RowRun& r, const RowRun& o, float cT, float cTt) {
  const float mz = fmaxf(r.mz, o.mz), mt = fmaxf(r.mt, o.mt);
  const float a1 = run_scale(r.mz, mz, kLog2e), b1 = run_scale(o.mz, mz, kLog2e);
  const float aT = run_scale(r.mz, mz, cT), bT = run_scale(o.mz, mz, cT);
  const float c1 = run_scale(r.mt, mt, kLog2e), d1 = run_scale(o.mt, mt, kLog2e);
  const float cTs = run_scale(r.mt, mt, cTt), dTs = run_scale(o.mt, mt, cTt);
  r.sz1 = r.sz1 * a1 + o.sz1 * b1;
  r.szT = r.szT * aT + o.szT * bT;
  r.ar = r.ar * aT + o.ar * bT;
  r.stT = r.stT * cTs + o.stT * dTs;
  r.at = r.at * cTs + o.at * dTs;
  r.st1 = r.st1 * c1 + o.st1 * d1;
  r.mz = mz;
  r.mt = mt;
}

// How the row kernels get the T = 1 student terms: from squares of the ones at
// T_s = 2, as those very terms (T_s = 1), or from their own exponentials.
enum RowZ1 { kZ1Square = 0, kZ1Same = 1, kZ1Own = 2 };

// max(x, -1e30) in one instruction: a -inf logit as a huge finite one
__device__ __forceinline__ float clamp_ninf(float x) {
  return __builtin_amdgcn_fmed3f(x, -1e30f, 3.0e38f);
}

// One step of a lane: raise the running maxima to cover the step's elements
// (rescaling the sums once), then add the elements' terms against them. Z1,
// REV (a reverse-direction KL) and T1 (teacher sums at T = 1 kept apart) are
// template arguments so that the step holds only the terms it needs.
template <typename T, int Z1, bool REV, bool T1>
__device__ __forceinline__ void rowstats_step(RowRun& r, const uint4 (&rz)[kRowUnroll],
                                              const uint4 (&rt)[kRowUnroll], const RowArgs& a) {
  constexpr int PC = Elem<T>::kPerChunk;
  float z[kRowUnroll][PC], t[kRowUnroll][PC];
#pragma unroll
  for (int u = 0; u < kRowUnroll; ++u) {
    row_unpack<T>(rz[u], z[u]);
    row_unpack<T>(rt[u], t[u]);
  }
  float mz = r.mz, mt = r.mt;
#pragma unroll
  for (int u = 0; u < kRowUnroll; ++u)
#pragma unroll
    for (int j = 0; j < PC; ++j) {
      mz = fmaxf(mz, z[u][j]);
      mt = fmaxf(mt, t[u][j]);
    }
  const float aT = run_scale(r.mz, mz, a.cT), cTs = run_scale(r.mt, mt, a.cTt);
  r.szT *= aT;
  r.ar *= aT;
  if constexpr (Z1 == kZ1Square) r.sz1 *= aT * aT;
  else if constexpr (Z1 == kZ1Own) r.sz1 *= run_scale(r.mz, mz, kLog2e);
  r.stT *= cTs;
  r.at *= cTs;
  if constexpr (T1) r.st1 *= run_scale(r.mt, mt, kLog2e);
  r.mz = mz;
  r.mt = mt;
  // an all -inf prefix keeps a finite base, so that its terms stay 0
  const float bz = (mz == -INFINITY) ? 0.f : mz, bt = (mt == -INFINITY) ? 0.f : mt;
  const float bzT = bz * a.cT, bz1 = bz * kLog2e, btT = bt * a.cTt, bt1 = bt * kLog2e;
#pragma unroll
  for (int u = 0; u < kRowUnroll; ++u)
#pragma unroll
    for (int j = 0; j < PC; ++j) {
      // a -inf logit (a zero probability, or past the row) has e = 0; in the
      // forward cross difference it stands as -1e30, so that 0 times it stays 0
      const float zz = z[u][j], tt = t[u][j];
      const float ezT = exp2_fast(fmaf(zz, a.cT, -bzT));
      const float etT = exp2_fast(fmaf(tt, a.cTt, -btT));
      if constexpr (Z1 == kZ1Square) r.sz1 = fmaf(ezT, ezT, r.sz1);
      else if constexpr (Z1 == kZ1Own) r.sz1 += exp2_fast(fmaf(zz, kLog2e, -bz1));
      r.szT += ezT;
      r.stT += etT;
      r.at = fmaf(etT, fmaf(clamp_ninf(tt), a.rho, -clamp_ninf(zz)), r.at);
      // reverse: a -inf teacher logit under student mass makes the KL +inf
      if constexpr (REV) r.ar = (ezT > 0.f) ? fmaf(ezT, fmaf(tt, -a.rho, zz), r.ar) : r.ar;
      if constexpr (T1) r.st1 += exp2_fast(fmaf(tt, kLog2e, -bt1));
    }
  if constexpr (Z1 == kZ1Same) r.sz1 = r.szT;
}

// Forward statistics of one slice of a row: one record, as a vocabulary tile
// of the projected paths leaves, for the merge.
template <typename T, int Z1, bool REV, bool T1>
__global__ __launch_bounds__(kThreads) void rowstats_kernel(RowArgs a) {
  constexpr int PC = Elem<T>::kPerChunk;
  constexpr int64_t kStep = kRowUnroll * 64 * PC;
  const int lane = threadIdx.x & 63;
  int64_t i, b0, b1;
  int sl;
  if (!row_wave(a, i, sl, b0, b1)) return;
  const T* zr = static_cast<const T*>(a.zl) + i * a.v;
  const T* tr = static_cast<const T*>(a.tl) + i * a.v;
  RowRun r{-INFINITY, -INFINITY, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int64_t b = b0;
  uint4 rz[kRowUnroll], rt[kRowUnroll];
  if (a.vec) {  // whole steps: plain 16-byte loads
    for (; b + kStep <= b1; b += kStep) {
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        const int64_t e0 = b + (u * 64 + lane) * PC;
        rz[u] = load_stream(zr + e0);
        rt[u] = load_stream(tr + e0);
      }
      rowstats_step<T, Z1, REV, T1>(r, rz, rt, a);
    }
  }
  for (; b < b1; b += kStep) {  // the ragged end (every step when rows are unaligned)
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int64_t e0 = b + (u * 64 + lane) * PC;
      rz[u] = row_fetch<T>(zr, e0, b1, a.vec != 0);
      rt[u] = row_fetch<T>(tr, e0, b1, a.vec != 0);
    }
    rowstats_step<T, Z1, REV, T1>(r, rz, rt, a);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    RowRun o;
    o.mz = __shfl_xor(r.mz, off);
    o.mt = __shfl_xor(r.mt, off);
    o.sz1 = __shfl_xor(r.sz1, off);
    o.szT = __shfl_xor(r.szT, off);
    o.ar = __shfl_xor(r.ar, off);
    o.stT = __shfl_xor(r.stT, off);
    o.at = __shfl_xor(r.at, off);
    o.st1 = __shfl_xor(r.st1, off);
    row_fold(r, o, a.cT, a.cTt);
  }
  if (lane == 0) {
    const int64_t n = (int64_t)a.n_slices * a.n;  // field stride
    float* p = a.rec + (int64_t)sl * a.n + i;
    p[0 * n] = r.mz * kLog2e;  p[1 * n] = r.sz1;
    p[2 * n] = r.mz * a.cT;    p[3 * n] = r.szT;
    p[4 * n] = r.mt * a.cTt;   p[5 * n] = r.stT;
    p[6 * n] = r.at;
    p[7 * n] = r.mt * kLog2e;  p[8 * n] = r.st1;
    p[9 * n] = r.ar;
  }
}

// Per-row constants of the logit gradient.
struct RowGrad {
  float cs, ckf, ckr;         // CE, forward-KL and reverse-KL coefficients
  float L1, LzT, LtT;         // log2-unit lse of z, z/T_s, t/T_t
  float k1;                   // T_s == 2: P(z) = P_T(z)^2 * k1
  float rev0, invT;
  int64_t y;                  // label (or out of range)
};

// d loss / d z of chunk elements [e0, e0 + PC): the dz formula of bwd_dz.
// CE says whether the student CE term is present (Z1 as for the forward
// step: how its P(z) comes), REV whether a reverse-direction KL term is.
template <typename T, bool CE, int Z1, bool REV>
__device__ __forceinline__ void logits_grad_chunk(const uint4& rz, const uint4& rt, int64_t e0,
                                                  const RowGrad& g, const RowArgs& a,
                                                  float (&o)[Elem<T>::kPerChunk]) {
  constexpr int PC = Elem<T>::kPerChunk;
  float z[PC], t[PC];
  row_unpack<T>(rz, z);
  row_unpack<T>(rt, t);
  const int64_t yl = g.y - e0;  // the label's place in the chunk (if in it)
#pragma unroll
  for (int j = 0; j < PC; ++j) {
    const float pz = exp2_fast(fmaf(z[j], a.cT, -g.LzT));  // P_T(z)
    const float pt = exp2_fast(fmaf(t[j], a.cTt, -g.LtT));
    float dv = fmaf(g.ckf, pz - pt, 0.f);
    if constexpr (CE) {
      float p1;
      if constexpr (Z1 == kZ1Square) p1 = pz * pz * g.k1;
      else if constexpr (Z1 == kZ1Same) p1 = pz;
      else p1 = exp2_fast(fmaf(z[j], kLog2e, -g.L1));
      dv = fmaf(g.cs, p1 - (yl == j ? 1.f : 0.f), dv);
    }
    // (a row of weight 0 skips it: its factor may be infinite)
    if constexpr (REV) {
      if (g.ckr != 0.f) dv = fmaf(g.ckr * pz, fmaf(fmaf(t[j], -a.rho, z[j]), g.invT, g.rev0), dv);
    }
    o[j] = dv;
  }
}

template <typename T>
__device__ __forceinline__ uint4 row_pack(const float (&x)[Elem<T>::kPerChunk]) {
  constexpr int PC = Elem<T>::kPerChunk;
  uint4 u;
  if constexpr (sizeof(T) == 2) {
    uint32_t* w32 = reinterpret_cast<uint32_t*>(&u);
#pragma unroll
    for (int j = 0; j < PC / 2; ++j) w32[j] = bf16x2_rne(x[2 * j], x[2 * j + 1]);
  } else {
    float* q = reinterpret_cast<float*>(&u);
#pragma unroll
    for (int j = 0; j < PC; ++j) q[j] = x[j];
  }
  return u;
}

// d loss / d z for given student logits, one slice of a row per wave, stored
// in the logits dtype (or added to what the output holds).
template <typename T, bool CE, int Z1, bool REV>
__global__ __launch_bounds__(kThreads) void logits_bwd_kernel(RowArgs a) {
  constexpr int PC = Elem<T>::kPerChunk;
  constexpr int64_t kStep = kRowUnroll * 64 * PC;
  const int lane = threadIdx.x & 63;
  int64_t i, b0, b1;
  int sl;
  if (!row_wave(a, i, sl, b0, b1)) return;
  const T* zr = static_cast<const T*>(a.zl) + i * a.v;
  const T* tr = static_cast<const T*>(a.tl) + i * a.v;
  T* out = static_cast<T*>(a.dz) + i * a.v;
  const float4 sv = reinterpret_cast<const float4*>(a.saved)[i];
  const float den = a.saved[4 * a.n];
  const float gl = a.grad ? *a.grad : 1.f;
  RowGrad g;
  g.y = a.labels ? a.labels[i] : a.ignore;
  const bool valid = a.labels == nullptr || (g.y != a.ignore && g.y >= 0 && g.y < a.v);
  const float coef = valid ? gl / den : 0.f;
  const float ck = coef * a.wkl * a.T;
  g.cs = coef * a.ws;
  g.ckf = (a.kl != KD_KL_REVERSE) ? ck : 0.f;
  g.ckr = (a.kl != KD_KL_FORWARD) ? ck : 0.f;
  g.L1 = sv.x * kLog2e;
  g.LzT = sv.y * kLog2e;
  g.LtT = sv.z * kLog2e;
  g.k1 = exp2_fast(2.f * g.LzT - g.L1);
  g.rev0 = sv.z - sv.y - sv.w;
  g.invT = 1.f / a.T;
  int64_t b = b0;
  uint4 rz[kRowUnroll], rt[kRowUnroll];
  if (a.vec) {  // whole steps: plain 16-byte loads and stores
    for (; b + kStep <= b1; b += kStep) {
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        const int64_t e0 = b + (u * 64 + lane) * PC;
        rz[u] = load_stream(zr + e0);
        rt[u] = load_stream(tr + e0);
      }
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        const int64_t e0 = b + (u * 64 + lane) * PC;
        float o[PC];
        logits_grad_chunk<T, CE, Z1, REV>(rz[u], rt[u], e0, g, a, o);
        if (a.accumulate) {
          float prev[PC];
          row_unpack<T>(load_stream(out + e0), prev);
#pragma unroll
          for (int j = 0; j < PC; ++j) o[j] += prev[j];
        }
        *reinterpret_cast<uint4*>(out + e0) = row_pack<T>(o);
      }
    }
  }
  for (; b < b1; b += kStep) {  // the ragged end (every step when rows are unaligned)
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int64_t e0 = b + (u * 64 + lane) * PC;
      rz[u] = row_fetch<T>(zr, e0, b1, a.vec != 0);
      rt[u] = row_fetch<T>(tr, e0, b1, a.vec != 0);
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int64_t e0 = b + (u * 64 + lane) * PC;
      float o[PC];
      logits_grad_chunk<T, CE, Z1, REV>(rz[u], rt[u], e0, g, a, o);
      if (a.vec && e0 + PC <= b1) {
        if (a.accumulate) {
          float prev[PC];
          row_unpack<T>(load_stream(out + e0), prev);
#pragma unroll
          for (int j = 0; j < PC; ++j) o[j] += prev[j];
        }
        *reinterpret_cast<uint4*>(out + e0) = row_pack<T>(o);
      } else {
#pragma unroll
        for (int j = 0; j < PC; ++j) {
          if (e0 + j < b1) {
            const float prev = a.accumulate ? to_f32(out[e0 + j]) : 0.f;
            if constexpr (sizeof(T) == 2) out[e0 + j] = bf16_rne(prev + o[j]);
            else out[e0 + j] = prev + o[j];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Merge: per-token outputs, saved statistics, per-block partial sums
// ---------------------------------------------------------------------------

struct MergeArgs {
  const float* rec;
  const float* prep;
  int n_slices;
  const float* prior;  // non-null: the running record of the earlier chunks ([kRecFields][n])
  int64_t n;
  int mode;
  float T;
  int need_zT, need_t1, teacher_ce;
  int kl;             // KD_KL_*
  int kl_unscaled;    // the per-token kl output without T^2
  float ws, wt, wkl;
  float* out_sce;
  float* out_tce;
  float* out_kl;
  float* saved;       // [n][4] or null: lse(z), lse(z/T), lse(t/T), M (top-K) or KL(P_S||P_T)
  double* partials;   // [blocks][4]: loss sum, valid count, bad count, 0
  const int32_t* pos; // compacted rows: record column of row i, -1 = left out; null = i
};

// A workgroup takes kMergeTok tokens; thread (token tl, group sg) folds the
// records of tiles sg, sg + kMergeGroups, ... in order, then the group
// partials are folded in the order sg = 0, 1, ... (deterministic).
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
  constexpr int kGroups = kMergeThreads / kMergeTok;
  __shared__ float part[kRecFields][kGroups][kMergeTok];
  __shared__ double red[3][kMergeTok];
  const int tid = threadIdx.x, tl = tid % kMergeTok, sg = tid / kMergeTok;
  const int64_t i = (int64_t)blockIdx.x * kMergeTok + tl;
  const bool live = i < a.n;
  // record column of this row: its compacted position, or -1 for a row the
  // compacted tiles left out (its label is ignored)
  const int64_t col = (live && a.pos) ? a.pos[i] : i;
  const bool has = live && col >= 0;
  RowStats s;
  stats_init(s);
  if (has) {
    if (sg == 0 && a.prior) rec_load(a.prior + col, a.n, s);
    const int64_t stride = (int64_t)a.n_slices * a.n;
    for (int sl = sg; sl < a.n_slices; sl += kGroups) {
      RowStats o;
      rec_load(a.rec + (int64_t)sl * a.n + col, stride, o);
      stats_merge(s, o);
    }
  }
  part[0][sg][tl] = s.mz1; part[1][sg][tl] = s.sz1; part[2][sg][tl] = s.mzT;
  part[3][sg][tl] = s.szT; part[4][sg][tl] = s.mtT; part[5][sg][tl] = s.stT;
  part[6][sg][tl] = s.a;   part[7][sg][tl] = s.mt1; part[8][sg][tl] = s.st1;
  part[9][sg][tl] = s.ar;
  __syncthreads();
  if (sg == 0) {
    for (int q = 1; q < kGroups; ++q) {
      RowStats o;
      o.mz1 = part[0][q][tl]; o.sz1 = part[1][q][tl]; o.mzT = part[2][q][tl];
      o.szT = part[3][q][tl]; o.mtT = part[4][q][tl]; o.stT = part[5][q][tl];
      o.a = part[6][q][tl];   o.mt1 = part[7][q][tl]; o.st1 = part[8][q][tl];
      o.ar = part[9][q][tl];
      stats_merge(s, o);
    }
    double contrib = 0.0, cnt = 0.0, bad = 0.0;
    if (live && !has) {
      // left out by the compaction: an ignored label, excluded from CE and KL
      bad = (a.prep[3 * a.n + i] == 2.f) ? 1.0 : 0.0;
      if (a.out_sce) a.out_sce[i] = 0.f;
      if (a.out_tce) a.out_tce[i] = 0.f;
      if (a.out_kl) a.out_kl[i] = 0.f;
      if (a.saved) {
        reinterpret_cast<float4*>(a.saved)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        a.saved[4 * a.n + kSavedHeaderBytes / 4 + i] = 0.f;
      }
    } else if (live) {
      const float lz1 = kLn2 * (s.mz1 + log2f(s.sz1));
      const float lzT = a.need_zT ? kLn2 * (s.mzT + log2f(s.szT)) : lz1;
      const float f0 = a.prep[i], f1 = a.prep[a.n + i], f2 = a.prep[2 * a.n + i];
      const float flag = a.prep[3 * a.n + i];
      float sce = 0.f, tce = 0.f, kl, kl_raw, ltT = 0.f, mass = 0.f, lt1 = 0.f;
      bool valid;
      if (a.mode == MODE_TOPK) {
        // sum p log p - sum p z[idx] + M lse(z); the cross term is the sum of
        // the tiles' record field 6
        kl = f1 - s.a + f2 * lz1;
        kl_raw = kl;  // T = 1
        mass = f2;
        valid = true;
      } else {
        ltT = kLn2 * (s.mtT + log2f(s.stT));
        lt1 = a.need_t1 ? kLn2 * (s.mt1 + log2f(s.st1)) : ltT;
        // KL(P_T || P_S) = E_{P_T}[(t - z) / T] - lse(t/T) + lse(z/T), and
        // KL(P_S || P_T) = E_{P_S}[(z - t) / T] - lse(z/T) + lse(t/T)
        // (orda-kernel, KL variants: forward, reverse, jeffreys = their sum).
        const float kl_f = s.a / (s.stT * a.T) - ltT + lzT;
        const float kl_r = (a.kl != KD_KL_FORWARD) ? s.ar / (s.szT * a.T) - lzT + ltT : 0.f;
        kl_raw = (a.kl != KD_KL_REVERSE ? kl_f : 0.f) + kl_r;
        kl = a.T * a.T * kl_raw;
        mass = kl_r;  // the reverse-direction gradient needs this row's KL(P_S || P_T)
        valid = flag == 1.f;
        sce = valid ? lz1 - f0 : 0.f;
        tce = (valid && a.teacher_ce) ? lt1 - f1 : 0.f;
      }
      bad = (flag == 2.f) ? 1.0 : 0.0;
      cnt = valid ? 1.0 : 0.0;
      // A term of weight 0 is left out, not multiplied: its value may be
      // infinite (a teacher CE at a label whose teacher logit is -inf).
      if (valid) {
        if (a.ws != 0.f) contrib += (double)a.ws * sce;
        if (a.wt != 0.f) contrib += (double)a.wt * tce;
        if (a.wkl != 0.f) contrib += (double)a.wkl * kl;
      }
      if (a.out_sce) a.out_sce[i] = sce;
      if (a.out_tce) a.out_tce[i] = tce;
      if (a.out_kl) a.out_kl[i] = a.kl_unscaled ? kl_raw : kl;
      if (a.saved) {
        float4 sv = make_float4(lz1, lzT, ltT, mass);
        reinterpret_cast<float4*>(a.saved)[i] = sv;
        a.saved[4 * a.n + kSavedHeaderBytes / 4 + i] = lt1;  // lse(t) at T = 1
      }
    }
    red[0][tl] = contrib;
    red[1][tl] = cnt;
    red[2][tl] = bad;
  }
  __syncthreads();
  if (tid == 0) {
    double t0 = 0.0, t1 = 0.0, t2 = 0.0;
    for (int q = 0; q < kMergeTok; ++q) {
      t0 += red[0][q];
      t1 += red[1][q];
      t2 += red[2][q];
    }
    double* p = a.partials + (int64_t)blockIdx.x * 4;
    p[0] = t0;
    p[1] = t1;
    p[2] = t2;
    p[3] = 0.0;
  }
}

// One vocabulary chunk's records folded into the running record (the first
// chunk starts it). Laid out like the merge: 16 tokens per workgroup, 16
// groups of slices; group 0 starts from the running record, each group adds
// its slices in order, then the groups in order.
struct FoldArgs {
  const float* rec;  // [kRecFields][n_slices][n]
  int n_slices;
  float* run;        // [kRecFields][n]
  int64_t n;
  int first;
};

__global__ __launch_bounds__(kMergeThreads) void fold_kernel(FoldArgs a) {
  constexpr int kGroups = kMergeThreads / kMergeTok;
  __shared__ RowStats part[kGroups][kMergeTok];
  const int tid = threadIdx.x, tl = tid % kMergeTok, sg = tid / kMergeTok;
  const int64_t i = (int64_t)blockIdx.x * kMergeTok + tl;
  RowStats s;
  stats_init(s);
  if (i < a.n) {
    if (sg == 0 && !a.first) rec_load(a.run + i, a.n, s);
    const int64_t stride = (int64_t)a.n_slices * a.n;
    for (int sl = sg; sl < a.n_slices; sl += kGroups) {
      RowStats o;
      rec_load(a.rec + (int64_t)sl * a.n + i, stride, o);
      stats_merge(s, o);
    }
  }
  part[sg][tl] = s;
  __syncthreads();
  if (sg == 0 && i < a.n) {
    for (int q = 1; q < kGroups; ++q) stats_merge(s, part[q][tl]);
    rec_store(a.run + i, a.n, s);
  }
}

struct FinalArgs {
  const double* partials;
  int blocks;
  float normalizer;
  int reduction;
  float* loss;       // nullable
  float* saved_hdr;  // nullable: [den, n_valid, n_bad, 0], then the kept layout
  int32_t* status;   // workspace flag word
  int32_t keep_tag[5];  // kKeepMagic (or 0 when nothing was kept), chunk, keep_ld, keep_ops, n
};

__global__ __launch_bounds__(kThreads) void finalize_kernel(FinalArgs a) {
  __shared__ double red[3][kThreads];
  const int tid = threadIdx.x;
  double s0 = 0.0, s1 = 0.0, s2 = 0.0;
  for (int b = tid; b < a.blocks; b += kThreads) {
    s0 += a.partials[b * 4 + 0];
    s1 += a.partials[b * 4 + 1];
    s2 += a.partials[b * 4 + 2];
  }
  red[0][tid] = s0;
  red[1][tid] = s1;
  red[2][tid] = s2;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (tid < off) {
      red[0][tid] += red[0][tid + off];
      red[1][tid] += red[1][tid + off];
      red[2][tid] += red[2][tid + off];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const double total = red[0][0], n_valid = red[1][0], n_bad = red[2][0];
    double den;
    if (a.normalizer > 0.f) den = a.normalizer;
    else if (a.reduction == KD_REDUCE_MEAN) den = n_valid > 1.0 ? n_valid : 1.0;
    else den = 1.0;
    if (a.loss) *a.loss = (float)(total / den);
    if (a.saved_hdr) {
      a.saved_hdr[0] = (float)den;
      a.saved_hdr[1] = (float)n_valid;
      a.saved_hdr[2] = (float)n_bad;
      a.saved_hdr[3] = 0.f;
      int32_t* tag = reinterpret_cast<int32_t*>(a.saved_hdr) + kHdrKeep;
      for (int j = 0; j < 5; ++j) tag[j] = a.keep_tag[j];
    }
    a.status[0] = n_bad > 0.0 ? kFlagRange : 0;
  }
}

// ---------------------------------------------------------------------------
// Backward: recompute a chunk and write the logit-gradient slab
// ---------------------------------------------------------------------------

struct BwdArgs {
  const void* hs;
  const void* w;
  const void* ht;
  const void* wt;
  const void* tlogits;    // teacher logits (TLOGITS)
  int64_t n, d, dt, v;
  const int64_t* labels;
  int64_t ignore;
  const float* saved;     // [n][4] + header at 16 n bytes
  const float* grad;      // device scalar or null
  float ws, wkl, T, cT;
  float cTt, rho;         // log2(e) / T_t, T_s / T_t
  float wtce;             // teacher-CE weight (MODE_TCE)
  int need_zT;
  int kl;                 // KD_KL_*
  int vec;                // teacher logits: given_mode (3 / 4 registers, 1 / 0 after the loop)
  int sqz;                // T_s == 2: softmax(z) is the square of one exponential of z/T
  const int32_t* idx;     // compacted rows: original row of each (null: rows are original)
  const int32_t* nv;      // compacted rows: their number
  int64_t c0;             // first vocabulary row of the chunk
  int n_vt, n_ttiles;     // tiles of the chunk
  void* dz;               // [dz_rows][ldz]
  int64_t ldz;
  int64_t dz_rows;        // n rounded up to the token tile; rows past n are written as 0
  // kept products of this chunk (the forward's last) in register order, the
  // teacher's keep_t elements after the student's
  const float* keep;
  int64_t keep_t;
  // the layout the kept products must have (header words kHdrKeep.. of saved)
  int32_t keep_tag[5];
  // top-K: each row's entries sorted by index and where each tile of this
  // chunk starts its run of them ([n][n_vt + 1]); the epilogue subtracts p
  const int32_t* tk_sidx;
  const float* tk_sprob;
  const int32_t* tk_off;
  int k;
  // workspace flag word: the chunk's first launch and the kept launch set it
  // (kFlagSaved when the kept products are not of the expected layout)
  int32_t* status;
  int set_status;
};

template <typename T>
__device__ __forceinline__ void store4(T* p, float x0, float x1, float x2, float x3);
template <>
__device__ __forceinline__ void store4<float>(float* p, float x0, float x1, float x2, float x3) {
  *reinterpret_cast<float4*>(p) = make_float4(x0, x1, x2, x3);
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float x0, float x1, float x2, float x3) {
  uint2 u;
  u.x = bf16x2_rne(x0, x1);
  u.y = bf16x2_rne(x2, x3);
  *reinterpret_cast<uint2*>(p) = u;
}

// kKept: the products are the forward's kept ones (a.keep), read instead of
// recomputed; the tile runs no main loop and needs no LDS.
template <typename T, int MODE, class G, bool kKept>
__global__ __launch_bounds__(G::kThreads, kKept ? 4 : 2) void bwd_dz_kernel(BwdArgs a) {
  constexpr int NB = (MODE == MODE_TIED) ? 2 : 1;
  constexpr int NBT = G::kNB;  // token blocks of 16 per wave
  using Acc = f32x4[kMB][NBT];
  constexpr bool kGiven = MODE == MODE_TLOGITS;
  constexpr int kMainBytes = G::template lds_bytes<NB>();
  constexpr bool kGivenRegs = kGiven && G::kPipe;  // a given logits tile in registers
  constexpr bool kKeptT = kKept && (MODE == MODE_TIED || MODE == MODE_SEPARATE);  // teacher's kept too
  __shared__ __attribute__((aligned(16))) uint8_t lds[kKept ? 16 : kMainBytes];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  // Compacted rows: token tiles from round_up(nv, 128) on would hold only zero
  // rows, which no GEMM reads (their K and M stop at nv); only the tiles below
  // are mapped, onto the first blocks of every XCD.
  const int64_t n_live = a.nv ? *a.nv : a.n;
  const int n_tt = a.nv ? (int)((n_live + G::kTT - 1) / G::kTT) : a.n_ttiles;
  int t;
  if (!xcd_live_tile(blockIdx.x, a.n_vt * n_tt, t)) return;
  int vt, tt;
  grouped_tile(t, a.n_vt, n_tt, tile_group(G::kVT, G::kTT), vt, tt);
  const int64_t v0 = a.c0 + (int64_t)vt * G::kVT;
  const int64_t t0 = (int64_t)tt * G::kTT;
  const T* hs = static_cast<const T*>(a.hs);
  const T* W = static_cast<const T*>(a.w);
  const T* ht = static_cast<const T*>(a.ht);
  const T* Wt = static_cast<const T*>(a.wt);
  // Kept products are read only if the forward that wrote `saved` kept them
  // in this layout (its header says so); otherwise every dz of the chunk is
  // NaN and the flag is raised, so the gradients cannot be silently wrong.
  bool kept_ok = true;
  if constexpr (kKept) {
    const int32_t* tag = reinterpret_cast<const int32_t*>(a.saved + 4 * a.n) + kHdrKeep;
#pragma unroll
    for (int j = 0; j < 5; ++j) kept_ok = kept_ok && tag[j] == a.keep_tag[j];
  }
  if (a.set_status && blockIdx.x == 0 && tid == 0) a.status[0] = kept_ok ? 0 : kFlagSaved;

  f32x4 acc[NB][kMB][NBT];
  f32x4 tacc[1][kMB][NBT];
  // a given teacher tile (pipelined: 256-token tiles) is kept packed and
  // unpacked at each use
  static_assert(!kGivenRegs || G::kTT > 128, "pipelined given tiles are 256-token tiles");
  constexpr bool kPackedT = kGivenRegs;
  GivenRawT<NBT> traw;
  if constexpr (kKept) {
    // the kept products are read per token block in the epilogue; a given
    // teacher tile is loaded here as in the recomputing tiles
    if constexpr (MODE == MODE_TLOGITS) {
      const T* L = static_cast<const T*>(a.tlogits);
      if constexpr (kPackedT) {
        given_raw_load<G>(reinterpret_cast<const bf16_t*>(L), a.n, a.v, t0, v0, wm, wn, lane, a.vec == 3, traw);
      } else {
        given_tile<T>(L, a.n, a.v, t0, v0, a.vec, wm, wn, lane, tacc[0]);
      }
    }
  } else if constexpr (MODE == MODE_TIED) {
    const T* const b[2] = {hs, ht};
    tile_product<T, G, 2>(W, a.d, a.v, b, a.d, a.n, v0, t0, a.d, lds, acc, tid);
  } else if constexpr (MODE == MODE_SEPARATE) {
    const T* const b[1] = {hs};
    tile_product<T, G, 1>(W, a.d, a.v, b, a.d, a.n, v0, t0, a.d, lds, acc, tid);
    const T* const bt[1] = {ht};
    tile_product<T, G, 1>(Wt, a.dt, a.v, bt, a.dt, a.n, v0, t0, a.dt, lds, tacc, tid);
  } else if constexpr (MODE == MODE_TLOGITS) {
    const T* L = static_cast<const T*>(a.tlogits);
    const T* const b[1] = {hs};
    if constexpr (kPackedT) {
      // the teacher tile, still packed, after the main loop
      tile_product<T, G, 1>(W, a.d, a.v, b, a.d, a.n, v0, t0, a.d, lds, acc, tid);
      given_raw_load<G>(reinterpret_cast<const bf16_t*>(L), a.n, a.v, t0, v0, wm, wn, lane, a.vec == 3, traw);
    } else {
      tile_product<T, G, 1>(W, a.d, a.v, b, a.d, a.n, v0, t0, a.d, lds, acc, tid);
      given_tile<T>(L, a.n, a.v, t0, v0, a.vec, wm, wn, lane, tacc[0]);
    }
  } else if constexpr (MODE == MODE_TCE) {  // the teacher tile alone
    const T* const bt[1] = {ht};
    tile_product<T, G, 1>(Wt, a.dt, a.v, bt, a.dt, a.n, v0, t0, a.dt, lds, acc, tid);
  } else {  // MODE_TOPK
    const T* const b[1] = {hs};
    tile_product<T, G, 1>(W, a.d, a.v, b, a.d, a.n, v0, t0, a.d, lds, acc, tid);
  }
  const Acc& z = acc[0];  // MODE_TCE: the teacher logits
  const Acc& tl_acc = (MODE == MODE_TIED) ? acc[NB - 1] : tacc[0];
  const auto tl = [&]() {
    if constexpr (kPackedT) return view(traw);
    else return view(tl_acc);
  }();

  // Pipelined bf16 tiles stage the dz tile in the (free) LDS and write whole
  // token rows of it (512 contiguous bytes) instead of 32-byte pieces.
  constexpr bool kStage = G::kPipe && !kKept && std::is_same<T, bf16_t>::value;
  const float* hdr = a.saved + 4 * a.n;
  const float den = hdr[0];
  const float g = a.grad ? *a.grad : 1.f;
  T* dz = static_cast<T*>(a.dz);

  // The reverse-direction term is compiled only into the variant that uses it,
  // so the forward-KL epilogue carries no extra arithmetic.
  // kSq (T_s = 2): e = 2^(z log2(e)/2 - L1/2) gives softmax(z) = e^2 and
  // softmax(z/2) = e 2^(L1/2 - LzT): one exponential of z per element, not two.
  // Vocabulary row of register (mb, r) is v0 + rb + 16 mb + r: the label test
  // and the vocabulary bound become 32-bit compares against constants.
  const int rb = acc_row(wm, 0, 0, lane);
  const int lim = (int)min(a.v - v0 - rb, (int64_t)1 << 30);  // rows k >= lim are past v
  // One token's inputs, read from indices that are always valid (a row that is
  // not live reads row 0, then reads as zero), so that no load is conditional.
  struct TokIn {
    float4 sv;   // saved statistics
    float l1;    // MODE_TCE: the teacher's log-normaliser at T = 1
    int64_t y;   // label, -1 without labels
    int j0, j1;  // top-K: this token's run of entries in the tile
  };
  auto tok_inputs = [&](int nb) {
    TokIn r;
    const int64_t tok = t0 + G::col(wn, nb, lane);
    const bool live = tok < n_live;
    const int64_t tc = live ? tok : 0;
    // (idx[0] may be unwritten when no row is usable: only a live row's entry is used)
    const int64_t ix = a.idx ? (int64_t)a.idx[tc] : tc;
    const int64_t orig = live ? ix : 0;  // original row
    const float4 s4 = reinterpret_cast<const float4*>(a.saved)[orig];
    r.sv = live ? s4 : make_float4(0.f, 0.f, 0.f, 0.f);
    r.l1 = 0.f;
    r.y = -1;
    r.j0 = r.j1 = 0;
    if constexpr (MODE == MODE_TCE) {
      const float x = a.saved[4 * a.n + kSavedHeaderBytes / 4 + orig];
      r.l1 = live ? x : 0.f;
    }
    if constexpr (MODE != MODE_TOPK) {
      const int64_t yy = a.labels ? a.labels[orig] : -1;
      r.y = live ? yy : -1;
    }
    if constexpr (MODE == MODE_TOPK) {
      const int32_t* off = a.tk_off + tc * (int64_t)(a.n_vt + 1) + vt;
      const int o0 = off[0], o1 = off[1];
      r.j0 = live ? o0 : 0;
      r.j1 = live ? o1 : 0;
    }
    return r;
  };
  // All token blocks' inputs are loaded before any is used, so that their
  // latencies overlap instead of adding up block by block. The tiles that hold
  // a packed teacher tile, and the kept-product tiles (four waves per SIMD),
  // have no registers to spare and load per block.
  constexpr bool kPreload = !kPackedT && !kKept;
  TokIn pre[kPreload ? NBT : 1];
  if constexpr (kPreload) {
#pragma unroll
    for (int nb = 0; nb < NBT; ++nb) pre[nb] = tok_inputs(nb);
  }
  auto epilogue = [&](auto rev_tag, auto sq_tag) {
  // No implicit multiply-add contraction here: which products the compiler
  // fuses depends on the surrounding code, and the kept-product and recompute
  // instantiations must round every value alike (every fusion meant is an
  // explicit fmaf).
#pragma clang fp contract(off)
  constexpr bool kRev = decltype(rev_tag)::value;
  constexpr bool kSq = decltype(sq_tag)::value;
#pragma unroll
  for (int nb = 0; nb < NBT; ++nb) {
    const int64_t tok = t0 + G::col(wn, nb, lane);
    if (tok >= a.dz_rows) continue;
    const bool live = tok < n_live;  // rows past n (or nv) are zero padding of the slab
    const TokIn ti = kPreload ? pre[kPreload ? nb : 0] : tok_inputs(nb);
    const float4 sv = ti.sv;
    // MODE_TCE: the softmax at T = 1 is the teacher's
    const float L1 = (MODE == MODE_TCE ? ti.l1 : sv.x) * kLog2e;
    const float LzT = sv.y * kLog2e, LtT = sv.z * kLog2e, mass = sv.w;
    const float L1h = 0.5f * L1;
    const float kz = kSq ? exp2_fast(L1h - LzT) : 0.f;
    int64_t y = -1;
    bool valid = live;
    if (live && MODE != MODE_TOPK && a.labels) {
      y = ti.y;
      valid = y != a.ignore && y >= 0 && y < a.v;
    }
    // coef = 0 zeroes every term of a row that is not valid (all are finite)
    const float coef = valid ? g / den : 0.f;
    const int yl = valid ? (int)(y - v0 - rb) : INT_MIN;  // the label's register index
    const float cs = coef * (MODE == MODE_TCE ? a.wtce : a.ws);  // student (teacher) CE
    const float ck = coef * a.wkl * a.T;     // T^2 KL -> T (P_S - P_T)
    const float cm = coef * a.wkl * mass;    // top-K: M softmax(z)
    // T^2 KL(P_S || P_T) -> T P_S (log P_S - log P_T - KL(P_S || P_T)); with
    // log P_S - log P_T = (z - t rho) / T - lse(z/T) + lse(t/T_t) (natural logs).
    const float ckf = (a.kl != KD_KL_REVERSE) ? ck : 0.f;
    const float ckr = ck;
    const float rev0 = sv.z - sv.y - mass;   // lse(t/T) - lse(z/T) - KL(P_S || P_T)
    const float invT = 1.f / a.T;
    T* row = dz + tok * a.ldz + (v0 - a.c0);
    // top-K: this token's run of index-sorted entries in this tile, whose p is
    // subtracted before the one rounding of dz (each index is distinct)
    int j0 = 0, j1 = 0;
    const int32_t* tix = nullptr;
    const float* tpr = nullptr;
    if constexpr (MODE == MODE_TOPK) {
      if (live) {
        j0 = ti.j0;
        j1 = ti.j1;
        tix = a.tk_sidx + tok * (int64_t)a.k;
        tpr = a.tk_sprob + tok * (int64_t)a.k;
      }
    }
    const float cp = coef * a.wkl;           // top-K: the p term
    // kept products of this token block: the student's (MODE_TCE: the
    // teacher's) and, for a TIED or SEPARATE teacher, the teacher's
    f32x4 zk[kMB], tk[kMB];
    if constexpr (kKept) {
      const int64_t tile = (int64_t)tt * a.n_vt + vt;
      constexpr int kWaves = G::kThreads / 64;
      kept_load<NBT>(a.keep + (MODE == MODE_TCE ? a.keep_t : 0), tile, kWaves, w, lane, nb, live, zk);
      if constexpr (kKeptT) kept_load<NBT>(a.keep + a.keep_t, tile, kWaves, w, lane, nb, live, tk);
    }
    // o[mb][r]: this token's dz at vocabulary row v0 + rb + 16 mb + r
    float o[kMB][4];
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      // registers r = 0..3 are four consecutive vocabulary rows
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int k = mb * 16 + r;
        float zz;
        if constexpr (kKept) zz = zk[mb][r];
        else zz = z[mb][nb][r];
        float p1, pz;
        if constexpr (kSq) {
          const float e = exp2_fast(fmaf(zz, a.cT, -L1h));
          p1 = e * e;
          pz = e * kz;
        } else {
          p1 = exp2_fast(fmaf(zz, kLog2e, -L1));
          pz = a.need_zT ? exp2_fast(fmaf(zz, a.cT, -LzT)) : p1;
        }
        float dv;
        if (MODE == MODE_TOPK) {
          dv = cm * p1;
        } else if (MODE == MODE_TCE) {
          dv = cs * (p1 - (yl == k ? 1.f : 0.f));
        } else {
          dv = cs * (p1 - (yl == k ? 1.f : 0.f));
          float tt;
          if constexpr (kKeptT) tt = tk[mb][r];
          else tt = tl(mb, nb, r);
          const float pt = exp2_fast(fmaf(tt, a.cTt, -LtT));
          dv = fmaf(ckf, pz - pt, dv);
          if constexpr (kRev) dv = fmaf(ckr * pz, fmaf(fmaf(tt, -a.rho, zz), invT, rev0), dv);
        }
        o[mb][r] = (k < lim) ? dv : 0.f;
      }
    }
    if constexpr (MODE == MODE_TOPK) {
      // the token's entries in this tile, each read once: the one at row
      // v0 + rb + 16 mb + r (if this lane holds it) subtracts its p term
      const int base = (int)(v0 + rb);
      for (int j = j0; j < j1; ++j) {
        const int d = tix[j] - base;
        const float q = cp * tpr[j];
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[mb][r] -= (d == 16 * mb + r) ? q : 0.f;
      }
    }
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      if constexpr (kKept) {
        if (!kept_ok) o[mb][0] = o[mb][1] = o[mb][2] = o[mb][3] = __builtin_nanf("");
      }
      if constexpr (kStage) {
        // into the LDS image of the tile: token-major rows of 256 bf16, the
        // 16-byte chunk index XOR-ed with the token's low bits
        const int tl = (int)(tok - t0);
        const int vl = rb + 16 * mb;
        uint2 u;
        u.x = bf16x2_rne(o[mb][0], o[mb][1]);
        u.y = bf16x2_rne(o[mb][2], o[mb][3]);
        *reinterpret_cast<uint2*>(lds + tl * 512 + (((vl >> 3) ^ (tl & 31)) << 4) + (vl & 7) * 2) = u;
      } else {
        store4<T>(row + acc_row(wm, mb, 0, lane), o[mb][0], o[mb][1], o[mb][2], o[mb][3]);
      }
    }
  }
  };
  constexpr bool kStudentKl = MODE != MODE_TOPK && MODE != MODE_TCE;
  if (kStudentKl && a.sqz) {
    if (a.kl != KD_KL_FORWARD) epilogue(std::true_type{}, std::true_type{});
    else epilogue(std::false_type{}, std::true_type{});
  } else {
    if (kStudentKl && a.kl != KD_KL_FORWARD) epilogue(std::true_type{}, std::false_type{});
    else epilogue(std::false_type{}, std::false_type{});
  }
  if constexpr (kStage) {
    static_assert(G::kTT * 512 <= kMainBytes, "the dz tile fits the main loop's LDS");
    __syncthreads();
    // two token rows per instruction: lanes 0-31 row tl, lanes 32-63 row tl + 1
    const int c = lane & 31;
#pragma unroll 4
    for (int pr = 2 * w; pr < G::kTT; pr += 2 * (G::kThreads / 64)) {
      const int tl = pr + (lane >> 5);
      const int64_t tok = t0 + tl;
      const uint4 v = *reinterpret_cast<const uint4*>(lds + tl * 512 + ((c ^ (tl & 31)) << 4));
      if (tok < a.dz_rows) *reinterpret_cast<uint4*>(dz + tok * a.ldz + (v0 - a.c0) + c * 8) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Compaction of the rows with a usable label (the others never enter the loss)
// ---------------------------------------------------------------------------

// idx[c] = the c-th row (in row order) whose label is usable, pos[i] = the
// compacted position of row i or -1, *nv = the number of such rows. One
// workgroup: thread t counts the rows of its segment, a workgroup scan of the
// counts gives each segment its first position, then the segment is written.
constexpr int kCompactThreads = 1024;
struct CompactArgs {
  const int64_t* labels;
  int64_t n, v, ignore;
  int32_t* idx;
  int32_t* pos;
  int32_t* nv;
};

__global__ __launch_bounds__(kCompactThreads) void compact_kernel(CompactArgs a) {
  __shared__ int32_t sc[kCompactThreads];
  const int t = threadIdx.x;
  const int64_t seg = (a.n + kCompactThreads - 1) / kCompactThreads;
  const int64_t r0 = min(a.n, (int64_t)t * seg), r1 = min(a.n, r0 + seg);
  auto usable = [&](int64_t i) {
    const int64_t y = a.labels[i];
    return y != a.ignore && y >= 0 && y < a.v;
  };
  int cnt = 0;
  for (int64_t i = r0; i < r1; ++i) cnt += usable(i) ? 1 : 0;
  sc[t] = cnt;
  __syncthreads();
  for (int off = 1; off < kCompactThreads; off <<= 1) {  // inclusive scan
    const int x = (t >= off) ? sc[t - off] : 0;
    __syncthreads();
    sc[t] += x;
    __syncthreads();
  }
  int c = sc[t] - cnt;
  for (int64_t i = r0; i < r1; ++i) {
    if (usable(i)) {
      a.idx[c] = (int32_t)i;
      a.pos[i] = c++;
    } else {
      a.pos[i] = -1;
    }
  }
  if (t == kCompactThreads - 1) *a.nv = sc[t];
}

// out[c, :] = in[idx[c], :] for c < nv and 0 for nv <= c < rows, in 16-byte
// pieces (row_bytes is a multiple of 16); one wave per row.
// Two matrices per launch (blockIdx.y selects one: student, teacher hidden).
struct GatherArgs {
  const uint8_t* in[2];
  uint8_t* out[2];
  int64_t row_bytes[2];
  const int32_t* idx;
  const int32_t* nv;
  int64_t rows;
};

__global__ __launch_bounds__(kThreads) void gather_rows_kernel(GatherArgs a) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.y;
  const int64_t c = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (c >= a.rows) return;
  const int64_t rb = a.row_bytes[m];
  uint4* dst = reinterpret_cast<uint4*>(a.out[m] + c * rb);
  const int64_t pieces = rb / 16;
  if (c < *a.nv) {
    const uint4* src = reinterpret_cast<const uint4*>(a.in[m] + (int64_t)a.idx[c] * rb);
    for (int64_t j = lane; j < pieces; j += 64) dst[j] = src[j];
  } else {
    for (int64_t j = lane; j < pieces; j += 64) dst[j] = make_uint4(0u, 0u, 0u, 0u);
  }
}

// m[0 .. cnt) = 0 (a fill kernel rather than a memset, so that a captured
// graph replays it like any other launch).
__global__ __launch_bounds__(kThreads) void fill_zero_kernel(float* m, int64_t cnt) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < cnt) m[i] = 0.f;
}

// Rows i with pos[i] < 0 (left out by the compaction) of a [n x d] matrix of
// `elem`-byte elements set to zero (d elem a multiple of 4); one wave per row.
__global__ __launch_bounds__(kThreads) void zero_rows_kernel(void* m, const int32_t* pos, int64_t n,
                                                              int64_t d, int elem) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (i >= n || pos[i] >= 0) return;
  const int64_t words = d * elem / 4;
  float* row = static_cast<float*>(m) + i * words;
  for (int64_t j = lane; j < words; j += 64) row[j] = 0.f;
}

// One element of a gradient output: the tile's value v, plus the fp32 partial
// of the earlier chunks (cadd, nullable), plus the old output (accumulate),
// stored as fp32 or rounded once to bf16.
__device__ __forceinline__ void store_grad(void* C, int out_bf16, const float* cadd, int accumulate,
                                           int64_t off, float v) {
  if (cadd) v += cadd[off];
  if (out_bf16) {
    bf16_t* p = static_cast<bf16_t*>(C) + off;
    if (accumulate) v += to_f32(*p);
    *p = bf16_rne(v);
  } else {
    float* p = static_cast<float*>(C) + off;
    *p = accumulate ? *p + v : v;
  }
}

// ---------------------------------------------------------------------------
// GEMM for dW and dH: C[M x N] (+)= sum_k A(m, k) B(n, k), fp32 output
// ---------------------------------------------------------------------------

template <typename T, bool AKC, bool BKC>
struct GemmArgs {
  Operand<T, AKC> A;
  Operand<T, BKC> B;
  void* C;             // fp32, or bf16 (out_bf16)
  int out_bf16;
  const float* cadd;   // nullable: an fp32 partial added to every element (same layout as C)
  int64_t ldc, M, N, K;
  int accumulate;
  int n_mt, n_nt;
  const int32_t* kdev;    // non-null: K = min(K, *kdev) (compacted token rows)
  const int32_t* mdev;    // non-null: M = min(M, *mdev)
  const int32_t* rowmap;  // non-null: C row m is stored at row rowmap[m]
};

template <typename T, bool AKC, bool BKC>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(GemmArgs<T, AKC, BKC> a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * 2 * kTileBytes];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  const int64_t M = a.mdev ? min(a.M, (int64_t)*a.mdev) : a.M;
  const int64_t K = a.kdev ? min(a.K, (int64_t)*a.kdev) : a.K;
  const int n_mt = a.mdev ? (int)((M + kTile - 1) / kTile) : a.n_mt;  // row tiles with work
  int t;
  if (!xcd_live_tile(blockIdx.x, n_mt * a.n_nt, t)) return;
  int mt, nt;
  grouped_tile(t, n_mt, a.n_nt, 8, mt, nt);
  const int64_t m0 = (int64_t)mt * kTile, n0 = (int64_t)nt * kTile;
  f32x4 acc[1][kMB][kNB];
  mainloop<T, AKC, BKC, 1>(a.A, &a.B, m0, n0, K, lds, acc, tid);
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      const int64_t col = n0 + acc_col(wn, nb, lane);
      if (col >= a.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + acc_row(wm, mb, r, lane);
        if (row < M) {
          const int64_t off = (a.rowmap ? (int64_t)a.rowmap[row] : row) * a.ldc + col;
          store_grad(a.C, a.out_bf16, a.cadd, a.accumulate, off, acc[0][mb][nb][r]);
        }
      }
    }
}

// Pipelined bf16 GEMM: C[M x N] (+)= sum_k A(m, k) B(n, k), fp32 output, tile
// 256 x BN, 8 waves, three A slots and two B slots (four for BN = 128). A / B
// are K-contiguous or row-contiguous; K is a multiple of 64 and both operands
// are zero (or read as zero) past their own K extent.
template <bool AKC, bool BKC, int BN>
struct GemmPipeArgs {
  std::conditional_t<AKC, PipeOperand, PipeOperandMN> A;
  std::conditional_t<BKC, PipeOperand, PipeOperandMN> B;
  void* C;             // fp32, or bf16 (out_bf16)
  int out_bf16;
  const float* cadd;   // nullable: an fp32 partial added to every element (same layout as C)
  int64_t ldc, M, N, K;
  int accumulate;
  int n_mt, n_nt;
  const int32_t* kdev;    // non-null: K = min(K, round_up(*kdev, 64)) (compacted token rows)
  const int32_t* mdev;    // non-null: M = min(M, *mdev)
  const int32_t* rowmap;  // non-null: C row m is stored at row rowmap[m]
};

// M and K of a launch (compacted rows bound them from device memory) and the
// number of row tiles that have work.
template <bool AKC, bool BKC, int BN>
__device__ __forceinline__ void gemm_pipe_bounds(const GemmPipeArgs<AKC, BKC, BN>& a, int64_t& M,
                                                 int64_t& K, int& n_mt) {
  M = a.mdev ? min(a.M, (int64_t)*a.mdev) : a.M;
  K = a.kdev ? min(a.K, ((int64_t)*a.kdev + kPipeBK - 1) / kPipeBK * kPipeBK) : a.K;
  n_mt = a.mdev ? (int)((M + 255) / 256) : a.n_mt;
}

// Output tile (mt, nt) of the pipelined GEMM.
template <bool AKC, bool BKC, int BN>
__device__ __forceinline__ void gemm_pipe_tile(const GemmPipeArgs<AKC, BKC, BN>& a, int mt, int nt,
                                               int64_t M, int64_t K, uint8_t* lds, int tid) {
  using C = PipeCfg<256, BN, 1, AKC, BKC>;
  const int lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  const int64_t m0 = (int64_t)mt * 256, n0 = (int64_t)nt * BN;
  f32x4 acc[1][C::MB][C::NBK];
  pipe_mainloop<C, 1>(a.A, &a.B, m0, n0, K, lds, acc, tid);
  // output row of each of this lane's MB x 4 accumulator rows
  int64_t orow[C::MB][4];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = m0 + pipe_row<C>(wm, mb, r, lane);
      orow[mb][r] = (row >= M) ? -1 : (a.rowmap ? (int64_t)a.rowmap[row] : row);
    }
  // One 16-row block at a time: the values added to it (the fp32 partial cadd,
  // the output being accumulated) are all loaded before any of the block is
  // stored, from offsets that are always valid (an element past M or N reads
  // element 0 and is not stored), so that their latencies overlap; per element,
  // the loads would wait one after another behind the stores before them. The
  // three options are compile-time in each variant, so no load is conditional.
  // The sum keeps store_grad's order: (acc + cadd) + old.
  auto finish = [&](auto c_tag, auto o_tag, auto b_tag) {
    constexpr bool kAddC = decltype(c_tag)::value, kAddOld = decltype(o_tag)::value;
    constexpr bool kBf16 = decltype(b_tag)::value;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      float xc[C::NBK][4], xo[C::NBK][4];
#pragma unroll
      for (int nb = 0; nb < C::NBK; ++nb) {
        const int64_t col = n0 + pipe_col<C>(wn, nb, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t o = (col < a.N && orow[mb][r] >= 0) ? orow[mb][r] * a.ldc + col : 0;
          if constexpr (kAddC) xc[nb][r] = a.cadd[o];
          if constexpr (kAddOld) {
            if constexpr (kBf16) xo[nb][r] = to_f32(static_cast<const bf16_t*>(a.C)[o]);
            else xo[nb][r] = static_cast<const float*>(a.C)[o];
          }
        }
      }
#pragma unroll
      for (int nb = 0; nb < C::NBK; ++nb) {
        const int64_t col = n0 + pipe_col<C>(wn, nb, lane);
        if (col >= a.N) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (orow[mb][r] < 0) continue;
          const int64_t o = orow[mb][r] * a.ldc + col;
          float v = acc[0][mb][nb][r];
          if constexpr (kAddC) v += xc[nb][r];
          if constexpr (kAddOld) v = xo[nb][r] + v;
          if constexpr (kBf16) static_cast<bf16_t*>(a.C)[o] = bf16_rne(v);
          else static_cast<float*>(a.C)[o] = v;
        }
      }
    }
  };
  using Y = std::true_type;
  using N_ = std::false_type;
  const int sel = (a.cadd ? 4 : 0) | (a.accumulate ? 2 : 0) | (a.out_bf16 ? 1 : 0);
  switch (sel) {
    case 0: finish(N_{}, N_{}, N_{}); break;
    case 1: finish(N_{}, N_{}, Y{}); break;
    case 2: finish(N_{}, Y{}, N_{}); break;
    case 3: finish(N_{}, Y{}, Y{}); break;
    case 4: finish(Y{}, N_{}, N_{}); break;
    case 5: finish(Y{}, N_{}, Y{}); break;
    case 6: finish(Y{}, Y{}, N_{}); break;
    default: finish(Y{}, Y{}, Y{}); break;
  }
}

template <bool AKC, bool BKC, int BN>
__global__ __launch_bounds__(512, 2) void gemm_pipe_kernel(GemmPipeArgs<AKC, BKC, BN> a) {
  using C = PipeCfg<256, BN, 1, AKC, BKC>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::kLdsBytes];
  int64_t M, K;
  int n_mt;
  gemm_pipe_bounds(a, M, K, n_mt);
  int t;
  if (!xcd_live_tile(blockIdx.x, n_mt * a.n_nt, t)) return;
  int mt, nt;
  grouped_tile(t, n_mt, a.n_nt, tile_group(256, BN), mt, nt);
  gemm_pipe_tile<AKC, BKC, BN>(a, mt, nt, M, K, lds, threadIdx.x);
}

// dH and dW of one chunk in one launch, both from the dz slab with 256 x 256
// tiles. dH alone has too few 256 x 256 tiles to fill the chip (N/256 x D/256)
// and its 256 x 128 form moves twice the operand bytes per MFMA; next to the dW
// tiles it needs no second wave: each XCD takes its share of one kind first
// and then its share of the other, so while some of an XCD's CUs run the long
// tiles of one kind the others run the shorter ones. dw_first: the dW tiles
// take the XCD's first places (the host picks the order that finishes first).
template <int BN>
__global__ __launch_bounds__(512, 2) void gemm_dual_kernel(GemmPipeArgs<true, false, BN> h,
                                                           GemmPipeArgs<false, false, BN> g, int dw_first) {
  using CH = PipeCfg<256, BN, 1, true, false>;
  using CW = PipeCfg<256, BN, 1, false, false>;
  static_assert(CH::kLdsBytes == CW::kLdsBytes, "one LDS image serves both");
  __shared__ __attribute__((aligned(16))) uint8_t lds[CH::kLdsBytes];
  int64_t mh, kh, mw, kw;
  int nmt_h, nmt_w;
  gemm_pipe_bounds(h, mh, kh, nmt_h);
  gemm_pipe_bounds(g, mw, kw, nmt_w);
  const int na = nmt_h * h.n_nt, nb = nmt_w * g.n_nt;
  const int x = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  const int qa = na / kXcds + (x < na % kXcds ? 1 : 0);
  const int qb = nb / kXcds + (x < nb % kXcds ? 1 : 0);
  // this block's kind and its place among the XCD's tiles of that kind
  const int q1 = dw_first ? qb : qa;
  const bool is_w = (local < q1) == (dw_first != 0);
  const int j = local < q1 ? local : local - q1;
  int mt, nt;
  if (!is_w) {
    if (j >= qa) return;
    grouped_tile(x * (na / kXcds) + min(x, na % kXcds) + j, nmt_h, h.n_nt, tile_group(256, BN), mt, nt);
    gemm_pipe_tile<true, false, BN>(h, mt, nt, mh, kh, lds, threadIdx.x);
  } else {
    if (j >= qb) return;
    grouped_tile(x * (nb / kXcds) + min(x, nb % kXcds) + j, nmt_w, g.n_nt, tile_group(256, BN), mt, nt);
    gemm_pipe_tile<false, false, BN>(g, mt, nt, mw, kw, lds, threadIdx.x);
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

namespace {

struct Launch {
  hipStream_t s;
  kd_trace* tr;
  template <class F>
  kd_status run(int kind, F&& f) {
    const bool rec = tr && tr->events && ((tr->mask >> kind) & 1u) && tr->count + 2 <= tr->capacity;
    if (rec && hipEventRecord(static_cast<hipEvent_t>(tr->events[tr->count]), s) != hipSuccess)
      return KD_ERR_HIP;
    f();
    if (hipGetLastError() != hipSuccess) return KD_ERR_HIP;
    if (rec) {
      if (hipEventRecord(static_cast<hipEvent_t>(tr->events[tr->count + 1]), s) != hipSuccess)
        return KD_ERR_HIP;
      if (tr->kinds) tr->kinds[tr->count / 2] = kind;
      tr->count += 2;
    }
    return KD_OK;
  }
};

#define KD_TRY(x)                     \
  do {                                \
    const kd_status st_ = (x);        \
    if (st_ != KD_OK) return st_;     \
  } while (0)

// Row kernels load 16-byte chunks when every row start of both matrices is
// 16-byte aligned.
template <typename T>
int row_vec(const void* a, const void* b, int64_t v) {
  return ((v * (int64_t)sizeof(T)) % 16 == 0 && (uintptr_t)a % 16 == 0 && (uintptr_t)b % 16 == 0) ? 1 : 0;
}

// The row kernels' way to the T = 1 student terms for student temperature T.
inline int row_z1(float T) { return (T == 1.f) ? kZ1Same : ((T == 2.f) ? kZ1Square : kZ1Own); }

// Forward row kernel instantiated for one launch's choices.
template <typename T, int Z1>
void rowstats_launch(bool rev, bool t1, dim3 grid, hipStream_t stream, const RowArgs& ra) {
  if (rev) {
    if (t1) rowstats_kernel<T, Z1, true, true><<<grid, kThreads, 0, stream>>>(ra);
    else rowstats_kernel<T, Z1, true, false><<<grid, kThreads, 0, stream>>>(ra);
  } else {
    if (t1) rowstats_kernel<T, Z1, false, true><<<grid, kThreads, 0, stream>>>(ra);
    else rowstats_kernel<T, Z1, false, false><<<grid, kThreads, 0, stream>>>(ra);
  }
}

template <typename T>
void rowstats_launch(int z1, bool rev, bool t1, dim3 grid, hipStream_t stream, const RowArgs& ra) {
  if (z1 == kZ1Same) rowstats_launch<T, kZ1Same>(rev, t1, grid, stream, ra);
  else if (z1 == kZ1Square) rowstats_launch<T, kZ1Square>(rev, t1, grid, stream, ra);
  else rowstats_launch<T, kZ1Own>(rev, t1, grid, stream, ra);
}

// Logit-gradient row kernel instantiated for one launch's choices.
template <typename T, int Z1>
void logits_bwd_launch(bool ce, bool rev, dim3 grid, hipStream_t stream, const RowArgs& ra) {
  if (ce) {
    if (rev) logits_bwd_kernel<T, true, Z1, true><<<grid, kThreads, 0, stream>>>(ra);
    else logits_bwd_kernel<T, true, Z1, false><<<grid, kThreads, 0, stream>>>(ra);
  } else {
    if (rev) logits_bwd_kernel<T, false, Z1, true><<<grid, kThreads, 0, stream>>>(ra);
    else logits_bwd_kernel<T, false, Z1, false><<<grid, kThreads, 0, stream>>>(ra);
  }
}

template <typename T>
void logits_bwd_launch(int z1, bool ce, bool rev, dim3 grid, hipStream_t stream, const RowArgs& ra) {
  if (!ce) logits_bwd_launch<T, kZ1Same>(false, rev, grid, stream, ra);  // Z1 unused
  else if (z1 == kZ1Same) logits_bwd_launch<T, kZ1Same>(true, rev, grid, stream, ra);
  else if (z1 == kZ1Square) logits_bwd_launch<T, kZ1Square>(true, rev, grid, stream, ra);
  else logits_bwd_launch<T, kZ1Own>(true, rev, grid, stream, ra);
}

// How a given [n x v] logits matrix is read: pipelined bf16 tiles hold it in
// registers from before the main loop (3: 8-byte vector loads, v a multiple of
// 4 and the matrix 8-byte aligned; 4: element loads); staged tiles load it
// after the main loop (1: a lane's four consecutive elements as one vector, v
// a multiple of 4 and vector-aligned; 0: element by element).
template <typename T, class G>
int given_mode(const void* ptr, int64_t v) {
  if (ptr == nullptr) return 0;
  if (G::kPipe && sizeof(T) == 2) return (v % 4 == 0 && (uintptr_t)ptr % 8 == 0) ? 3 : 4;
  return (v % 4 == 0 && ((uintptr_t)ptr % (4 * sizeof(T))) == 0) ? 1 : 0;
}

// Compaction of the usable-label rows into workspace copies of the token-side
// operands: idx / pos / nv, then H_s (and H_t) gathered into hc / htc.
struct Compacted {
  const int32_t* idx;
  const int32_t* pos;
  const int32_t* nv;
  const void* hs;
  const void* ht;
};

template <typename T>
kd_status compact_rows(const Plan& p, const Tensors& x, uint8_t* base, Launch& L, hipStream_t stream,
                       Compacted* out) {
  int32_t* idx = reinterpret_cast<int32_t*>(base + p.off_cidx);
  int32_t* pos = reinterpret_cast<int32_t*>(base + p.off_cpos);
  int32_t* nv = reinterpret_cast<int32_t*>(base + kNvOffset);
  CompactArgs ca{x.labels, p.n, p.v, p.ignore, idx, pos, nv};
  KD_TRY(L.run(KD_KERNEL_PREP, [&] { compact_kernel<<<1, kCompactThreads, 0, stream>>>(ca); }));
  const dim3 grid((unsigned)((p.dz_rows + kThreads / 64 - 1) / (kThreads / 64)), 2);
  GatherArgs ga{{static_cast<const uint8_t*>(x.hs), static_cast<const uint8_t*>(x.ht)},
                {base + p.off_hc, base + p.off_htc},
                {p.d * (int64_t)sizeof(T), p.dt * (int64_t)sizeof(T)}, idx, nv, p.dz_rows};
  KD_TRY(L.run(KD_KERNEL_PREP, [&] { gather_rows_kernel<<<grid, kThreads, 0, stream>>>(ga); }));
  *out = Compacted{idx, pos, nv, base + p.off_hc, base + p.off_htc};
  return KD_OK;
}

template <typename T, class G>
kd_status forward_t(const Plan& p, const Tensors& x, const kd_outputs* out, void* saved, void* ws,
                    hipStream_t stream, kd_trace* trace, int32_t* status_out) {
  Launch L{stream, trace};
  uint8_t* base = static_cast<uint8_t*>(ws);
  float* prep = reinterpret_cast<float*>(base + p.off_prep);
  float* rec = reinterpret_cast<float*>(base + p.off_rec);
  double* part = reinterpret_cast<double*>(base + p.off_part);
  int32_t* status = status_out ? status_out : reinterpret_cast<int32_t*>(base);

  int32_t* tk_idx = reinterpret_cast<int32_t*>(base + p.off_tks);
  float* tk_prob = reinterpret_cast<float*>(base + p.off_tks + 4 * (size_t)p.n * (size_t)p.k);
  int32_t* tk_off = reinterpret_cast<int32_t*>(base + p.off_tko);
  PrepArgs pa{x.hs, x.w, x.ht, x.wt, x.logits, x.tlogits, x.labels, x.topk_idx, x.topk_prob,
              p.n, p.d, p.dt, p.v, p.ignore, p.k, 0, prep, tk_idx, tk_prob};
  pa.want_teacher = p.mode != MODE_TOPK && (p.wt > 0.f || (out && out->teacher_ce));
  const dim3 pgrid((unsigned)((p.n + 3) / 4));
  KD_TRY(L.run(KD_KERNEL_PREP, [&] {
    switch (p.mode) {
      case MODE_TOPK: prep_kernel<T, MODE_TOPK><<<pgrid, kThreads, 0, stream>>>(pa); break;
      case MODE_LOGITS: prep_kernel<T, MODE_LOGITS><<<pgrid, kThreads, 0, stream>>>(pa); break;
      case MODE_TLOGITS: prep_kernel<T, MODE_TLOGITS><<<pgrid, kThreads, 0, stream>>>(pa); break;
      case MODE_BOTH: prep_kernel<T, MODE_BOTH><<<pgrid, kThreads, 0, stream>>>(pa); break;
      default: prep_kernel<T, MODE_TIED><<<pgrid, kThreads, 0, stream>>>(pa); break;
    }
  }));

  // Rows with an ignored label left out: the tiles run on compacted copies.
  Compacted cp{nullptr, nullptr, nullptr, x.hs, x.ht};
  if (p.compact) KD_TRY(compact_rows<T>(p, x, base, L, stream, &cp));

  // Teacher statistics at T = 1 only feed the teacher CE.
  const int need_t1 = (p.need_t1 && pa.want_teacher) ? 1 : 0;
  const void* given = (p.mode == MODE_TLOGITS) ? x.tlogits : x.logits;
  FwdArgs fa{cp.hs, x.w, cp.ht, x.wt, x.logits, x.tlogits, p.n, p.d, p.dt, p.v,
             p.n_ttiles, p.n_vtiles, p.tps, p.n_slices, kLog2e / p.T, kLog2e / p.Tt, p.T / p.Tt,
             p.need_zT, need_t1, p.kl, given_mode<T, G>(given, p.v),
             (p.T == 2.f && p.need_zT) ? 1 : 0, rec, cp.nv, tk_idx, tk_prob, tk_off, p.k, 0};
  float* run = reinterpret_cast<float*>(base + p.off_run);
  const bool folded = p.fwd_slices < p.n_slices;  // several forward launches
  int last_slices = p.fwd_slices;                 // records of the last launch
  if (p.mode == MODE_BOTH) {
    RowArgs ra{};
    ra.zl = x.logits;
    ra.tl = x.tlogits;
    ra.n = p.n;
    ra.v = p.v;
    ra.cT = kLog2e / p.T;
    ra.cTt = kLog2e / p.Tt;
    ra.rho = p.T / p.Tt;
    ra.vec = row_vec<T>(x.logits, x.tlogits, p.v);
    ra.rec = rec;
    ra.slice = p.row_slice;
    ra.n_slices = p.n_slices;
    const dim3 grid((unsigned)((p.n * (int64_t)p.n_slices + 3) / 4));
    KD_TRY(L.run(KD_KERNEL_FWD, [&] {
      rowstats_launch<T>(row_z1(p.T), p.kl != KD_KL_FORWARD, need_t1 != 0, grid, stream, ra);
    }));
  } else {
    // one launch per vocabulary chunk of fwd_slices tiles
    for (int s0 = 0; s0 < p.n_vtiles; s0 += p.fwd_slices) {
      fa.slice0 = s0;
      fa.n_slices = std::min(p.fwd_slices, p.n_vtiles - s0);
      // the last chunk's products are kept in `saved` for the backward
      const bool keep = p.keep && saved && s0 + fa.n_slices >= p.n_vtiles;
      fa.keep = keep ? reinterpret_cast<float*>(static_cast<uint8_t*>(saved) + p.keep_off) : nullptr;
      fa.keep_t = (p.keep_ops == 2) ? p.dz_rows * p.keep_ld : 0;
      const dim3 fgrid((unsigned)((int64_t)fa.n_slices * p.n_ttiles));
      if (p.mode == MODE_TOPK) {
        const TileStartArgs ts{tk_idx, p.n, p.v, p.k, p.vt_rows, s0, fa.n_slices, tk_off};
        const int64_t cnt = p.n * (int64_t)(fa.n_slices + 1);
        KD_TRY(L.run(KD_KERNEL_PREP, [&] {
          topk_tile_starts_kernel<<<dim3((unsigned)((cnt + kThreads - 1) / kThreads)), kThreads, 0,
                                    stream>>>(ts);
        }));
      }
      KD_TRY(L.run(KD_KERNEL_FWD, [&] {
        switch (p.mode) {
          case MODE_TIED: fwd_tiles_kernel<T, MODE_TIED, G><<<fgrid, G::kThreads, 0, stream>>>(fa); break;
          case MODE_SEPARATE: fwd_tiles_kernel<T, MODE_SEPARATE, G><<<fgrid, G::kThreads, 0, stream>>>(fa); break;
          case MODE_TOPK:  // one B operand: the 256-token tiles in the pipelined geometry
            fwd_tiles_kernel<T, MODE_TOPK, std::conditional_t<G::kPipe, GeoWide, G>>
                <<<fgrid, G::kThreads, 0, stream>>>(fa);
            break;
          case MODE_TLOGITS:
            fwd_tiles_kernel<T, MODE_TLOGITS, std::conditional_t<G::kPipe, GeoWide, G>>
                <<<fgrid, G::kThreads, 0, stream>>>(fa);
            break;
          default:  // one B operand: the 256-token tiles in the pipelined geometry
            fwd_tiles_kernel<T, MODE_LOGITS, std::conditional_t<G::kPipe, GeoWide, G>>
                <<<fgrid, G::kThreads, 0, stream>>>(fa);
            break;
        }
      }));
      last_slices = fa.n_slices;
      if (s0 + fa.n_slices < p.n_vtiles) {  // the last chunk goes to the merge itself
        const FoldArgs fo{rec, fa.n_slices, run, p.n, s0 == 0 ? 1 : 0};
        KD_TRY(L.run(KD_KERNEL_MERGE, [&] {
          fold_kernel<<<dim3((unsigned)p.merge_blocks), kMergeThreads, 0, stream>>>(fo);
        }));
      }
    }
  }

  MergeArgs ma{rec, prep, last_slices, folded ? run : nullptr, p.n, p.mode, p.T, p.need_zT, need_t1,
               (p.mode != MODE_TOPK) ? 1 : 0, p.kl, p.kl_unscaled, p.ws, p.wt, p.wkl,
               out ? out->student_ce : nullptr, out ? out->teacher_ce : nullptr,
               out ? out->kl : nullptr, static_cast<float*>(saved), part, cp.pos};
  ma.teacher_ce = pa.want_teacher;
  KD_TRY(L.run(KD_KERNEL_MERGE, [&] {
    merge_kernel<<<dim3((unsigned)p.merge_blocks), kMergeThreads, 0, stream>>>(ma);
  }));

  FinalArgs fin{part, p.merge_blocks, p.normalizer, p.reduction, out ? out->loss : nullptr,
                saved ? static_cast<float*>(saved) + 4 * p.n : nullptr, status,
                {p.keep ? kKeepMagic : 0, (int32_t)p.chunk, (int32_t)p.keep_ld, p.keep_ops,
                 (int32_t)p.n}};
  KD_TRY(L.run(KD_KERNEL_FINALIZE, [&] { finalize_kernel<<<1, kThreads, 0, stream>>>(fin); }));
  return KD_OK;
}

template <typename T, class G>
// teacher = false: the student's dH / dW from the loss's logit gradient;
// teacher = true: the teacher's from its CE gradient (dh / dw are then the
// teacher's hidden and weight gradients, of width d_t).
kd_status backward_t(const Plan& p, const Tensors& x, const void* saved, const float* grad,
                     void* dh, void* dw, int accumulate, void* ws, hipStream_t stream,
                     kd_trace* trace, bool teacher) {
  Launch L{stream, trace};
  uint8_t* base = static_cast<uint8_t*>(ws);
  T* dz = reinterpret_cast<T*>(base + p.off_dz);
  const int64_t ldz = p.chunk;
  const int64_t gd = teacher ? p.dt : p.d;  // width of the gradients
  const int eh = p.dh_bf16 ? 2 : 4, ew = p.dw_bf16 ? 2 : 4;  // gradient element bytes
  if (teacher && p.wt == 0.f) {  // no teacher CE: nothing reaches the teacher
    if (!accumulate) {
      for (void* m : {dh, dw}) {
        if (!m) continue;
        const int64_t cnt = (m == dh ? p.n * eh : p.v * ew) * gd / 4;  // fp32 words (gd % 8 == 0)
        KD_TRY(L.run(KD_KERNEL_GEMM_DH, [&] {
          fill_zero_kernel<<<dim3((unsigned)((cnt + kThreads - 1) / kThreads)), kThreads, 0, stream>>>(
              static_cast<float*>(m), cnt);
        }));
      }
    }
    return KD_OK;
  }
  // bf16 dH over several chunks: the chunks before the last sum into an fp32
  // buffer, which the last chunk's launch adds before its one rounding
  float* dh_acc = (p.dh_bf16 && p.n_chunks > 1) ? reinterpret_cast<float*>(base + p.off_dhacc) : nullptr;
  struct DhTarget {
    void* C;
    int out_bf16;
    const float* cadd;
    int accumulate;
  };
  auto dh_target = [&](int c) -> DhTarget {
    const bool last = c == p.n_chunks - 1;
    if (dh_acc && !last) return DhTarget{dh_acc, 0, nullptr, c > 0 ? 1 : 0};
    if (dh_acc) return DhTarget{dh, 1, dh_acc, accumulate};
    return DhTarget{dh, p.dh_bf16, nullptr, (accumulate || c > 0) ? 1 : 0};
  };
  void* const dw_base = dw;
  Compacted cp{nullptr, nullptr, nullptr, x.hs, x.ht};
  if (p.compact) {
    KD_TRY(compact_rows<T>(p, x, base, L, stream, &cp));
    // dH rows of left-out tokens: the compacted GEMMs never write them
    if (dh && !accumulate) {
      KD_TRY(L.run(KD_KERNEL_GEMM_DH, [&] {
        zero_rows_kernel<<<dim3((unsigned)((p.n + kThreads / 64 - 1) / (kThreads / 64))), kThreads, 0,
                           stream>>>(dh, cp.pos, p.n, gd, eh);
      }));
    }
  }
  // the token-side operand and the weight of the GEMMs
  const T* hs = static_cast<const T*>(teacher ? cp.ht : cp.hs);
  const T* wmat = static_cast<const T*>(teacher ? x.wt : x.w);
  const int mode = teacher ? (int)MODE_TCE : p.mode;
  // Top-K: each row's entries sorted by index, as the forward sorted them, so
  // the dz epilogue finds the entries of each tile as one run.
  int32_t* tk_idx = reinterpret_cast<int32_t*>(base + p.off_btks);
  float* tk_prob = reinterpret_cast<float*>(base + p.off_btks + 4 * (size_t)p.n * (size_t)p.k);
  int32_t* tk_off = reinterpret_cast<int32_t*>(base + p.off_btko);
  if (mode == MODE_TOPK) {
    PrepArgs pa{x.hs, x.w, x.ht, x.wt, x.logits, x.tlogits, x.labels, x.topk_idx, x.topk_prob,
                p.n, p.d, p.dt, p.v, p.ignore, p.k, 0, nullptr, tk_idx, tk_prob};
    KD_TRY(L.run(KD_KERNEL_PREP, [&] {
      prep_kernel<T, MODE_TOPK><<<dim3((unsigned)((p.n + 3) / 4)), kThreads, 0, stream>>>(pa);
    }));
  }
  for (int c = 0; c < p.n_chunks; ++c) {
    const int64_t c0 = (int64_t)c * p.chunk;
    const int64_t cw = (p.v - c0 < p.chunk) ? (p.v - c0) : p.chunk;  // valid columns
    const int n_vt = (int)((cw + G::kVT - 1) / G::kVT);  // fused tiles of the chunk
    BwdArgs ba{cp.hs, x.w, cp.ht, x.wt, x.tlogits, p.n, p.d, p.dt, p.v, x.labels, p.ignore,
               static_cast<const float*>(saved), grad, p.ws, p.wkl, p.T, kLog2e / p.T,
               kLog2e / p.Tt, p.T / p.Tt, p.wt, p.need_zT, p.kl, given_mode<T, G>(x.tlogits, p.v),
               (!teacher && p.T == 2.f && p.need_zT) ? 1 : 0, cp.idx, cp.nv, c0, n_vt, p.n_ttiles,
               dz, ldz, p.dz_rows};
    // The forward's last chunk: its products were kept in `saved` (the
    // teacher's as well for a TIED or SEPARATE teacher).
    const bool kept = p.keep && c == p.n_chunks - 1 && (!teacher || p.keep_ops == 2);
    if (kept) {
      ba.keep = reinterpret_cast<const float*>(static_cast<const uint8_t*>(saved) + p.keep_off);
      ba.keep_t = (p.keep_ops == 2) ? p.dz_rows * p.keep_ld : 0;
      const int32_t tag[5] = {kKeepMagic, (int32_t)p.chunk, (int32_t)p.keep_ld, p.keep_ops, (int32_t)p.n};
      for (int j = 0; j < 5; ++j) ba.keep_tag[j] = tag[j];
    }
    ba.status = reinterpret_cast<int32_t*>(base);
    ba.set_status = (c == 0 || kept) ? 1 : 0;
    if (mode == MODE_TOPK) {
      ba.tk_sidx = tk_idx;
      ba.tk_sprob = tk_prob;
      ba.tk_off = tk_off;
      ba.k = p.k;
      const TileStartArgs ts{tk_idx, p.n, p.v, p.k, G::kVT, (int)(c0 / G::kVT), n_vt, tk_off};
      const int64_t cnt = p.n * (int64_t)(n_vt + 1);
      KD_TRY(L.run(KD_KERNEL_PREP, [&] {
        topk_tile_starts_kernel<<<dim3((unsigned)((cnt + kThreads - 1) / kThreads)), kThreads, 0,
                                  stream>>>(ts);
      }));
    }
    const dim3 grid((unsigned)((int64_t)n_vt * p.n_ttiles));
    auto launch = [&](auto kept_tag) {
      constexpr bool K = decltype(kept_tag)::value;
      switch (mode) {
        case MODE_TCE: bwd_dz_kernel<T, MODE_TCE, G, K><<<grid, G::kThreads, 0, stream>>>(ba); break;
        case MODE_TIED: bwd_dz_kernel<T, MODE_TIED, G, K><<<grid, G::kThreads, 0, stream>>>(ba); break;
        case MODE_SEPARATE: bwd_dz_kernel<T, MODE_SEPARATE, G, K><<<grid, G::kThreads, 0, stream>>>(ba); break;
        case MODE_TLOGITS:
          bwd_dz_kernel<T, MODE_TLOGITS, std::conditional_t<G::kPipe, GeoWide, G>, K>
              <<<grid, G::kThreads, 0, stream>>>(ba);
          break;
        default:
          bwd_dz_kernel<T, MODE_TOPK, std::conditional_t<G::kPipe, GeoWide, G>, K>
              <<<grid, G::kThreads, 0, stream>>>(ba);
          break;
      }
    };
    KD_TRY(L.run(kept ? KD_KERNEL_BWD_KEPT : KD_KERNEL_BWD_DZ, [&] {
      if (kept) launch(std::true_type{});
      else launch(std::false_type{});
    }));
    const int64_t cpad = (int64_t)n_vt * G::kVT;  // columns written by bwd_dz
    const int n_gemm_mt = (int)((cw + kTile - 1) / kTile);
    if constexpr (G::kPipe) {
      // dW[c0 + m, :] = sum_i dz[i, m] H[i, :]: A(m, i) = dz[i * ldz + m], B(n, i) = H[i * d + n],
      // both row-contiguous; the slab's zero rows past n pad K to a multiple of 64.
      auto dw_args = [&](auto bn_tag) {
        constexpr int BN = decltype(bn_tag)::value;
        GemmPipeArgs<false, false, BN> ga;
        ga.A = PipeOperandMN{dz, ldz, cpad, p.dz_rows};
        ga.B = PipeOperandMN{hs, gd, gd, p.n};
        ga.C = static_cast<uint8_t*>(dw_base) + c0 * gd * ew;
        ga.out_bf16 = p.dw_bf16;
        ga.cadd = nullptr;
        ga.ldc = gd;
        ga.M = cw;
        ga.N = gd;
        ga.K = p.dz_rows;
        ga.accumulate = accumulate;
        ga.n_mt = (int)((cw + 255) / 256);
        ga.n_nt = (int)((gd + BN - 1) / BN);
        ga.kdev = cp.nv;  // compacted: the token rows stop at nv
        ga.mdev = nullptr;
        ga.rowmap = nullptr;
        return ga;
      };
      // dH[i, :] += sum_m dz[i, m] W[c0 + m, :]: A(i, m) = dz[i * ldz + m] (K-contiguous),
      // B(n, m) = W[(c0 + m) * d + n] (row-contiguous); slab columns past cw are zero.
      auto dh_args = [&](auto bn_tag) {
        constexpr int BN = decltype(bn_tag)::value;
        GemmPipeArgs<true, false, BN> gb;
        gb.A = PipeOperand{dz, ldz, p.n};
        gb.B = PipeOperandMN{wmat + c0 * gd, gd, gd, cw};
        const DhTarget tg = dh_target(c);
        gb.C = tg.C;
        gb.out_bf16 = tg.out_bf16;
        gb.cadd = tg.cadd;
        gb.ldc = gd;
        gb.M = p.n;
        gb.N = gd;
        gb.K = cpad;
        gb.accumulate = tg.accumulate;
        gb.n_mt = (int)((p.n + 255) / 256);
        gb.n_nt = (int)((gd + BN - 1) / BN);
        gb.kdev = nullptr;
        gb.mdev = cp.nv;      // compacted: rows past nv are not tokens
        gb.rowmap = cp.idx;   // compacted row m is token idx[m]
        return gb;
      };
      using W256 = std::integral_constant<int, 256>;
      using W128 = std::integral_constant<int, 128>;
      if (dw && dh) {
        // one launch, 256 x 256 tiles for both; the grid covers the largest
        // per-XCD share of dH plus dW tiles
        const auto gb = dh_args(W256{});
        const auto ga = dw_args(W256{});
        const int na = gb.n_mt * gb.n_nt, nb = ga.n_mt * ga.n_nt;
        int most = 0;
        for (int xc = 0; xc < kXcds; ++xc)
          most = std::max(most, na / kXcds + (xc < na % kXcds) + nb / kXcds + (xc < nb % kXcds));
        // Order of the two kinds on an XCD: a greedy schedule of its tiles (one
        // per CU at a time, in dispatch order) on its CUs, in K steps, for each
        // order; dH first unless dW first finishes sooner (a short last chunk:
        // few long dW tiles left over after the short dH tiles would run alone).
        auto makespan = [](int n1, int64_t k1, int n2, int64_t k2) {
          std::vector<int64_t> cu(kCusPerXcd, 0);
          auto take = [&](int cnt, int64_t k) {
            for (int j = 0; j < cnt; ++j) *std::min_element(cu.begin(), cu.end()) += k;
          };
          take(n1, k1);
          take(n2, k2);
          return *std::max_element(cu.begin(), cu.end());
        };
        const int qa = (na + kXcds - 1) / kXcds, qb = (nb + kXcds - 1) / kXcds;
        const int64_t sh = (gb.K + kPipeBK - 1) / kPipeBK, sw = (ga.K + kPipeBK - 1) / kPipeBK;
        const int dw_first = makespan(qb, sw, qa, sh) < makespan(qa, sh, qb, sw) ? 1 : 0;
        KD_TRY(L.run(KD_KERNEL_GEMM_DWDH, [&] {
          gemm_dual_kernel<256><<<dim3((unsigned)(kXcds * most)), 512, 0, stream>>>(gb, ga, dw_first);
        }));
      } else {
        // 256-wide tiles when they still give every CU a tile, else 128-wide.
        auto wide = [&](int64_t m) { return ((m + 255) / 256) * ((gd + 255) / 256) >= 256; };
        auto run = [&](int kind, auto args, auto kern) {
          return L.run(kind, [&] { kern<<<dim3((unsigned)(args.n_mt * args.n_nt)), 512, 0, stream>>>(args); });
        };
        if (dw) {
          KD_TRY(wide(cw) ? run(KD_KERNEL_GEMM_DW, dw_args(W256{}), gemm_pipe_kernel<false, false, 256>)
                          : run(KD_KERNEL_GEMM_DW, dw_args(W128{}), gemm_pipe_kernel<false, false, 128>));
        }
        if (dh) {
          KD_TRY(wide(p.n) ? run(KD_KERNEL_GEMM_DH, dh_args(W256{}), gemm_pipe_kernel<true, false, 256>)
                           : run(KD_KERNEL_GEMM_DH, dh_args(W128{}), gemm_pipe_kernel<true, false, 128>));
        }
      }
    } else {
    if (dw) {
      // dW[c0 + m, :] = sum_i dz[i, m] H_s[i, :]; A(m, i) = dz[i * ldz + m], B(n, i) = H_s[i * d + n]
      GemmArgs<T, false, false> ga;
      ga.A = Operand<T, false>{dz, ldz, cpad, p.n};
      ga.B = Operand<T, false>{hs, gd, gd, p.n};
      ga.C = static_cast<uint8_t*>(dw_base) + c0 * gd * ew;
      ga.out_bf16 = p.dw_bf16;
      ga.cadd = nullptr;
      ga.ldc = gd;
      ga.M = cw;
      ga.N = gd;
      ga.K = p.n;
      ga.accumulate = accumulate;
      ga.n_mt = n_gemm_mt;
      ga.n_nt = (int)((gd + kTile - 1) / kTile);
      ga.kdev = cp.nv;
      ga.mdev = nullptr;
      ga.rowmap = nullptr;
      KD_TRY(L.run(KD_KERNEL_GEMM_DW, [&] {
        gemm_kernel<T, false, false>
            <<<dim3((unsigned)(ga.n_mt * ga.n_nt)), kThreads, 0, stream>>>(ga);
      }));
    }
    if (dh) {
      // dH[i, :] += sum_m dz[i, m] W[c0 + m, :]; A(i, m) = dz[i * ldz + m], B(n, m) = W[(c0 + m) * d + n]
      GemmArgs<T, true, false> gb;
      gb.A = Operand<T, true>{dz, ldz, p.n, cpad};
      gb.B = Operand<T, false>{wmat + c0 * gd, gd, gd, cw};
      const DhTarget tg = dh_target(c);
      gb.C = tg.C;
      gb.out_bf16 = tg.out_bf16;
      gb.cadd = tg.cadd;
      gb.ldc = gd;
      gb.M = p.n;
      gb.N = gd;
      gb.K = cw;
      gb.accumulate = tg.accumulate;
      gb.n_mt = p.n_ttiles;
      gb.n_nt = (int)((gd + kTile - 1) / kTile);
      gb.kdev = nullptr;
      gb.mdev = cp.nv;
      gb.rowmap = cp.idx;
      KD_TRY(L.run(KD_KERNEL_GEMM_DH, [&] {
        gemm_kernel<T, true, false>
            <<<dim3((unsigned)(gb.n_mt * gb.n_nt)), kThreads, 0, stream>>>(gb);
      }));
    }
    }
  }
  return KD_OK;
}

}  // namespace

static_assert(kPipeK == kPipeBK, "K step of the pipelined path");
static_assert(GeoWide::kVT == GeoFused::kVT, "one vocabulary tile for every pipelined mode");
int pipe_vocab_rows() { return GeoFused::kVT; }
int fused_token_rows(int mode, int pipe) {
  const bool one_b = mode == MODE_TOPK || mode == MODE_LOGITS || mode == MODE_TLOGITS;
  return (pipe && one_b) ? GeoWide::kTT : GeoFused::kTT;
}

kd_status run_forward(const Plan& p, const Tensors& x, const kd_outputs* out, void* saved,
                      void* workspace, hipStream_t stream, kd_trace* trace, int32_t* status_out) {
  if (p.dtype == KD_BF16) {
    if (p.pipe) return forward_t<bf16_t, GeoFused>(p, x, out, saved, workspace, stream, trace, status_out);
    return forward_t<bf16_t, GeoStaged>(p, x, out, saved, workspace, stream, trace, status_out);
  }
  return forward_t<float, GeoStaged>(p, x, out, saved, workspace, stream, trace, status_out);
}

}  // namespace kd

// Scratch of the forward that allocates nothing (kd_loss_fwd_noalloc): the
// forward workspace of every such call on a device, a file-scope device array
// that each device holds until the process ends. Host code never passes the
// array's name to a kernel (on the host it is a stand-in, not a device
// address): it takes the address hipGetSymbolAddress gives for the current
// device, looked up once per device.
static __device__ __align__(256) uint8_t scratch[kd::kScratchBytes];

namespace kd {

void* scratch_address(kd_status* st) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *st = KD_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      *st = KD_ERR_HIP;
      return nullptr;
    }
    addr[dev] = ptr;
  }
  *st = KD_OK;
  return addr[dev];
}

namespace {
kd_status backward_any(const Plan& p, const Tensors& x, const void* saved, const float* grad_loss,
                       void* d_hidden, void* d_weight, int accumulate, void* workspace,
                       hipStream_t stream, kd_trace* trace, bool teacher) {
  if (p.dtype == KD_BF16) {
    if (p.pipe)
      return backward_t<bf16_t, GeoFused>(p, x, saved, grad_loss, d_hidden, d_weight, accumulate,
                                         workspace, stream, trace, teacher);
    return backward_t<bf16_t, GeoStaged>(p, x, saved, grad_loss, d_hidden, d_weight, accumulate,
                                         workspace, stream, trace, teacher);
  }
  return backward_t<float, GeoStaged>(p, x, saved, grad_loss, d_hidden, d_weight, accumulate,
                                      workspace, stream, trace, teacher);
}
}  // namespace

kd_status run_backward(const Plan& p, const Tensors& x, const void* saved, const float* grad_loss,
                       void* d_hidden, void* d_weight, int accumulate, void* workspace,
                       hipStream_t stream, kd_trace* trace) {
  return backward_any(p, x, saved, grad_loss, d_hidden, d_weight, accumulate, workspace, stream,
                      trace, false);
}

kd_status run_backward_logits(const Plan& p, const Tensors& x, const void* saved,
                              const float* grad_loss, void* d_logits, int accumulate,
                              hipStream_t stream, kd_trace* trace) {
  Launch L{stream, trace};
  RowArgs ra{};
  ra.zl = x.logits;
  ra.tl = x.tlogits;
  ra.n = p.n;
  ra.v = p.v;
  ra.cT = kLog2e / p.T;
  ra.cTt = kLog2e / p.Tt;
  ra.rho = p.T / p.Tt;
  ra.labels = x.labels;
  ra.ignore = p.ignore;
  ra.saved = static_cast<const float*>(saved);
  ra.grad = grad_loss;
  ra.ws = p.ws;
  ra.wkl = p.wkl;
  ra.T = p.T;
  ra.kl = p.kl;
  ra.accumulate = accumulate;
  ra.dz = d_logits;
  ra.slice = p.row_slice;
  ra.n_slices = p.n_slices;
  const dim3 grid((unsigned)((p.n * (int64_t)p.n_slices + 3) / 4));
  const int z1 = row_z1(p.T);
  const bool ce = p.ws != 0.f, rev = p.kl != KD_KL_FORWARD;
  if (p.dtype == KD_BF16) {
    ra.vec = row_vec<bf16_t>(x.logits, x.tlogits, p.v) && row_vec<bf16_t>(d_logits, d_logits, p.v);
    return L.run(KD_KERNEL_BWD_DZ, [&] { logits_bwd_launch<bf16_t>(z1, ce, rev, grid, stream, ra); });
  }
  ra.vec = row_vec<float>(x.logits, x.tlogits, p.v) && row_vec<float>(d_logits, d_logits, p.v);
  return L.run(KD_KERNEL_BWD_DZ, [&] { logits_bwd_launch<float>(z1, ce, rev, grid, stream, ra); });
}

kd_status run_backward_teacher(const Plan& p, const Tensors& x, const void* saved,
                               const float* grad_loss, void* d_hidden, void* d_weight,
                               int accumulate, void* workspace, hipStream_t stream, kd_trace* trace) {
  return backward_any(p, x, saved, grad_loss, d_hidden, d_weight, accumulate, workspace, stream,
                      trace, true);
}

}  // namespace kd
