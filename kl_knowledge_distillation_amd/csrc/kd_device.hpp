// Device building blocks for gfx950 (CDNA4): element types, LDS operand
// staging, and the double-buffered MFMA main loop of the register-staged path
// (fp32, and bf16 hidden sizes that are not a multiple of 64).
//
// Tile shape. A workgroup has 256 threads = 4 wave64s arranged 2 x 2 and
// computes a 128 x 128 output tile; each wave owns a 64 x 64 sub-tile made of
// 4 x 4 blocks of the 16x16 MFMA (v_mfma_f32_16x16x32_bf16 for bf16,
// v_mfma_f32_16x16x4_f32 for fp32). One K step moves 64 bytes of every
// operand row: 32 bf16 or 16 fp32 elements.
//
// LDS layout. Each staged operand tile is 128 rows x 80 bytes: the 64 data
// bytes of a row, K-contiguous, plus 16 pad bytes, which makes the 16-byte
// fragment reads of 16 consecutive rows land in distinct bank groups. Two
// stages are kept (double buffering); one barrier per K step.
//
// Output layout of the 16x16 MFMA (both element types, and the pipelined bf16
// path): lane l holds column l % 16 and rows 4 (l / 16) + r, r in [0, 4), of
// its block. The tile kernels put vocabulary on the row axis, so the per-token
// reductions of the epilogue run over a lane's own registers and then over the
// four lanes l % 16 + 16 q.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kd {

constexpr int kThreads = 256;
constexpr int kTile = 128;
constexpr int kRowBytes = 80;
constexpr int kTileBytes = kTile * kRowBytes;  // 10240
constexpr int kXcds = 8;                       // MI355X: 8 XCDs, each with its own L2
constexpr int kCusPerXcd = 32;                 // 256 CUs in all
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef uint16_t bf16_t;  // bf16 storage
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kBK = 16;       // elements per K step
  static constexpr int kPerChunk = 4;  // elements per 16-byte chunk
};
template <> struct Elem<bf16_t> {
  static constexpr int kBK = 32;
  static constexpr int kPerChunk = 8;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN): gfx950's
// v_cvt_pk_bf16_f32, two values per instruction.
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const f32x2_hw v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_hw));
}
__device__ __forceinline__ bf16_t bf16_rne(float f) { return (bf16_t)(bf16x2_rne(f, 0.f) & 0xffffu); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// A 16-byte load of data streamed once, marked nontemporal so the caches do
// not keep it in place of data that is reused. (Nontemporal stores of the
// given-logits gradient measured slower than plain ones, so stores stay plain.)
typedef uint32_t u32x4_hw __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const void* p) {
  const u32x4_hw v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_hw*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// The dispatcher hands workgroup b to XCD b % 8. Remap so that each XCD owns a
// contiguous range of tile indices: neighbouring tiles then share its L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int per = nblocks / kXcds, rem = nblocks % kXcds;
  const int x = bid % kXcds, local = bid / kXcds;
  return x * per + min(x, rem) + local;
}

// The same split for a grid sized for more tiles than have work: only the
// first `live` tiles (in tile order) do, and they are spread evenly over the
// XCDs. Returns false for a block past its XCD's share (it has nothing to do).
// With live == nblocks this is xcd_remap.
__device__ __forceinline__ bool xcd_live_tile(int bid, int live, int& t) {
  const int per = live / kXcds, rem = live % kXcds;
  const int x = bid % kXcds, local = bid / kXcds;
  if (local >= per + (x < rem ? 1 : 0)) return false;
  t = x * per + min(x, rem) + local;
  return true;
}

// Grouped order over an (na x nb) grid of tiles: runs of `group` consecutive
// b values for each a, so a window of consecutive tiles covers a near-square
// block and both operands are re-read from L2 rather than HBM.
__device__ __forceinline__ void grouped_tile(int t, int na, int nb, int group, int& a, int& b) {
  const int width = group * na;
  const int g = t / width;
  const int first = g * group;
  const int gsz = min(nb - first, group);
  const int r = t - g * width;
  a = r / gsz;
  b = first + r % gsz;
}

// The group of an XCD's 32 concurrent tiles (a x b = 32 / group x group): the
// shape that touches the fewest distinct operand bytes per K step, and, where
// two shapes tie (square tiles), the one in which each b-side (B operand) block
// serves more tiles, since the pipelined loop copies that operand with less
// lead and its L2 misses cost more. 256-row A and 128-row B tiles: 4 x 8
// (256 KB per step against 320 KB for 8 x 4); 256 x 256: 8 x 4. (The
// register-staged 128 x 128 tiles keep 4 x 8.)
constexpr int tile_group(int a_rows, int b_rows) { return a_rows == 256 && b_rows == 256 ? 4 : 8; }

// An operand of C = A B^T-style contractions, seen as (row, k) elements.
// KC  (K-contiguous):  element (row, k) at ptr[row * ld + k]; rows < `rows`, k < `kdim`.
// !KC (row-contiguous): element (row, k) at ptr[k * ld + row]; `rows` a multiple of
//                       the chunk width, k < `kdim`.
template <typename T, bool KC>
struct Operand {
  const T* ptr;
  int64_t ld;
  int64_t rows;
  int64_t kdim;
};

// Stages one 128-row x K-step tile of an operand: global -> registers -> LDS.
// Out-of-range rows / k are zero-filled, so ragged edges contribute nothing.
//
// K-contiguous operands move 16-byte chunks straight through. Row-contiguous
// operands are transposed on the way: lane L of wave w owns rows 2L and 2L+1
// and the 16-byte K chunk w of both (8 bf16 or 4 fp32 k-values). It reads one
// element pair from each of those k-rows (each load instruction of the wave
// covers 256 contiguous bytes of one k-row), repacks the pairs in registers,
// and writes two 16-byte LDS chunks whose addresses fall in distinct banks.
template <typename T, bool KC>
struct Stager {
  uint4 r[2];

  __device__ __forceinline__ void load(const Operand<T, KC>& op, int64_t row0, int64_t k0, int tid) {
    constexpr int PC = Elem<T>::kPerChunk;
    if constexpr (KC) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int q = tid + kThreads * j;
        const int row = q >> 2, c = q & 3;
        const int64_t grow = row0 + row, k = k0 + (int64_t)c * PC;
        if (grow < op.rows && k < op.kdim)
          r[j] = *reinterpret_cast<const uint4*>(op.ptr + grow * op.ld + k);
        else
          r[j] = make_uint4(0u, 0u, 0u, 0u);
      }
    } else {
      const int lane = tid & 63, w = tid >> 6;
      const int64_t m = row0 + 2 * lane;
      const bool mok = m < op.rows;  // rows is a multiple of the chunk width, so m+1 too
      uint32_t* u = reinterpret_cast<uint32_t*>(r);
      if constexpr (sizeof(T) == 2) {
        // k-rows k0 + 8w + j, j = 0..7; one 32-bit pair (rows m, m+1) each.
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int64_t k = k0 + 8 * w + j;
          u[j] = (mok && k < op.kdim)
                     ? *reinterpret_cast<const uint32_t*>(op.ptr + k * op.ld + m)
                     : 0u;
        }
      } else {
        // k-rows k0 + 4w + j, j = 0..3; one 64-bit pair (rows m, m+1) each.
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t k = k0 + 4 * w + j;
          uint2 p = make_uint2(0u, 0u);
          if (mok && k < op.kdim) p = *reinterpret_cast<const uint2*>(op.ptr + k * op.ld + m);
          u[2 * j] = p.x;
          u[2 * j + 1] = p.y;
        }
      }
    }
  }

  __device__ __forceinline__ void store(uint8_t* lds, int tid) const {
    if constexpr (KC) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int q = tid + kThreads * j;
        const int row = q >> 2, c = q & 3;
        *reinterpret_cast<uint4*>(lds + row * kRowBytes + c * 16) = r[j];
      }
    } else {
      const int lane = tid & 63, w = tid >> 6;
      const uint32_t* u = reinterpret_cast<const uint32_t*>(r);
      uint4 lo, hi;  // k-values of row 2L and of row 2L+1
      if constexpr (sizeof(T) == 2) {
        // u[j] = (row m at k_j) | (row m+1 at k_j) << 16
        lo.x = (u[0] & 0xffffu) | (u[1] << 16);
        lo.y = (u[2] & 0xffffu) | (u[3] << 16);
        lo.z = (u[4] & 0xffffu) | (u[5] << 16);
        lo.w = (u[6] & 0xffffu) | (u[7] << 16);
        hi.x = (u[0] >> 16) | (u[1] & 0xffff0000u);
        hi.y = (u[2] >> 16) | (u[3] & 0xffff0000u);
        hi.z = (u[4] >> 16) | (u[5] & 0xffff0000u);
        hi.w = (u[6] >> 16) | (u[7] & 0xffff0000u);
      } else {
        // u[2j] = row m at k_j, u[2j+1] = row m+1 at k_j
        lo = make_uint4(u[0], u[2], u[4], u[6]);
        hi = make_uint4(u[1], u[3], u[5], u[7]);
      }
      *reinterpret_cast<uint4*>(lds + (2 * lane) * kRowBytes + w * 16) = lo;
      *reinterpret_cast<uint4*>(lds + (2 * lane + 1) * kRowBytes + w * 16) = hi;
    }
  }
};

// One K step of MFMAs: acc[g] += A_tile * B_tile[g]^T for every B operand g.
// Lane l reads 16-byte chunk l / 16 of rows l % 16 of each 16-row block. For
// bf16 that is the 8 k values of one 16x16x32 MFMA; for fp32 the 4 k values
// feed 4 MFMAs of 16x16x4, MFMA e taking element e (k = 4 (l / 16) + e), the
// same order for both operands, so the sum over k is unchanged.
template <typename T, int NB>
__device__ __forceinline__ void mma_step(const uint8_t* ldsA, const uint8_t* ldsB0,
                                         f32x4 (&acc)[NB][4][4], int wm, int wn, int lane) {
  const int r = lane & 15, cb = (lane >> 4) * 16;
  if constexpr (sizeof(T) == 2) {
    bf16x8 a[4], b[NB][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      a[mb] = *reinterpret_cast<const bf16x8*>(ldsA + (wm * 64 + mb * 16 + r) * kRowBytes + cb);
#pragma unroll
    for (int g = 0; g < NB; ++g)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        b[g][nb] = *reinterpret_cast<const bf16x8*>(ldsB0 + g * kTileBytes +
                                                    (wn * 64 + nb * 16 + r) * kRowBytes + cb);
#pragma unroll
    for (int g = 0; g < NB; ++g)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[g][mb][nb] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb], b[g][nb], acc[g][mb][nb], 0, 0, 0);
  } else {
    f32x4 a[4], b[NB][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      a[mb] = *reinterpret_cast<const f32x4*>(ldsA + (wm * 64 + mb * 16 + r) * kRowBytes + cb);
#pragma unroll
    for (int g = 0; g < NB; ++g)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        b[g][nb] = *reinterpret_cast<const f32x4*>(ldsB0 + g * kTileBytes +
                                                   (wn * 64 + nb * 16 + r) * kRowBytes + cb);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int g = 0; g < NB; ++g)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            acc[g][mb][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[mb][e], b[g][nb][e],
                                                                 acc[g][mb][nb], 0, 0, 0);
  }
}

// acc[g] = A[a_row0 : a_row0+128, 0:K] * B[g][b_row0 : b_row0+128, 0:K]^T.
// `lds` holds 2 stages of (1 + NB) tiles. Ends with a barrier, so the caller
// may reuse `lds` right after.
template <typename T, bool AKC, bool BKC, int NB>
__device__ __forceinline__ void mainloop(const Operand<T, AKC>& A, const Operand<T, BKC>* B,
                                         int64_t a_row0, int64_t b_row0, int64_t K, uint8_t* lds,
                                         f32x4 (&acc)[NB][4][4], int tid) {
  constexpr int BK = Elem<T>::kBK;
  constexpr int kStage = (1 + NB) * kTileBytes;
  const int lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int g = 0; g < NB; ++g)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int x = 0; x < 4; ++x) acc[g][mb][nb][x] = 0.f;

  const int64_t nk = (K + BK - 1) / BK;
  Stager<T, AKC> sa;
  Stager<T, BKC> sb[NB];
  sa.load(A, a_row0, 0, tid);
#pragma unroll
  for (int g = 0; g < NB; ++g) sb[g].load(B[g], b_row0, 0, tid);
  sa.store(lds, tid);
#pragma unroll
  for (int g = 0; g < NB; ++g) sb[g].store(lds + (1 + g) * kTileBytes, tid);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    uint8_t* cur = lds + (kt & 1) * kStage;
    uint8_t* nxt = lds + ((kt + 1) & 1) * kStage;
    const bool more = kt + 1 < nk;
    if (more) {
      sa.load(A, a_row0, (kt + 1) * BK, tid);
#pragma unroll
      for (int g = 0; g < NB; ++g) sb[g].load(B[g], b_row0, (kt + 1) * BK, tid);
    }
    mma_step<T, NB>(cur, cur + kTileBytes, acc, wm, wn, lane);
    if (more) {
      sa.store(nxt, tid);
#pragma unroll
      for (int g = 0; g < NB; ++g) sb[g].store(nxt + (1 + g) * kTileBytes, tid);
    }
    __syncthreads();
  }
}

// Both tile geometries give each wave a 64 x 64 sub-tile of 4 x 4 blocks.
constexpr int kMB = 4, kNB = 4;
typedef f32x4 WaveAcc[kMB][kNB];

// Vocabulary row (within the tile) of accumulator register r of block mb.
__device__ __forceinline__ int acc_row(int wm, int mb, int r, int lane) {
  return wm * 64 + mb * 16 + 4 * (lane >> 4) + r;
}
// Token column (within the tile) of block nb.
__device__ __forceinline__ int acc_col(int wn, int nb, int lane) { return wn * 64 + nb * 16 + (lane & 15); }

}  // namespace kd
