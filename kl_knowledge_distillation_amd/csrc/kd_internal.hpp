// Internal plan shared by the C ABI (kd_api.cpp) and the launchers
// (kd_kernels.hip). Not part of the public interface.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "kd_loss.h"

namespace kd {

// TIED / SEPARATE / TOPK: projection student with that teacher; LOGITS: given
// student logits with a separate teacher (forward only); TLOGITS: projection
// student with given dense teacher logits.
enum Mode { MODE_TIED = 0, MODE_SEPARATE = 1, MODE_TOPK = 2, MODE_LOGITS = 3, MODE_TLOGITS = 4,
            MODE_TCE = 5 /* backward only: the teacher tile and its CE gradient */,
            MODE_BOTH = 6 /* student and teacher logits both given: row kernels, no GEMM */ };

// Number of fp32 fields of one per-(token, vocabulary tile) record.
constexpr int kRecFields = 10;
// Tokens per merge workgroup; also the number of partial sums per block.
constexpr int kMergeThreads = 256;
constexpr int kMergeTok = 16;  // tokens per merge workgroup
// Bytes reserved at the start of the workspace for device flags (int32 at 0)
// and the compacted row count (int32 at kNvOffset).
constexpr size_t kStatusBytes = 256;
constexpr size_t kNvOffset = 8;
// `saved`: [n] x 16 bytes of row statistics, a 64-byte header at 16 n, then
// [n] fp32 lse(t) at T = 1 (the teacher-CE backward) at 16 n + 64.
constexpr size_t kSavedHeaderBytes = 64;
// Header words (4 bytes each, from 16 n): 0 den, 1 n_valid, 2 n_bad (fp32);
// 4..8 the layout of the kept products (int32): kKeepMagic or 0, chunk,
// keep_ld, keep_ops, n. A backward that reads kept products checks them.
constexpr int kHdrKeep = 4;
constexpr int32_t kKeepMagic = 0x4b454550;
// Device flag bits of the workspace's first word (kd_read_status).
constexpr int32_t kFlagRange = 1;  // forward: a label or top-K index out of range
constexpr int32_t kFlagSaved = 2;  // backward: `saved` holds no kept products of this layout
// Given-logits row kernels: one wave per (row, slice of the row); each lane
// takes kRowUnroll 16-byte chunks of each matrix per step, and a launch aims
// at about kRowWaves waves (8 per SIMD over 256 CUs, twice over).
#ifndef KD_ROW_UNROLL
#define KD_ROW_UNROLL 2
#endif
#ifndef KD_ROW_WAVES
#define KD_ROW_WAVES 16384
#endif
constexpr int kRowUnroll = KD_ROW_UNROLL;
constexpr int64_t kRowWaves = KD_ROW_WAVES;
// Elements of one row kernel step of a wave (64 lanes x kRowUnroll chunks).
constexpr int64_t row_step_elems(int dtype) { return kRowUnroll * 64 * (dtype == KD_BF16 ? 8 : 4); }

struct Plan {
  int mode = 0;
  int dtype = 0;  // KD_F32 | KD_BF16
  int64_t n = 0, d = 0, dt = 0, v = 0;
  int k = 0;
  float ws = 0.f, wt = 0.f, wkl = 0.f, T = 1.f;
  float Tt = 1.f;     // teacher temperature (T unless set apart)
  int64_t ignore = -100;
  int reduction = KD_REDUCE_MEAN;
  float normalizer = 0.f;
  int kl = KD_KL_FORWARD;  // KD_KL_*
  int kl_unscaled = 0;     // the per-token kl output without the T^2 factor
  int dh_bf16 = 0, dw_bf16 = 0;  // gradient outputs in bf16 (else fp32)
  int need_zT = 0;    // statistics at z/T kept apart from z (T != 1, or a reverse-direction KL)
  int need_t1 = 0;    // teacher statistics at t kept apart from t/T_t (T_t != 1)
  int has_labels = 0;
  int compact = 0;    // rows with an ignored label left out of the tiles and GEMMs
  int pipe = 0;       // bf16 with hidden sizes multiple of 32: 256-row pipelined tiles
  int vt_rows = 128;  // vocabulary rows per fused tile
  int n_ttiles = 0, n_vtiles = 0, tps = 1, n_slices = 0;  // forward grid
  int64_t row_slice = 0;  // row kernels: elements per slice (a whole number of steps)
  // forward tiles: vocabulary tiles per launch (one chunk of `chunk` columns);
  // with several launches each chunk's records are folded into a running record
  int fwd_slices = 0;
  int64_t chunk = 0;  // backward vocabulary chunk (multiple of the fused tile rows)
  int tt_rows = 128;     // token rows per fused tile
  int64_t dz_rows = 0;  // rows of the logit-gradient slab: n rounded up to the token tile
  int n_chunks = 0;
  int merge_blocks = 0;
  // forward workspace layout (bytes from the workspace base)
  size_t off_prep = 0, off_rec = 0, off_part = 0, fwd_bytes = 0;
  size_t off_run = 0;  // running record [kRecFields][n] (several forward launches)
  // top-K: each row's entries sorted by vocabulary index (int32 idx [n][k], then
  // fp32 prob [n][k]) and where each vocabulary tile of one forward launch
  // starts its run of them (int32 [n][fwd_slices + 1])
  size_t off_tks = 0, off_tko = 0;
  // backward workspace layout; top-K: the row entries sorted again (off_btks,
  // as off_tks) and where each tile of one chunk starts its run (off_btko,
  // int32 [n][chunk / vt_rows + 1]), so the dz epilogue subtracts p itself
  size_t off_dz = 0, bwd_bytes = 0;
  size_t off_btks = 0, off_btko = 0;
  // bf16 dH with several chunks: the chunks' fp32 sum [n][max(d, dt)] (off_dhacc)
  size_t off_dhacc = 0;
  // Kept products of the last chunk in `saved` (keep_last_chunk): keep_ops
  // fp32 [dz_rows][keep_ld] matrices (student, then teacher) from byte keep_off.
  int keep = 0, keep_ops = 0;
  int64_t keep_ld = 0;
  size_t keep_off = 0, saved_bytes = 0;
  // compaction buffers (same offsets in both workspaces): idx, pos [n] int32,
  // compacted H_s [dz_rows x d] and H_t [dz_rows x dt] in the input dtype
  size_t off_cidx = 0, off_cpos = 0, off_hc = 0, off_htc = 0;
};

struct Tensors {
  const void* hs = nullptr;      // student hidden [n, d]
  const void* w = nullptr;       // student weight [v, d]
  const void* logits = nullptr;  // student logits [n, v]
  const void* ht = nullptr;      // teacher hidden [n, d_t]
  const void* wt = nullptr;      // teacher weight [v, d_t] (tied: == w)
  const void* tlogits = nullptr; // dense teacher logits [n, v]
  const int32_t* topk_idx = nullptr;
  const float* topk_prob = nullptr;
  const int64_t* labels = nullptr;
};

// Vocabulary rows per tile of the pipelined bf16 geometry compiled in.
int pipe_vocab_rows();
// Token rows per fused tile for a mode (pipe: the pipelined bf16 geometry).
int fused_token_rows(int mode, int pipe);
// Contraction lengths of the pipelined path are multiples of this (one K step).
constexpr int kPipeK = 64;

// status_out: where the forward's device flags go (null: the workspace's first word).
kd_status run_forward(const Plan& p, const Tensors& x, const kd_outputs* out, void* saved,
                      void* workspace, hipStream_t stream, kd_trace* trace,
                      int32_t* status_out = nullptr);
// The no-allocation forward's scratch: kScratchBytes of device memory per
// device; scratch_address gives the current device's address (looked up once
// per device), or null with *st set.
constexpr size_t kScratchBytes = (size_t)64 << 20;
void* scratch_address(kd_status* st);
kd_status run_backward(const Plan& p, const Tensors& x, const void* saved, const float* grad_loss,
                       void* d_hidden, void* d_weight, int accumulate, void* workspace,
                       hipStream_t stream, kd_trace* trace);
// The backward to given student logits (student and teacher logits given).
kd_status run_backward_logits(const Plan& p, const Tensors& x, const void* saved,
                              const float* grad_loss, void* d_logits, int accumulate,
                              hipStream_t stream, kd_trace* trace);
// The teacher-CE backward: d_hidden / d_weight are the teacher's.
kd_status run_backward_teacher(const Plan& p, const Tensors& x, const void* saved,
                               const float* grad_loss, void* d_hidden, void* d_weight,
                               int accumulate, void* workspace, hipStream_t stream, kd_trace* trace);

}  // namespace kd
