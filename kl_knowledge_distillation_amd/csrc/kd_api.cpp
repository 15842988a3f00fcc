// C ABI of the distillation-loss library: argument validation, launch
// planning and workspace sizing. Every check here runs on the host before
// anything is enqueued, so invalid calls never reach the GPU.
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <string.h>

#include <algorithm>

#include "kd_internal.hpp"

namespace {

using kd::Plan;

constexpr int64_t kMaxDim = (int64_t)1 << 31;
// Default backward chunk: flash_kd's chunk_size default (flash_ce_kd_loss). A
// 16384-column slab is n x 32 KB of bf16 (134 MB at 4096 tokens), and half as
// many chunks as 8192 save launches and tile tails (2.8% per quickstart step).
constexpr int64_t kDefaultChunk = 16384;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool finite_nonneg(float x) { return isfinite(x) && x >= 0.f; }

kd_status plan_call(const kd_student* s, const kd_teacher* t, const kd_params* p,
                    const int64_t* labels, bool check_labels_ptr, bool backward, Plan* out) {
  if (!s || !t || !p || !out) return KD_ERR_NULL;
  Plan q;
  if (s->dtype != KD_F32 && s->dtype != KD_BF16) return KD_ERR_DTYPE;
  q.dtype = s->dtype;
  if (s->n < 1 || s->n >= kMaxDim || s->v < 1 || s->v >= kMaxDim) return KD_ERR_SHAPE;
  q.n = s->n;
  q.v = s->v;
  const int64_t vec = (s->dtype == KD_BF16) ? 8 : 4;  // elements per 16-byte chunk

  if (s->kind == KD_STUDENT_PROJECTION) {
    if (!s->hidden || !s->weight) return KD_ERR_NULL;
    if (s->d < 1 || s->d >= kMaxDim) return KD_ERR_SHAPE;
    if (s->d % 8 != 0 || !aligned16(s->hidden) || !aligned16(s->weight)) return KD_ERR_ALIGN;
    q.d = s->d;
  } else if (s->kind == KD_STUDENT_LOGITS) {
    if (!s->logits) return KD_ERR_NULL;
    if (t->kind != KD_TEACHER_SEPARATE && t->kind != KD_TEACHER_LOGITS) return KD_ERR_UNSUPPORTED;
    // no hidden states or weight to differentiate (the scorer is forward only,
    // flash_kd; given student logits take kd_loss_bwd_logits)
    if (backward) return KD_ERR_UNSUPPORTED;
    if (((uintptr_t)s->logits & (s->dtype == KD_BF16 ? 1u : 3u)) != 0) return KD_ERR_ALIGN;
  } else {
    return KD_ERR_PARAM;
  }
  (void)vec;

  switch (t->kind) {
    case KD_TEACHER_TIED:
      if (s->kind != KD_STUDENT_PROJECTION) return KD_ERR_UNSUPPORTED;
      if (!t->hidden) return KD_ERR_NULL;
      if (t->d_t != 0 && t->d_t != s->d) return KD_ERR_SHAPE;
      if (!aligned16(t->hidden)) return KD_ERR_ALIGN;
      q.mode = kd::MODE_TIED;
      q.dt = s->d;
      break;
    case KD_TEACHER_SEPARATE:
      if (!t->hidden || !t->weight) return KD_ERR_NULL;
      if (t->d_t < 1 || t->d_t >= kMaxDim) return KD_ERR_SHAPE;
      if (t->d_t % 8 != 0 || !aligned16(t->hidden) || !aligned16(t->weight)) return KD_ERR_ALIGN;
      q.mode = (s->kind == KD_STUDENT_LOGITS) ? kd::MODE_LOGITS : kd::MODE_SEPARATE;
      q.dt = t->d_t;
      break;
    case KD_TEACHER_LOGITS:
      if (!t->logits) return KD_ERR_NULL;
      if (((uintptr_t)t->logits & (s->dtype == KD_BF16 ? 1u : 3u)) != 0) return KD_ERR_ALIGN;
      q.mode = (s->kind == KD_STUDENT_LOGITS) ? kd::MODE_BOTH : kd::MODE_TLOGITS;
      break;
    case KD_TEACHER_TOPK:
      if (s->kind != KD_STUDENT_PROJECTION) return KD_ERR_UNSUPPORTED;
      if (!t->topk_idx || !t->topk_prob) return KD_ERR_NULL;
      if (t->k < 1 || (int64_t)t->k > s->v) return KD_ERR_SHAPE;
      if (((uintptr_t)t->topk_idx & 3u) || ((uintptr_t)t->topk_prob & 3u)) return KD_ERR_ALIGN;
      q.mode = kd::MODE_TOPK;
      q.k = t->k;
      break;
    default:
      return KD_ERR_PARAM;
  }

  if (!isfinite(p->temperature) || p->temperature <= 0.f) return KD_ERR_PARAM;
  if (!isfinite(p->teacher_temperature) || p->teacher_temperature < 0.f) return KD_ERR_PARAM;
  if (!finite_nonneg(p->student_ce_weight) || !finite_nonneg(p->teacher_ce_weight) ||
      !finite_nonneg(p->kl_weight))
    return KD_ERR_PARAM;
  if (p->reduction != KD_REDUCE_MEAN && p->reduction != KD_REDUCE_SUM &&
      p->reduction != KD_REDUCE_NONE)
    return KD_ERR_PARAM;
  if (!isfinite(p->normalizer) || p->normalizer < 0.f) return KD_ERR_PARAM;
  if (p->vocab_chunk < 0) return KD_ERR_PARAM;
  if (p->kl_divergence != KD_KL_FORWARD && p->kl_divergence != KD_KL_REVERSE &&
      p->kl_divergence != KD_KL_JEFFREYS)
    return KD_ERR_PARAM;
  if (backward && p->reduction == KD_REDUCE_NONE) return KD_ERR_UNSUPPORTED;
  if (q.mode == kd::MODE_TOPK) {
    // The cached teacher has no temperature and no labels (Full-Chunked-KL-Loss, Methods).
    if (p->temperature != 1.f) return KD_ERR_UNSUPPORTED;
    if (p->teacher_temperature != 0.f && p->teacher_temperature != 1.f) return KD_ERR_UNSUPPORTED;
    // Its distribution is zero off the support: only KL(teacher || student) is finite.
    if (p->kl_divergence != KD_KL_FORWARD) return KD_ERR_UNSUPPORTED;
    if (p->student_ce_weight != 0.f || p->teacher_ce_weight != 0.f) return KD_ERR_PARAM;
    if (check_labels_ptr && labels) return KD_ERR_PARAM;
  } else if (check_labels_ptr && !labels &&
             (p->student_ce_weight != 0.f || p->teacher_ce_weight != 0.f)) {
    return KD_ERR_NULL;
  }
  if (check_labels_ptr && labels && ((uintptr_t)labels & 7u)) return KD_ERR_ALIGN;
  if (p->compact_valid != 0 && p->compact_valid != 1) return KD_ERR_PARAM;
  if (p->keep_last_chunk != 0 && p->keep_last_chunk != 1) return KD_ERR_PARAM;
  if (p->saved_bytes < 0) return KD_ERR_PARAM;
  if (p->kl_output_unscaled != 0 && p->kl_output_unscaled != 1) return KD_ERR_PARAM;
  if ((p->dh_dtype != KD_F32 && p->dh_dtype != KD_BF16) ||
      (p->dw_dtype != KD_F32 && p->dw_dtype != KD_BF16))
    return KD_ERR_DTYPE;
  if (p->compact_valid && q.mode != kd::MODE_TIED && q.mode != kd::MODE_SEPARATE)
    return KD_ERR_UNSUPPORTED;

  q.ws = p->student_ce_weight;
  q.wt = p->teacher_ce_weight;
  q.wkl = p->kl_weight;
  q.T = p->temperature;
  q.Tt = (p->teacher_temperature > 0.f) ? p->teacher_temperature : p->temperature;
  q.ignore = p->ignore_index;
  q.reduction = p->reduction;
  q.normalizer = p->normalizer;
  q.kl = p->kl_divergence;
  q.kl_unscaled = p->kl_output_unscaled;
  q.dh_bf16 = p->dh_dtype == KD_BF16;
  q.dw_bf16 = p->dw_dtype == KD_BF16;
  // Student statistics at z/T: needed for the KL at T != 1, and always for the
  // reverse direction, whose weights are the student's softmax(z/T).
  q.need_zT = (q.T != 1.f || q.kl != KD_KL_FORWARD) ? 1 : 0;
  // Teacher statistics at t (T = 1) beside those at t/T_t, for the teacher CE.
  q.need_t1 = (q.Tt != 1.f && q.mode != kd::MODE_TOPK) ? 1 : 0;
  q.has_labels = labels ? 1 : 0;
  // Without labels no row is ignored; the workspace query (labels unknown)
  // still reserves the compaction buffers.
  q.compact = (p->compact_valid && (labels || !check_labels_ptr)) ? 1 : 0;

  // Tile geometry: bf16 with every contraction length a multiple of 64 runs the
  // pipelined 256-row tiles; everything else the register-staged 128-row tiles.
  const bool d_ok = q.mode == kd::MODE_LOGITS || q.d % kd::kPipeK == 0;
  const bool dt_ok = (q.mode != kd::MODE_SEPARATE && q.mode != kd::MODE_LOGITS) || q.dt % kd::kPipeK == 0;
  q.pipe = (q.dtype == KD_BF16 && d_ok && dt_ok) ? 1 : 0;
  q.vt_rows = q.pipe ? kd::pipe_vocab_rows() : 128;
  const int64_t vt = q.vt_rows;
  // Forward grid: (vocabulary tile) x (128-token tile), one tile per workgroup,
  // so the per-token statistics are only live after the main loop; each
  // vocabulary tile leaves one record per token for the merge.
  q.tt_rows = kd::fused_token_rows(q.mode, q.pipe);
  q.n_ttiles = (int)ceil_div(q.n, q.tt_rows);
  q.n_vtiles = (int)ceil_div(q.v, vt);
  if (q.mode == kd::MODE_BOTH) {
    // Row kernels: each row split into slices of whole steps, enough of them
    // that the launch has about kRowWaves waves; one record per slice.
    const int64_t step = kd::row_step_elems(q.dtype);
    const int64_t steps = ceil_div(q.v, step);
    const int64_t want = std::min<int64_t>(steps, std::max<int64_t>(1, ceil_div(kd::kRowWaves, q.n)));
    q.row_slice = ceil_div(steps, want) * step;
    q.n_vtiles = (int)ceil_div(q.v, q.row_slice);
  }
  q.tps = 1;
  q.n_slices = q.n_vtiles;
  // Backward chunk: a whole number of fused vocabulary tiles.
  int64_t chunk = (p->vocab_chunk > 0) ? ceil_div(p->vocab_chunk, vt) * vt : kDefaultChunk;
  chunk = std::min<int64_t>(chunk, ceil_div(q.v, vt) * vt);
  q.chunk = chunk;
  q.n_chunks = (int)ceil_div(q.v, chunk);
  // The forward runs the same vocabulary chunks, one launch each, so its
  // records take O(N * chunk / vt_rows), not O(N * V / vt_rows).
  q.fwd_slices = (q.mode == kd::MODE_BOTH) ? q.n_slices : (int)std::min<int64_t>(q.n_vtiles, chunk / vt);
  q.merge_blocks = (int)ceil_div(q.n, kd::kMergeTok);

  const size_t elem = (q.dtype == KD_BF16) ? 2 : 4;
  q.dz_rows = (int64_t)q.n_ttiles * q.tt_rows;
  // Compaction buffers first, at the same offsets in both workspaces.
  size_t off = kd::kStatusBytes;
  if (q.compact) {
    q.off_cidx = off;
    off = align_up(off + 4 * (size_t)q.n, 256);
    q.off_cpos = off;
    off = align_up(off + 4 * (size_t)q.n, 256);
    q.off_hc = off;
    off = align_up(off + (size_t)q.dz_rows * (size_t)q.d * elem, 256);
    q.off_htc = off;
    off = align_up(off + (size_t)q.dz_rows * (size_t)q.dt * elem, 256);
  }
  const size_t off_common = off;
  q.off_prep = off;
  off = align_up(off + 4 * sizeof(float) * (size_t)q.n, 256);
  q.off_rec = off;
  off = align_up(off + (size_t)kd::kRecFields * q.fwd_slices * (size_t)q.n * sizeof(float), 256);
  if (q.fwd_slices < q.n_slices) {
    q.off_run = off;
    off = align_up(off + (size_t)kd::kRecFields * (size_t)q.n * sizeof(float), 256);
  }
  q.off_part = off;
  off = align_up(off + (size_t)q.merge_blocks * 4 * sizeof(double), 256);
  if (q.mode == kd::MODE_TOPK) {
    q.off_tks = off;
    off = align_up(off + 8 * (size_t)q.n * (size_t)q.k, 256);
    q.off_tko = off;
    off = align_up(off + 4 * (size_t)q.n * (size_t)(q.fwd_slices + 1), 256);
  }
  q.fwd_bytes = off;
  q.off_dz = off_common;
  off = align_up(q.off_dz + (size_t)q.dz_rows * (size_t)q.chunk * elem, 256);
  if (q.mode == kd::MODE_TOPK) {
    q.off_btks = off;
    off = align_up(off + 8 * (size_t)q.n * (size_t)q.k, 256);
    q.off_btko = off;
    off = align_up(off + 4 * (size_t)q.n * (size_t)(q.chunk / vt + 1), 256);
  }
  if (q.dh_bf16 && q.n_chunks > 1) {
    q.off_dhacc = off;
    off = align_up(off + 4 * (size_t)q.n * (size_t)std::max(q.d, q.dt), 256);
  }
  q.bwd_bytes = off;
  // The last chunk's products, kept in `saved` for the backward: columns of
  // that chunk rounded up to whole tiles, every row of the token tiles.
  q.saved_bytes = 20 * (size_t)q.n + kd::kSavedHeaderBytes;
  if (p->keep_last_chunk && (q.mode == kd::MODE_TIED || q.mode == kd::MODE_SEPARATE ||
                             q.mode == kd::MODE_TLOGITS || q.mode == kd::MODE_TOPK)) {
    q.keep = 1;
    q.keep_ops = (q.mode == kd::MODE_TIED || q.mode == kd::MODE_SEPARATE) ? 2 : 1;
    q.keep_ld = ceil_div(q.v - (int64_t)(q.n_chunks - 1) * q.chunk, vt) * vt;
    q.keep_off = align_up(q.saved_bytes, 256);
    q.saved_bytes = q.keep_off + (size_t)q.keep_ops * (size_t)q.dz_rows * (size_t)q.keep_ld * sizeof(float);
  }
  *out = q;
  return KD_OK;
}

kd::Tensors tensors_of(const kd_student* s, const kd_teacher* t, const int64_t* labels) {
  kd::Tensors x;
  x.hs = s->hidden;
  x.w = s->weight;
  x.logits = s->logits;
  x.labels = labels;
  if (t->kind == KD_TEACHER_TIED) {
    x.ht = t->hidden;
    x.wt = s->weight;
  } else if (t->kind == KD_TEACHER_SEPARATE) {
    x.ht = t->hidden;
    x.wt = t->weight;
  } else if (t->kind == KD_TEACHER_LOGITS) {
    x.tlogits = t->logits;
  } else {
    x.topk_idx = t->topk_idx;
    x.topk_prob = t->topk_prob;
  }
  return x;
}

}  // namespace

extern "C" {

kd_status kd_workspace_bytes(const kd_student* s, const kd_teacher* t, const kd_params* p,
                             int32_t for_backward, size_t* bytes) {
  if (!bytes) return KD_ERR_NULL;
  Plan q;
  const kd_status st = plan_call(s, t, p, nullptr, false, for_backward != 0, &q);
  if (st != KD_OK) return st;
  *bytes = for_backward ? q.bwd_bytes : q.fwd_bytes;
  return KD_OK;
}

size_t kd_saved_bytes(int64_t n) {
  if (n < 0) return 0;
  return 20 * (size_t)n + kd::kSavedHeaderBytes;
}

kd_status kd_saved_bytes_for(const kd_student* s, const kd_teacher* t, const kd_params* p,
                             size_t* bytes) {
  if (!bytes) return KD_ERR_NULL;
  Plan q;
  const kd_status st = plan_call(s, t, p, nullptr, false, false, &q);
  if (st != KD_OK) return st;
  *bytes = q.saved_bytes;
  return KD_OK;
}

kd_status kd_loss_fwd(const kd_student* s, const kd_teacher* t, const kd_params* p,
                      const int64_t* labels, const kd_outputs* out, void* saved, void* workspace,
                      size_t ws_bytes, void* stream, kd_trace* trace) {
  Plan q;
  const kd_status st = plan_call(s, t, p, labels, true, false, &q);
  if (st != KD_OK) return st;
  if (!workspace) return KD_ERR_NULL;
  if (ws_bytes < q.fwd_bytes) return KD_ERR_WORKSPACE;
  if (!aligned16(workspace) || (saved && !aligned16(saved))) return KD_ERR_ALIGN;
  // the kept products go past the row statistics: the caller must have said it has the room
  if (saved && q.keep && (size_t)p->saved_bytes < q.saved_bytes) return KD_ERR_WORKSPACE;
  if (out) {
    const void* ptrs[4] = {out->loss, out->student_ce, out->teacher_ce, out->kl};
    for (const void* ptr : ptrs)
      if (ptr && ((uintptr_t)ptr & 3u)) return KD_ERR_ALIGN;
  }
  return kd::run_forward(q, tensors_of(s, t, labels), out, saved, workspace,
                         static_cast<hipStream_t>(stream), trace);
}

kd_status kd_loss_fwd_noalloc(const kd_student* s, const kd_teacher* t, const kd_params* p,
                              const int64_t* labels, const kd_outputs* out, void* saved,
                              int32_t* device_flags, void* stream, kd_trace* trace) {
  Plan q;
  kd_status st = plan_call(s, t, p, labels, true, false, &q);
  if (st != KD_OK) return st;
  // the forward workspace must fit the library's per-device scratch
  if (q.fwd_bytes > kd::kScratchBytes) return KD_ERR_WORKSPACE;
  if (saved && !aligned16(saved)) return KD_ERR_ALIGN;
  if (saved && q.keep && (size_t)p->saved_bytes < q.saved_bytes) return KD_ERR_WORKSPACE;
  if (device_flags && ((uintptr_t)device_flags & 3u)) return KD_ERR_ALIGN;
  if (out) {
    const void* ptrs[4] = {out->loss, out->student_ce, out->teacher_ce, out->kl};
    for (const void* ptr : ptrs)
      if (ptr && ((uintptr_t)ptr & 3u)) return KD_ERR_ALIGN;
  }
  void* ws = kd::scratch_address(&st);
  if (ws == nullptr) return st;
  return kd::run_forward(q, tensors_of(s, t, labels), out, saved, ws,
                         static_cast<hipStream_t>(stream), trace, device_flags);
}

kd_status kd_loss_bwd(const kd_student* s, const kd_teacher* t, const kd_params* p,
                      const int64_t* labels, const void* saved, const float* grad_loss,
                      void* d_hidden, void* d_weight, int32_t accumulate, void* workspace,
                      size_t ws_bytes, void* stream, kd_trace* trace) {
  Plan q;
  const kd_status st = plan_call(s, t, p, labels, true, true, &q);
  if (st != KD_OK) return st;
  if (!saved) return KD_ERR_WORKSPACE;
  if (!workspace) return KD_ERR_NULL;
  if (ws_bytes < q.bwd_bytes) return KD_ERR_WORKSPACE;
  if (!aligned16(workspace) || !aligned16(saved)) return KD_ERR_ALIGN;
  if (q.keep && (size_t)p->saved_bytes < q.saved_bytes) return KD_ERR_WORKSPACE;
  if ((d_hidden && !aligned16(d_hidden)) || (d_weight && !aligned16(d_weight))) return KD_ERR_ALIGN;
  if (grad_loss && ((uintptr_t)grad_loss & 3u)) return KD_ERR_ALIGN;
  if (!d_hidden && !d_weight) return KD_OK;
  return kd::run_backward(q, tensors_of(s, t, labels), saved, grad_loss, d_hidden, d_weight,
                          accumulate ? 1 : 0, workspace, static_cast<hipStream_t>(stream), trace);
}

kd_status kd_loss_bwd_logits(const kd_student* s, const kd_teacher* t, const kd_params* p,
                             const int64_t* labels, const void* saved, const float* grad_loss,
                             void* d_logits, int32_t accumulate, void* stream, kd_trace* trace) {
  Plan q;
  const kd_status st = plan_call(s, t, p, labels, true, false, &q);
  if (st != KD_OK) return st;
  if (q.mode != kd::MODE_BOTH || p->reduction == KD_REDUCE_NONE) return KD_ERR_UNSUPPORTED;
  if (!saved) return KD_ERR_WORKSPACE;
  if (!aligned16(saved)) return KD_ERR_ALIGN;
  if (grad_loss && ((uintptr_t)grad_loss & 3u)) return KD_ERR_ALIGN;
  if (!d_logits) return KD_OK;
  if (((uintptr_t)d_logits & (s->dtype == KD_BF16 ? 1u : 3u)) != 0) return KD_ERR_ALIGN;
  return kd::run_backward_logits(q, tensors_of(s, t, labels), saved, grad_loss, d_logits,
                                 accumulate ? 1 : 0, static_cast<hipStream_t>(stream), trace);
}

kd_status kd_loss_bwd_teacher(const kd_student* s, const kd_teacher* t, const kd_params* p,
                              const int64_t* labels, const void* saved, const float* grad_loss,
                              void* d_teacher_hidden, void* d_teacher_weight, int32_t accumulate,
                              void* workspace, size_t ws_bytes, void* stream, kd_trace* trace) {
  Plan q;
  const kd_status st = plan_call(s, t, p, labels, true, true, &q);
  if (st != KD_OK) return st;
  if (q.mode != kd::MODE_TIED && q.mode != kd::MODE_SEPARATE) return KD_ERR_UNSUPPORTED;
  if (!labels && p->teacher_ce_weight != 0.f) return KD_ERR_NULL;
  if (!saved) return KD_ERR_WORKSPACE;
  if (!workspace) return KD_ERR_NULL;
  if (ws_bytes < q.bwd_bytes) return KD_ERR_WORKSPACE;
  if (!aligned16(workspace) || !aligned16(saved)) return KD_ERR_ALIGN;
  if (q.keep && (size_t)p->saved_bytes < q.saved_bytes) return KD_ERR_WORKSPACE;
  if ((d_teacher_hidden && !aligned16(d_teacher_hidden)) ||
      (d_teacher_weight && !aligned16(d_teacher_weight)))
    return KD_ERR_ALIGN;
  if (grad_loss && ((uintptr_t)grad_loss & 3u)) return KD_ERR_ALIGN;
  if (!d_teacher_hidden && !d_teacher_weight) return KD_OK;
  return kd::run_backward_teacher(q, tensors_of(s, t, labels), saved, grad_loss, d_teacher_hidden,
                                  d_teacher_weight, accumulate ? 1 : 0, workspace,
                                  static_cast<hipStream_t>(stream), trace);
}

kd_status kd_read_status(const void* workspace, void* stream, int32_t* flags) {
  if (!workspace) return KD_ERR_NULL;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return KD_ERR_HIP;
  int32_t f = 0;
  if (hipMemcpy(&f, workspace, sizeof(f), hipMemcpyDeviceToHost) != hipSuccess) return KD_ERR_HIP;
  if (flags) *flags = f;
  if (f & kd::kFlagSaved) return KD_ERR_SAVED;
  return (f & kd::kFlagRange) ? KD_ERR_LABEL_RANGE : KD_OK;
}

const char* kd_status_string(kd_status st) {
  switch (st) {
    case KD_OK: return "ok";
    case KD_ERR_NULL: return "a required pointer is NULL";
    case KD_ERR_SHAPE: return "shape out of range or inconsistent";
    case KD_ERR_DTYPE: return "unsupported dtype";
    case KD_ERR_PARAM: return "invalid parameter";
    case KD_ERR_ALIGN: return "misaligned pointer or hidden size not a multiple of 8";
    case KD_ERR_WORKSPACE: return "workspace too small or saved buffer missing";
    case KD_ERR_UNSUPPORTED: return "unsupported combination";
    case KD_ERR_LABEL_RANGE: return "a label or top-K index was out of range";
    case KD_ERR_HIP: return "HIP runtime error";
    case KD_ERR_SAVED: return "saved holds no kept products of this layout (forward/backward mismatch)";
    default: return "unknown status";
  }
}

int32_t kd_device_supported(int32_t device) {
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return 0;
  return strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
}

kd_status kd_events_create(void** events, int32_t n) {
  if (!events || n < 0) return KD_ERR_NULL;
  for (int32_t i = 0; i < n; ++i) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return KD_ERR_HIP;
    events[i] = e;
  }
  return KD_OK;
}

kd_status kd_events_destroy(void** events, int32_t n) {
  if (!events || n < 0) return KD_ERR_NULL;
  kd_status st = KD_OK;
  for (int32_t i = 0; i < n; ++i)
    if (events[i]) {
      if (hipEventDestroy(static_cast<hipEvent_t>(events[i])) != hipSuccess) st = KD_ERR_HIP;
      events[i] = nullptr;
    }
  return st;
}

kd_status kd_event_elapsed_ms(void* start, void* stop, float* ms) {
  if (!start || !stop || !ms) return KD_ERR_NULL;
  if (hipEventSynchronize(static_cast<hipEvent_t>(stop)) != hipSuccess) return KD_ERR_HIP;
  if (hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop)) !=
      hipSuccess)
    return KD_ERR_HIP;
  return KD_OK;
}

const char* kd_version(void) { return "0.1.0 gfx950"; }

}  // extern "C"
