/*
 * kd_loss.h — C ABI of the fused LM-head + cross-entropy + KL distillation loss
 * for AMD MI355X (gfx950).
 *
 * What it computes (sources are the four pages this library follows, cited by
 * page title and section):
 *
 *   z = H_s W^T (student logits, never stored), t = teacher logits:
 *     TIED      t = H_t W^T      (orda-kernel, Teacher descriptors: TiedTeacher)
 *     SEPARATE  t = H_t W_t^T    (orda-kernel, Teacher descriptors: SeparateTeacher;
 *                                 the hidden+weight form of PrecomputedTeacher)
 *     TOPK      cached (idx, p)  (CompactifAI/Full-Chunked-KL-Loss, Methods)
 *   per token i, with valid_i = (y_i != ignore_index and 0 <= y_i < V):
 *     student_ce_i = valid_i * (lse(z_i) - z_i[y_i])              (T = 1)
 *     teacher_ce_i = valid_i * (lse(t_i) - t_i[y_i])              (T = 1)
 *     kl_i = T^2 * KL(softmax(t_i/T) || softmax(z_i/T))   for every row
 *            (nemo kd_loss, KDLoss temperature; orda-kernel, KL variants "forward")
 *     TOPK: kl_i = sum_k p log p - sum_k p z[idx_k] + M_i lse(z_i), M_i = sum_k p
 *            (CompactifAI/Full-Chunked-KL-Loss, Methods: objective)
 *   loss = sum_i valid_i (w_s student_ce_i + w_t teacher_ce_i + w_kl kl_i) / den
 *     den = normalizer if > 0 (nemo kd_loss, KDLoss.forward num_batch_labels),
 *           max(n_valid, 1) for MEAN, 1 for SUM (orda-kernel, Parameters: reduction).
 *   Gradients (teacher detached; CompactifAI/Full-Chunked-KL-Loss, Full Chunked KL):
 *     dz_i = (g / den) valid_i [w_s (softmax z_i - e_y) + w_kl T (softmax(z_i/T) - softmax(t_i/T))]
 *     TOPK: dz_i = (g / den) w_kl (M_i softmax z_i - p_i scattered)
 *     dH = dZ W,  dW = dZ^T H_s.
 *
 * The (n, v) logits are never materialised: the forward streams vocabulary
 * tiles through registers with online (max, rescaled sum) statistics
 * (flash_kd, module description), and the backward recomputes each vocabulary
 * chunk and writes only an (n, chunk) gradient slab (with keep_last_chunk, the
 * forward's last chunk is read back from `saved` instead of recomputed).
 *
 * Conventions.
 *   - Every pointer in the structs below is a DEVICE pointer, except the
 *     structs themselves and the host pointers named as such.
 *   - Row-major everywhere: hidden [n, d], weight [v, d], logits [n, v],
 *     topk_idx / topk_prob [n, k], labels [n].
 *   - The caller allocates and owns every buffer (inputs, outputs, saved,
 *     workspace). The library never allocates, frees or synchronises, except
 *     kd_read_status, which synchronises the stream it is given.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = default stream)
 *     and returns before it runs. Calls that overlap in time need distinct
 *     workspaces. Inputs are read only; outputs are overwritten (except dH/dW
 *     with accumulate = 1).
 *   - Results are deterministic: no atomics, fixed reduction orders.
 *   - Errors found on the host return synchronously before anything is
 *     enqueued. A label outside [0, v) that is not ignore_index, or a top-K
 *     index outside [0, v), is treated as ignored / skipped and raises a device
 *     flag read by kd_read_status; such values are never used as addresses
 *     (orda-kernel, Parameters: ignore_index).
 *   - No C++ exception crosses this interface.
 */
#ifndef KD_LOSS_H
#define KD_LOSS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kd_status;
enum {
  KD_OK = 0,
  KD_ERR_NULL = 1,         /* a required pointer is NULL */
  KD_ERR_SHAPE = 2,        /* n, d, v, d_t or k out of range, or inconsistent */
  KD_ERR_DTYPE = 3,        /* unknown dtype, or a mode that does not accept it */
  KD_ERR_PARAM = 4,        /* temperatures/weights not finite or not allowed, bad reduction or KL variant */
  KD_ERR_ALIGN = 5,        /* a pointer not 16-byte aligned, or d / d_t not a multiple of 8 */
  KD_ERR_WORKSPACE = 6,    /* workspace smaller than kd_workspace_bytes, or saved missing */
  KD_ERR_UNSUPPORTED = 7,  /* valid but not provided (backward of the logits scorer, a non-forward KL with a TOPK teacher) */
  KD_ERR_LABEL_RANGE = 8,  /* device flag: a label or top-K index was out of range */
  KD_ERR_HIP = 9,          /* a HIP launch or runtime call failed */
  KD_ERR_SAVED = 10        /* device flag: a backward that reads kept products found `saved`
                              without kept products of its layout (see keep_last_chunk) */
};

/* Element type of hidden / weight / logits. Accumulation is always fp32. */
enum { KD_F32 = 0, KD_BF16 = 1 };

/* Student side. PROJECTION: logits z = hidden @ weight^T (forward + backward).
 * LOGITS: z is given as `logits` [n, v], with a SEPARATE teacher (flash_kd,
 * flash_ce_kd_loss: student_logits; forward only) or a LOGITS teacher (nemo
 * kd_loss, KDLoss.forward: student_logits and teacher_logits; the gradient to
 * the student logits comes from kd_loss_bwd_logits). */
enum { KD_STUDENT_PROJECTION = 0, KD_STUDENT_LOGITS = 1 };

/* Teacher descriptor kinds (orda-kernel, Teacher descriptors). LOGITS is the
 * cached dense form of PrecomputedTeacher: teacher logits [n, v] given
 * directly, read tile by tile in place of the teacher projection; it needs a
 * PROJECTION student. */
enum { KD_TEACHER_TIED = 1, KD_TEACHER_SEPARATE = 2, KD_TEACHER_TOPK = 3, KD_TEACHER_LOGITS = 4 };

/* Loss reduction (orda-kernel, Parameters: reduction). NONE produces the
 * per-token outputs and the sum in `loss`; it has no backward. */
enum { KD_REDUCE_MEAN = 0, KD_REDUCE_SUM = 1, KD_REDUCE_NONE = 2 };

/* KL variant of the distillation term (orda-kernel, KL variants; p = student
 * softmax(z / T), q = teacher softmax(t / T_t), T_t = teacher_temperature or
 * T). FORWARD is KL(q || p), REVERSE KL(p || q), JEFFREYS their sum; the
 * per-token value and the loss carry T^2 (orda-kernel, Parameters: each KL row
 * scales by T_s^2), and the teacher is always detached. A TOPK teacher allows
 * FORWARD only (its distribution is zero off the support). */
enum { KD_KL_FORWARD = 0, KD_KL_REVERSE = 1, KD_KL_JEFFREYS = 2 };

typedef struct {
  int32_t kind;        /* KD_STUDENT_* */
  int32_t dtype;       /* KD_F32 | KD_BF16: hidden, weight, logits and the teacher tensors */
  int64_t n;           /* tokens (flattened batch x sequence), 1 <= n < 2^31 */
  int64_t d;           /* student hidden size (PROJECTION), multiple of 8 */
  int64_t v;           /* vocabulary size, 1 <= v < 2^31 */
  const void* hidden;  /* [n, d]  PROJECTION */
  const void* weight;  /* [v, d]  PROJECTION */
  const void* logits;  /* [n, v]  LOGITS */
} kd_student;

typedef struct {
  int32_t kind;             /* KD_TEACHER_* */
  int32_t k;                /* TOPK: entries per row, 1 <= k <= v */
  int64_t d_t;              /* SEPARATE: teacher hidden size (multiple of 8); TIED: 0 or d */
  const void* hidden;       /* TIED [n, d], SEPARATE [n, d_t]; student dtype */
  const void* weight;       /* SEPARATE [v, d_t]; student dtype */
  const int32_t* topk_idx;  /* TOPK [n, k], distinct per row */
  const float* topk_prob;   /* TOPK [n, k], not renormalised (sum = retained mass M) */
  const void* logits;       /* LOGITS [n, v] row-major, student dtype, element-aligned. A -inf
                               entry is a zero teacher probability: it adds 0 to the forward KL
                               and makes the reverse KL +inf. Every row needs a finite entry.
                               With a PROJECTION student the tiles read it in place of the
                               teacher projection; with a LOGITS student (both given) row
                               kernels stream the two matrices (no GEMM). */
} kd_teacher;

typedef struct {
  float student_ce_weight;   /* w_s >= 0, finite (orda-kernel, Parameters) */
  float teacher_ce_weight;   /* w_t >= 0; the teacher is detached: no gradient */
  float kl_weight;           /* w_kl >= 0 */
  float temperature;         /* T > 0, finite; TOPK requires T == 1 */
  int64_t ignore_index;      /* label value excluded from CE and from the loss */
  int32_t reduction;         /* KD_REDUCE_* */
  float normalizer;          /* > 0: divide the summed loss by it (num_batch_labels) */
  int64_t vocab_chunk;       /* vocabulary columns per chunk, rounded up to whole tiles; 0 =
                                library default (16384, flash_kd's chunk_size default). The
                                backward's dz slab holds n x chunk; the forward runs one tile
                                launch per chunk and keeps one chunk's tile records (40 bytes
                                per token and 256 columns). */
  int32_t assume_valid_labels; /* accepted and ignored (orda-kernel, Parameters: the flag lets a
                                caller skip label validation). Labels are always range-checked:
                                the check is one compare per row, and an unchecked label would
                                become a memory address (z[y] reads row y of the weight). */
  int32_t kl_divergence;     /* KD_KL_* */
  float teacher_temperature; /* T_t > 0, finite: the teacher's own temperature (orda-kernel,
                                Parameters: kl_teacher_temperature); 0 = T. TOPK: 0 or 1 */
  int32_t compact_valid;     /* 1: rows whose label is ignored (or out of range) are left out of
                                every projection and GEMM (orda-kernel, Parameters: ignore_index is
                                excluded from CE and KL); their per-token outputs are 0, the loss
                                and gradients are unchanged. TIED and SEPARATE teachers with labels
                                only (else KD_ERR_UNSUPPORTED); workspaces grow by
                                8 n + 16 ceil(n/128) (d + d_t) bytes (bf16). 0: every row is
                                projected and its KL reported. */
  int32_t keep_last_chunk;   /* 1: kd_loss_fwd also writes the fp32 products of its last
                                vocabulary chunk (student, and the teacher's for TIED and
                                SEPARATE teachers) into `saved`, and the backward calls read
                                them there instead of recomputing that chunk's products. The
                                chunk runs last in the forward and its products are the same
                                accumulators either way, so every result is bit-identical to
                                keep_last_chunk = 0; saved grows to kd_saved_bytes_for (4 bytes
                                per token row, rounded up to 128 rows, per column of the last
                                chunk rounded up to whole tiles, per product). Takes effect for
                                PROJECTION students when `saved` is given; no effect otherwise.
                                0: saved is kd_saved_bytes(n) and the backward recomputes every
                                chunk (CompactifAI/Full-Chunked-KL-Loss, Full Chunked KL:
                                logits are recomputed chunk by chunk in the backward). */
  int64_t saved_bytes;       /* bytes of the `saved` buffer the calls are given; with
                                keep_last_chunk taking effect, kd_loss_fwd, kd_loss_bwd and
                                kd_loss_bwd_teacher return KD_ERR_WORKSPACE before enqueuing
                                anything when it is below kd_saved_bytes_for. Not read
                                otherwise (0 is fine). */
  int32_t kl_output_unscaled; /* 1: the per-token `kl` output is the divergence without the
                                T^2 factor (flash_kd, flash_ce_kd_loss Returns: the KD term is
                                not multiplied by T^2); the loss and the gradients keep it.
                                0: the per-token kl includes T^2 (nemo kd_loss, KDLoss
                                temperature; orda-kernel, KL variants). */
  int32_t dh_dtype;          /* element type of the d_hidden output of kd_loss_bwd and
                                kd_loss_bwd_teacher: KD_F32 (0) or KD_BF16 (1). bf16 is the fp32
                                result rounded once to nearest even: dH sums its vocabulary
                                chunks in an fp32 buffer of the workspace (n x max(d, d_t) x 4
                                bytes more when there are several chunks) and rounds at the
                                last one; with accumulate = 1 the old bf16 value is added in
                                fp32 before that rounding. */
  int32_t dw_dtype;          /* element type of the d_weight output, as dh_dtype: each
                                vocabulary row is written once per call, rounded once (with
                                accumulate = 1, old value + new in fp32, then rounded). */
} kd_params;

/* Forward outputs, all device pointers, each nullable (NULL = not written).
 * loss: one fp32; student_ce, teacher_ce, kl: fp32 [n]. The per-token kl
 * includes T^2 and is given for every row, ignored ones too; the CE terms are
 * 0 on ignored rows (flash_kd, flash_ce_kd_loss: labels and Returns). */
typedef struct {
  float* loss;
  float* student_ce;
  float* teacher_ce;
  float* kl;
} kd_outputs;

/* Optional timing hook for profiling. When non-NULL, the library records
 * events[count] before and events[count+1] after each launch whose class bit
 * is set in `mask`, stores the class in kinds[count/2] and adds 2 to count,
 * while count + 2 <= capacity. Events are hipEvent_t handles made by
 * kd_events_create; `kinds` is a host array of capacity/2 entries. */
enum {
  KD_KERNEL_PREP = 0,      /* label logits, validity, top-K sums */
  KD_KERNEL_FWD = 1,       /* forward projection tiles + online-softmax epilogue */
  KD_KERNEL_MERGE = 2,     /* per-token merge of the vocabulary-tile records */
  KD_KERNEL_FINALIZE = 3,  /* loss reduction */
  KD_KERNEL_BWD_DZ = 4,    /* backward recompute tiles + logit-gradient epilogue */
  KD_KERNEL_SCATTER = 5,   /* reserved (the top-K p is subtracted inside the dz epilogue) */
  KD_KERNEL_GEMM_DW = 6,   /* dW[chunk] = dZ_chunk^T H */
  KD_KERNEL_GEMM_DH = 7,   /* dH += dZ_chunk W[chunk] */
  KD_KERNEL_GEMM_DWDH = 8, /* both GEMMs of a chunk in one launch */
  KD_KERNEL_BWD_KEPT = 9   /* logit-gradient epilogue on the kept last chunk (keep_last_chunk) */
};
typedef struct {
  void** events;     /* host array of hipEvent_t */
  int32_t* kinds;    /* host array */
  int32_t capacity;  /* number of entries in events */
  int32_t count;     /* events recorded so far (updated by the library) */
  uint32_t mask;     /* bit KD_KERNEL_x set: bracket launches of that class */
} kd_trace;

/* Bytes of device workspace one call needs (for_backward = 0: kd_loss_fwd,
 * 1: kd_loss_bwd). Validates the descriptors like the calls do. */
kd_status kd_workspace_bytes(const kd_student* s, const kd_teacher* t, const kd_params* p,
                             int32_t for_backward, size_t* bytes /* host */);

/* Bytes of the buffer that carries per-row statistics from forward to
 * backward: 20 per row plus a 64-byte header, enough whenever keep_last_chunk
 * is 0 (else see kd_saved_bytes_for). One backward per forward (orda-kernel,
 * Quickstart: each fused forward supports one backward pass). */
size_t kd_saved_bytes(int64_t n);

/* Bytes of `saved` for these descriptors and params: kd_saved_bytes(n), plus
 * the kept products of the last chunk when keep_last_chunk takes effect.
 * Validates the descriptors like the calls do; *bytes is host memory. */
kd_status kd_saved_bytes_for(const kd_student* s, const kd_teacher* t, const kd_params* p,
                             size_t* bytes /* host */);

/* Forward: per-token outputs, the reduced loss, and `saved` for the backward
 * (saved may be NULL when no backward follows). labels: int64 [n]; NULL means
 * every row is valid and no CE is computed (then w_s and w_t must be 0); TOPK
 * takes no labels. workspace: ws_bytes >= kd_workspace_bytes(..., 0). */
kd_status kd_loss_fwd(const kd_student* s, const kd_teacher* t, const kd_params* p,
                      const int64_t* labels, const kd_outputs* out, void* saved,
                      void* workspace, size_t ws_bytes, void* stream, kd_trace* trace);

/* kd_loss_fwd without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation). The forward's workspace is a library-owned scratch
 * array of 64 MiB per device (allocated with the library's device code on
 * each device it runs on and held until the process ends); the call itself
 * allocates and frees nothing. Same arguments and results as kd_loss_fwd
 * (the outputs and `saved` are bit-identical), with the current device the
 * one `stream` runs on. Returns KD_ERR_WORKSPACE, before enqueuing
 * anything, when kd_workspace_bytes(..., 0) for these descriptors exceeds
 * 64 MiB (about 2.5 KB per token at the default vocab_chunk of 16384 with a
 * 256-column tile; a smaller vocab_chunk shrinks it). device_flags (device
 * int32, nullable) receives the flag word kd_read_status would report (bit 0:
 * a label or top-K index out of range). Every call on a device shares that
 * device's scratch and leaves its contents behind: calls that overlap in time
 * on one device race and must be serialised (one stream, or events). */
kd_status kd_loss_fwd_noalloc(const kd_student* s, const kd_teacher* t, const kd_params* p,
                              const int64_t* labels, const kd_outputs* out, void* saved,
                              int32_t* device_flags, void* stream, kd_trace* trace);

/* Backward of the reduced loss to the student hidden states and weight.
 * saved: written by the matching kd_loss_fwd with the same inputs and params.
 * grad_loss: device fp32 scalar (upstream gradient of loss), NULL = 1.
 * d_hidden: [n, d], d_weight: [v, d], row-major, of the element types
 * kd_params.dh_dtype / dw_dtype (fp32 by default), 16-byte aligned, each
 * nullable (NULL = skip).
 * accumulate = 1 adds into d_hidden / d_weight (orda-kernel, Parameters:
 * KernelConfig weight-gradient accumulation); 0 overwrites.
 * Not available for LOGITS students or REDUCE_NONE (KD_ERR_UNSUPPORTED). */
kd_status kd_loss_bwd(const kd_student* s, const kd_teacher* t, const kd_params* p,
                      const int64_t* labels, const void* saved, const float* grad_loss,
                      void* d_hidden, void* d_weight, int32_t accumulate,
                      void* workspace, size_t ws_bytes, void* stream, kd_trace* trace);

/* Backward to given student logits (nemo kd_loss, KDLoss: the loss is
 * differentiated in student_logits): LOGITS student with a LOGITS teacher.
 * d_logits: [n, v] in the student dtype (bf16 rounded to nearest even),
 * row-major, overwritten (accumulate = 0) or added to (1); NULL = nothing.
 * saved and grad_loss as for kd_loss_bwd; no workspace is needed. Not for
 * REDUCE_NONE (KD_ERR_UNSUPPORTED). */
kd_status kd_loss_bwd_logits(const kd_student* s, const kd_teacher* t, const kd_params* p,
                             const int64_t* labels, const void* saved, const float* grad_loss,
                             void* d_logits, int32_t accumulate, void* stream, kd_trace* trace);

/* Backward to a teacher trained through its CE (orda-kernel, Teacher
 * descriptors: with teacher_ce_weight > 0 the teacher trains via CE; the KL
 * variants here detach the teacher, so only w_t CE(t) at T = 1 reaches it).
 * TIED or SEPARATE teacher, PROJECTION student, same arguments as kd_loss_bwd
 * (the same workspace size serves). d_teacher_hidden: [n, d_t];
 * d_teacher_weight: [v, d_t], of the types dh_dtype / dw_dtype (TIED: d_t = d and this is the teacher
 * half of the shared weight's gradient: pass d_weight with accumulate = 1
 * after kd_loss_bwd to sum the halves). Each nullable; accumulate as above.
 * With teacher_ce_weight = 0 the gradients are 0. */
kd_status kd_loss_bwd_teacher(const kd_student* s, const kd_teacher* t, const kd_params* p,
                              const int64_t* labels, const void* saved, const float* grad_loss,
                              void* d_teacher_hidden, void* d_teacher_weight, int32_t accumulate,
                              void* workspace, size_t ws_bytes, void* stream, kd_trace* trace);

/* Synchronises `stream`, then reads the device flags left in `workspace` by
 * the last call that used it (a backward that computes no logit gradient,
 * as with a zero teacher-CE weight, leaves them as they were): *flags (host,
 * nullable) receives them. Bit 0, set by
 * kd_loss_fwd: a label or top-K index was out of range (returns
 * KD_ERR_LABEL_RANGE). Bit 1, set by kd_loss_bwd / kd_loss_bwd_teacher with
 * keep_last_chunk: `saved` was not written by a forward that kept its last
 * chunk with the same vocab_chunk and n; the gradients are then NaN rather
 * than silently wrong (returns KD_ERR_SAVED). */
kd_status kd_read_status(const void* workspace, void* stream, int32_t* flags);

/* Static description of a status code. */
const char* kd_status_string(kd_status st);

/* 1 if `device` is a gfx950 GPU this library was built for, else 0
 * (cf. orda-kernel, Installation: is_available). */
int32_t kd_device_supported(int32_t device);

/* Timing helpers for kd_trace: create / destroy n timing events, and the
 * elapsed milliseconds between two recorded events (waits for the second). */
kd_status kd_events_create(void** events /* host [n] */, int32_t n);
kd_status kd_events_destroy(void** events, int32_t n);
kd_status kd_event_elapsed_ms(void* start, void* stop, float* ms /* host */);

/* Library version string, e.g. "0.1.0 gfx950". */
const char* kd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KD_LOSS_H */
