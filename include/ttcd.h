/*
 * ttcd.h -- C ABI of the IP-TTCD layer forward for AMD Instinct MI355X (gfx950).
 *
 * IP-TTCD ("Learning What to Remember: Test-Time Training via Context
 * Distillation") runs one shared Q/K/V through causal sliding-window
 * attention twice -- a long teacher window w_T and a short student window
 * w_S -- and writes the teacher/student gap of the SwiGLU MLP activations
 * into the MLP down-projection as a chunk-wise fast weight.
 *
 * Conventions shared by every entry point
 *   - Every tensor is caller-owned DEVICE memory, row-major, contiguous,
 *     16-byte aligned.  The library allocates nothing, never synchronises
 *     the host and enqueues all work on `stream` (a hipStream_t; NULL is
 *     the default stream).
 *   - All arguments are validated on the host before anything is
 *     enqueued.  On error nothing is enqueued, outputs are untouched and
 *     ttcd_last_error() holds a message (thread-local).
 *   - Element types: TTCD_BF16 (bfloat16) or TTCD_F32.  Intermediate
 *     accumulation is fp32 in every kernel.
 *   - Outputs must not alias inputs.  Results are bitwise deterministic
 *     run to run (no atomics in any reduction).
 *   - Scratch memory is a caller-provided `workspace` of at least the
 *     size returned by the matching *_workspace_size() call.
 *   - Weights use the pages' column-vector convention (W_down is d x f and
 *     maps an f-vector z to W_down z); as row-major arrays that is the
 *     [out_features, in_features] layout.
 */
#ifndef TTCD_H
#define TTCD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TTCD_OK = 0,
  TTCD_ERR_NULL_POINTER = 1,       /* a required pointer is NULL          */
  TTCD_ERR_BAD_SHAPE = 2,          /* sizes inconsistent or out of range  */
  TTCD_ERR_UNSUPPORTED = 3,        /* valid but not implemented (dtype, head_dim) */
  TTCD_ERR_WORKSPACE_TOO_SMALL = 4,
  TTCD_ERR_ALIGNMENT = 5,          /* a pointer is not 16-byte aligned    */
  TTCD_ERR_HIP = 6                 /* a HIP launch or runtime call failed */
} ttcd_status;

typedef enum { TTCD_F32 = 0, TTCD_BF16 = 1 } ttcd_dtype;

/* Which path's MLP output receives the fast weight and forms the layer
 * output.  The pages do not say; the teacher (the model's own long-window
 * attention) is the default. */
typedef enum { TTCD_MAIN_TEACHER = 0, TTCD_MAIN_STUDENT = 1 } ttcd_main_path;

/* ------------------------------------------------------------------------
 * Dual-window causal sliding-window attention.
 *
 * Defined by the paper's two views of one backbone (papernotes.org notes,
 * "overall framework"; podcast transcript, sliding-window cue): a query at
 * position t attends to the keys j with 0 <= t - j < w, for the teacher
 * window w_T and the student window w_S <= w_T, over the SAME q/k/v.  Both
 * outputs come out of one pass over K/V (README "Fused inference
 * kernels").  Softmax scale `scale` (<= 0 means 1/sqrt(head_dim)).
 *
 *   q        [batch, seq_q, n_q_heads, head_dim]          in_dtype
 *   k, v     [batch, kv_rows, n_kv_heads, head_dim]        in_dtype
 *            key row j sits at absolute position j; query row i sits at
 *            position q_pos0 + i.  kv_rows (0 = seq_k) is the per-sequence
 *            row capacity of k/v (a decode cache may be larger than seq_k).
 *   o_teacher, o_student [batch, seq_q, n_q_heads, head_dim] out_dtype
 *   lse_teacher, lse_student [batch, n_q_heads, seq_q] fp32, natural-log
 *            log-sum-exp of each row's scaled scores; either may be NULL.
 * Query head h reads kv head h / (n_q_heads / n_kv_heads) (GQA).
 * Requires batch, seq_q, seq_k >= 1 (an empty call is TTCD_ERR_BAD_SHAPE),
 * q_pos0 + seq_q <= seq_k <= kv_rows, 1 <= w_student <= w_teacher,
 * head_dim in {64, 128}, batch * max(seq_q, kv_rows) * n_q_heads < 2^31 and
 * batch * kv_rows * n_kv_heads * head_dim <= 2^40.  Keys older than the teacher window of every query
 * are never read, so they may hold anything (NaN included).
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t batch;
  int32_t seq_q;
  int32_t seq_k;
  int32_t kv_rows;      /* 0 -> seq_k */
  int32_t q_pos0;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t w_teacher;
  int32_t w_student;
  float scale;          /* <= 0 -> 1/sqrt(head_dim) */
  ttcd_dtype in_dtype;
  ttcd_dtype out_dtype;
} ttcd_attn_desc;

size_t ttcd_dual_window_attn_workspace_size(const ttcd_attn_desc* desc);

ttcd_status ttcd_dual_window_attn(const ttcd_attn_desc* desc,
                                  const void* q, const void* k, const void* v,
                                  void* o_teacher, void* o_student,
                                  float* lse_teacher, float* lse_student,
                                  void* workspace, size_t workspace_bytes,
                                  void* stream);

/* ------------------------------------------------------------------------
 * The same attention through the LSE-combination path (README "Fused
 * inference kernels", the LSE-combination variant): a student-window call,
 * a call over the far band w_S <= t - j < w_T (the queries shifted back by
 * w_S against a window of w_T - w_S), and the exact merge of the two
 * normalised outputs through their log-sum-exps:
 *   LSE_T = log(e^LSE_S + e^LSE_far),
 *   O_T   = e^(LSE_S - LSE_T) O_S + e^(LSE_far - LSE_T) O_far.
 * Arguments, layouts, requirements and errors are those of
 * ttcd_dual_window_attn; o_teacher and o_student must not alias.  The
 * workspace (size from ttcd_dual_window_attn_lse_split_workspace_size, never
 * zero) holds V^T for bf16 inputs, O_far in fp32 and two LSE rows.  The
 * outputs equal the fused kernel's up to rounding (O_T here is formed from
 * O_S as stored in out_dtype).
 * ---------------------------------------------------------------------- */
size_t ttcd_dual_window_attn_lse_split_workspace_size(const ttcd_attn_desc* desc);

ttcd_status ttcd_dual_window_attn_lse_split(const ttcd_attn_desc* desc,
                                            const void* q, const void* k, const void* v,
                                            void* o_teacher, void* o_student,
                                            float* lse_teacher, float* lse_student,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream);

/* ------------------------------------------------------------------------
 * Backward of the dual-window attention (training; the papernotes.org notes
 * price it in their limitations section).  Both windows read the same q, k
 * and v, so their gradients add: with P_w = exp(s - LSE_w) on the keys of
 * window w, D_w = rowsum(dO_w * O_w) and dS = sum_w P_w (dO_w v^T - D_w),
 *   dq = scale dS k,   dk = scale dS^T q,   dv = sum_w P_w^T dO_w
 * (a kv head's gradients sum over its q heads).
 *
 * Prefill only: seq_q == seq_k == kv_rows (or kv_rows 0), q_pos0 == 0.
 *   q, k, v, o_teacher, o_student, do_teacher, do_student: layouts of
 *            ttcd_dual_window_attn, all in in_dtype (o_* are that call's
 *            outputs, produced with out_dtype == in_dtype)
 *   lse_teacher, lse_student [batch, n_q_heads, seq_q] fp32 (required)
 *   dq [batch, seq, n_q_heads, head_dim], dk, dv [batch, seq, n_kv_heads,
 *            head_dim]: out_dtype, written in full.
 * Deterministic: no atomics; the key and query sides each recompute the
 * scores.  The workspace (size from
 * ttcd_dual_window_attn_backward_workspace_size) holds the per-row LSE and
 * D values and, for bf16, transposed copies of q, dO_T, dO_S and k.
 * Outputs must not alias inputs.
 * ---------------------------------------------------------------------- */
size_t ttcd_dual_window_attn_backward_workspace_size(const ttcd_attn_desc* desc);

ttcd_status ttcd_dual_window_attn_backward(const ttcd_attn_desc* desc,
                                           const void* q, const void* k, const void* v,
                                           const void* o_teacher, const void* o_student,
                                           const float* lse_teacher, const float* lse_student,
                                           const void* do_teacher, const void* do_student,
                                           void* dq, void* dk, void* dv,
                                           void* workspace, size_t workspace_bytes,
                                           void* stream);

/* ------------------------------------------------------------------------
 * Chunk-wise fast-weight update of W_down (IP-TTCD, off-policy).
 *
 * From the papernotes.org notes, key design 3 (the practical update, the
 * paper's Eq. 12 in the podcast transcript) and key design 2 (off-policy
 * activations at W_down^(0), causal prefix over chunks):
 *   Zbar_T = conv_T(Z_T), Zbar_S = conv_S(Z_S)   depthwise causal conv over
 *            the whole sequence, zero left padding, tap kc-1 multiplies the
 *            current token, no bias;
 *   r_t    = W_down0 W_proj (Zbar_T[t] - Zbar_S[t])                 [d]
 *   k_t    = Zbar_S[t] / max(||Zbar_S[t]||_2, l2_eps)               [f]
 *   dW_i   = beta[i] * sum_{t in chunk i} r_t k_t^T                 [d x f]
 *   S_0    = W_down0,  S_{i+1} = S_i + dW_i
 *   y_t    = S_{floor(t/chunk)} z_main[t]       (writes act on later chunks)
 *
 *   z_teacher, z_student, z_main  [batch, seq, d_ff]  in_dtype
 *            (z_main may alias z_teacher or z_student)
 *   conv_t, conv_s  [d_ff, conv_k]  in_dtype
 *   w_down0 [d_model, d_ff], w_proj [d_ff, d_ff]     in_dtype
 *   beta    [batch, ceil(seq/chunk)] fp32 (the exact coefficient of R_i K_i^T)
 *   y       [batch, seq, d_model]  out_dtype
 *   state_out [batch, d_model, d_ff] fp32 or NULL: S_n, the weight after
 *            the writes of the n = floor(seq/chunk) chunks that hold all
 *            `chunk` tokens.  A short last chunk is still pending: its
 *            writes take effect once it completes, so a decode step that
 *            continues the sequence starts from S_n and appends the pending
 *            chunk's tokens to its lists (ttcd_fastweight_decode_append).
 *   r_out   [batch, seq, d_model] in_dtype or NULL: r_t, the residual terms
 *   k_out   [batch, seq, d_ff]    in_dtype or NULL: k_t, the unit keys
 *            (without beta): the low-rank chunk lists of ttcd_fw_state, rows
 *            [j*chunk, (j+1)*chunk) holding chunk j, so that a decode loop
 *            continues from this prefill in list form.
 * Requires batch, seq >= 1 (an empty call is TTCD_ERR_BAD_SHAPE),
 * batch * seq <= 2^28, chunk % 16 == 0, d_model % 8 == 0, d_ff % 8 == 0,
 * conv_k in [1,8].
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t batch;
  int32_t seq;
  int32_t d_model;
  int32_t d_ff;
  int32_t chunk;
  int32_t conv_k;
  float l2_eps;          /* <= 0 -> 1e-12 */
  ttcd_dtype in_dtype;
  ttcd_dtype out_dtype;
} ttcd_fw_desc;

size_t ttcd_fastweight_scan_workspace_size(const ttcd_fw_desc* desc);

ttcd_status ttcd_fastweight_scan(const ttcd_fw_desc* desc,
                                 const void* z_teacher, const void* z_student,
                                 const void* z_main,
                                 const void* conv_t, const void* conv_s,
                                 const void* w_down0, const void* w_proj,
                                 const float* beta,
                                 void* y, float* state_out,
                                 void* r_out, void* k_out,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);

/* The same chunk-wise update with the on-policy recurrence, a variant of
 * the update rule (papernotes.org notes, key design 2, and the podcast
 * transcript's Eq. 12 state the practical rule with the residual taken at
 * W_down^(0); here it is taken at the fast weight in force for the chunk):
 *   r_t  = S_{floor(t/chunk)} W_proj (Zbar_T[t] - Zbar_S[t])
 * with everything else as above (keys, beta, prefix, apply).  The chunks
 * are processed one after another.  Arguments, layouts and errors are those
 * of ttcd_fastweight_scan (state_out is S_n after the complete chunks; this
 * call has no list outputs); state_out, when given, also serves as the fp32
 * running state.  Its workspace adds d_model * d_ff fp32 values. */
size_t ttcd_fastweight_scan_on_policy_workspace_size(const ttcd_fw_desc* desc);

ttcd_status ttcd_fastweight_scan_on_policy(const ttcd_fw_desc* desc,
                                           const void* z_teacher, const void* z_student,
                                           const void* z_main,
                                           const void* conv_t, const void* conv_s,
                                           const void* w_down0, const void* w_proj,
                                           const float* beta,
                                           void* y, float* state_out,
                                           void* workspace, size_t workspace_bytes,
                                           void* stream);

/* The unprojected write of the distillation gradient, a variant of the
 * update rule (the podcast transcript's Eq. 4 and Eq. 6 cues: half the
 * squared gap between the student's and the detached teacher's MLP outputs;
 * its negative gradient in W_down is the output gap times the student's
 * activation).  Evaluated off-policy at W_down^(0), with no short convs, no
 * W_proj and no key normalisation:
 *   r_t     = W_down^(0) (Z_T[t] - Z_S[t])                            [d]
 *   S_{i+1} = S_i + beta[b,i] * sum_{t in chunk i} r_t Z_S[t]^T,  S_0 = W_down^(0)
 *   y[t]    = S_{floor(t/chunk)} z_main[t]
 * beta carries the step size (and any 1/|chunk| of the loss).  desc's
 * conv_k and l2_eps are ignored; everything else (layouts, state_out after
 * the complete chunks, workspace, errors) is as for ttcd_fastweight_scan,
 * which alone has the list outputs. */
size_t ttcd_fastweight_scan_eq6_workspace_size(const ttcd_fw_desc* desc);

ttcd_status ttcd_fastweight_scan_eq6(const ttcd_fw_desc* desc,
                                     const void* z_teacher, const void* z_student,
                                     const void* z_main, const void* w_down0,
                                     const float* beta,
                                     void* y, float* state_out,
                                     void* workspace, size_t workspace_bytes,
                                     void* stream);

/* ------------------------------------------------------------------------
 * Backward pass of ttcd_fastweight_scan (the training cost of the method is
 * 1.1-1.2x a standard layer on the papernotes.org notes, 局限与展望; the
 * gradient itself is the chain rule of the update above).  Given dy, the
 * gradient of a loss with respect to y, it returns the gradients of that
 * loss with respect to every input of the scan:
 *   dS_i       = sum_{t in chunk i} dy_t z_main[t]^T
 *   dz_main[t] = S_{floor(t/chunk)}^T dy_t
 *   G_j        = sum_{i > j} dS_i          (chunk j's write reaches later chunks)
 *   dbeta[j]   = sum_{t in chunk j} r_t . (G_j k_t)
 *   dr_t = beta_j G_j k_t,  dk_t = beta_j G_j^T r_t
 *   dW_down0   = sum_i dS_i + sum_t dr_t (W_proj dbar_t)^T
 *   dW_proj    = sum_t (W_down0^T dr_t) dbar_t^T
 * then the l2 backward of the keys and the backward of both short convs.
 *
 *   inputs as for ttcd_fastweight_scan (desc->out_dtype is the type of the
 *            activation gradients); dy [batch, seq, d_model] in_dtype
 *   dz_teacher, dz_student, dz_main [batch, seq, d_ff] out_dtype: the
 *            gradients through the conv paths and through the apply (when
 *            z_main aliases an input, its gradient is the sum of the two)
 *   dconv_t, dconv_s [d_ff, conv_k], dw_down0 [d_model, d_ff],
 *   dw_proj [d_ff, d_ff] fp32: summed over the batch, overwritten
 *   dbeta [batch, ceil(seq/chunk)] fp32 (the last chunk's entry is 0: its
 *            write reaches no token)
 * Requirements and errors as for ttcd_fastweight_scan; every output is
 * required.
 * ---------------------------------------------------------------------- */
size_t ttcd_fastweight_scan_backward_workspace_size(const ttcd_fw_desc* desc);

ttcd_status ttcd_fastweight_scan_backward(const ttcd_fw_desc* desc,
                                          const void* z_teacher, const void* z_student,
                                          const void* z_main,
                                          const void* conv_t, const void* conv_s,
                                          const void* w_down0, const void* w_proj,
                                          const float* beta, const void* dy,
                                          void* dz_teacher, void* dz_student, void* dz_main,
                                          float* dconv_t, float* dconv_s,
                                          float* dw_down0, float* dw_proj, float* dbeta,
                                          void* workspace, size_t workspace_bytes,
                                          void* stream);

/* ------------------------------------------------------------------------
 * The fast-weight stream alone: the first, memory-bound step of
 * ttcd_fastweight_scan (papernotes.org notes, key design 3: the short
 * causal convs of both paths, their difference and the per-token l2 norm of
 * the student activations).  Same conv and norm conventions as above.
 *
 *   desc: batch, seq, d_ff, chunk, conv_k, l2_eps, in_dtype (d_model and
 *         out_dtype are ignored)
 *   z_teacher, z_student [batch, seq, d_ff], conv_t, conv_s [d_ff, conv_k],
 *         beta [batch, ceil(seq/chunk)] fp32
 * Outputs, with seq_pad = 64 * ceil(seq / 64):
 *   dbar      [batch, seq_pad, d_ff] in_dtype: Zbar_T - Zbar_S, token-major
 *   zbar_s_t  [batch, d_ff, seq_pad] in_dtype: Zbar_S, feature-major
 *   key_scale [batch, seq_pad] fp32: beta[t/chunk] / max(||Zbar_S[t]||, eps),
 *             so the scaled key beta_i k_t is key_scale[t] * Zbar_S[t]
 * Rows t >= seq of every output are zero.
 * ---------------------------------------------------------------------- */
size_t ttcd_fastweight_stream_workspace_size(const ttcd_fw_desc* desc);

ttcd_status ttcd_fastweight_stream(const ttcd_fw_desc* desc,
                                   const void* z_teacher, const void* z_student,
                                   const void* conv_t, const void* conv_s,
                                   const float* beta,
                                   void* dbar, void* zbar_s_t, float* key_scale,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

/* ------------------------------------------------------------------------
 * Whole IP-TTCD layer forward from Q/K/V onward.
 *
 * Per path p in {teacher, student} (the glue around attention and the MLP
 * is a standard pre-norm decoder block; the pages do not describe it):
 *   h_p = x + concat_heads(O_p) W_o^T
 *   Z_p = silu(RMSNorm(h_p) W_gate^T) * (RMSNorm(h_p) W_up^T)
 * then the fast-weight update above with z_main = Z_main and
 *   out = h_main + y.
 *
 *   w_o [d_model, n_q_heads*head_dim], rms_gamma [d_model] (NULL = ones),
 *   w_gate, w_up [d_ff, d_model], w_down0 [d_model, d_ff],
 *   w_proj [d_ff, d_ff], conv_t, conv_s [d_ff, conv_k]: attn.in_dtype;
 *   beta [batch, ceil(seq/chunk)] fp32.
 *   x   [batch, seq_q, d_model]  attn.in_dtype (residual stream)
 *   out [batch, seq_q, d_model]  fp32
 *
 * Requirements of ttcd_dual_window_attn and of the fast-weight scan, and
 * attn.batch * attn.seq_q <= 2^28.
 * Prefill: dec == NULL, attn.seq_q == attn.seq_k, attn.q_pos0 == 0.
 * Decode:  dec != NULL, attn.seq_q == 1, attn.q_pos0 = L, attn.seq_k = L+1
 *          (the new token's k/v already written at row L of the cache).
 *          The fast weight is W_down0 + sum_j beta_list[j] R_j^T K_j over
 *          the dec->n_chunks completed chunks (low-rank lists), or
 *          dec->state_dense when it is not NULL.
 * ---------------------------------------------------------------------- */
typedef struct {
  const void* w_o;
  const void* rms_gamma;
  const void* w_gate;
  const void* w_up;
  const void* w_down0;
  const void* w_proj;
  const void* conv_t;
  const void* conv_s;
  const float* beta;
} ttcd_layer_weights;

typedef struct {
  ttcd_attn_desc attn;
  int32_t d_model;
  int32_t d_ff;
  int32_t chunk;
  int32_t conv_k;
  float rms_eps;          /* <= 0 -> 1e-6 */
  float l2_eps;           /* <= 0 -> 1e-12 */
  ttcd_main_path main_path;
} ttcd_layer_desc;

typedef struct {
  const float* state_dense;  /* [batch, d_model, d_ff] fp32, or NULL        */
  const void* r_list;        /* [batch, n_chunks*chunk, d_model] in_dtype   */
  const void* k_list;        /* [batch, n_chunks*chunk, d_ff] in_dtype (unit keys) */
  const float* beta_list;    /* [batch, n_chunks]                           */
  int32_t n_chunks;
} ttcd_fw_state;

/* Optional intermediate outputs (any member may be NULL). */
typedef struct {
  void* o_teacher;      /* [batch, seq_q, n_q_heads, head_dim] attn.in_dtype */
  void* o_student;
  float* lse_teacher;   /* [batch, n_q_heads, seq_q] */
  float* lse_student;
  void* z_teacher;      /* [batch, seq_q, d_ff] attn.in_dtype */
  void* z_student;      /* in a decode step the non-main path runs only when
                           its Z is asked for here (the append below needs
                           both) */
  float* y;             /* [batch, seq_q, d_model] fast-weight MLP output */
  float* state_out;     /* prefill only: [batch, d_model, d_ff], the weight
                           after the complete chunks (as in
                           ttcd_fastweight_scan) */
  void* r;              /* prefill only: [batch, seq_q, d_model] attn.in_dtype,
                           the residual terms r_t of the chunk lists */
  void* k;              /* prefill only: [batch, seq_q, d_ff] attn.in_dtype,
                           the unit keys k_t of the chunk lists */
} ttcd_layer_aux;

size_t ttcd_layer_forward_workspace_size(const ttcd_layer_desc* desc,
                                         const ttcd_fw_state* dec);

ttcd_status ttcd_layer_forward(const ttcd_layer_desc* desc,
                               const ttcd_layer_weights* weights,
                               const void* q, const void* k, const void* v,
                               const void* x, float* out,
                               const ttcd_fw_state* dec,
                               const ttcd_layer_aux* aux,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/* ------------------------------------------------------------------------
 * The layer forward without allocation, for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops (one decode step per token), harnesses that forbid
 * hipMalloc.  Same arguments, semantics and errors as ttcd_layer_forward,
 * except that the scratch is a device array of TTCD_NOALLOC_SCRATCH_MIB MiB
 * inside the library (one per GPU, held until the process ends) rather than
 * a workspace argument.  The call allocates nothing (no hipMalloc, no host
 * allocation); its first call on a device looks the array's address up
 * once (hipGetSymbolAddress), so make that first call outside graph capture.
 *
 * A call whose ttcd_layer_forward_workspace_size() exceeds
 * ttcd_layer_forward_noalloc_max_bytes() is rejected with
 * TTCD_ERR_WORKSPACE_TOO_SMALL before anything is enqueued: decode steps
 * (batch 32, a 64K cache, 64 chunk lists: about 52 MB) and short prefills
 * fit; a 64K prefill does not.
 *
 * Every call on one GPU shares that GPU's array and leaves its last
 * contents there (no call relies on them).  Calls that overlap in time on
 * one GPU -- on different streams, or from different threads -- race on the
 * array: serialise them.
 * ---------------------------------------------------------------------- */
#define TTCD_NOALLOC_SCRATCH_MIB 64

size_t ttcd_layer_forward_noalloc_max_bytes(void);

ttcd_status ttcd_layer_forward_noalloc(const ttcd_layer_desc* desc,
                                       const ttcd_layer_weights* weights,
                                       const void* q, const void* k, const void* v,
                                       const void* x, float* out,
                                       const ttcd_fw_state* dec,
                                       const ttcd_layer_aux* aux,
                                       void* stream);

/* ------------------------------------------------------------------------
 * Decode-time fast-weight stream: the per-token part of the chunk writes
 * (papernotes.org notes, key design 3; the paper's Eq. 12 in the podcast
 * transcript) for a generated token, so that a decode loop can grow the
 * chunk lists (or fold them with ttcd_fastweight_fold) exactly as a prefill
 * over the same tokens would.
 *
 * ttcd_fastweight_residual_proj:  M = W_down0 W_proj  [d_model, d_ff]
 *   in_dtype, the matrix that maps the conv difference to the residual
 *   r_t; computed once per weight set.  Workspace: d_ff * d_ff elements.
 *
 * ttcd_fastweight_decode_append: for each sequence b of the batch, with
 *   z_teacher, z_student [batch, d_ff] the new token's SwiGLU outputs of
 *   both paths (ttcd_layer_forward in decode returns them through
 *   ttcd_layer_aux) and hist_t, hist_s [batch, conv_k-1, d_ff] the last
 *   conv_k-1 rows of each path before it (oldest first; the caller seeds
 *   them with zeros at the sequence start or with the prefill's last rows):
 *     zbar_p = sum_r conv_p[:, r] * window_p[r]    (row conv_k-1 = the token)
 *     dbar   = zbar_T - zbar_S                     (rounded to in_dtype)
 *     r      = M dbar          -> r_out + b * r_stride   [d_model] in_dtype
 *     k      = zbar_S / max(||zbar_S||_2, l2_eps)
 *                              -> k_out + b * k_stride   [d_ff]    in_dtype
 *   and the histories advance by one row in place.  The strides (elements,
 *   multiples of 8) let r and k land in row j of chunk-list buffers.  The
 *   desc supplies batch, d_model, d_ff, conv_k, l2_eps and in_dtype.
 * ---------------------------------------------------------------------- */
size_t ttcd_fastweight_residual_proj_workspace_size(const ttcd_fw_desc* desc);

ttcd_status ttcd_fastweight_residual_proj(const ttcd_fw_desc* desc,
                                          const void* w_down0, const void* w_proj,
                                          void* m_out, void* workspace,
                                          size_t workspace_bytes, void* stream);

size_t ttcd_fastweight_decode_append_workspace_size(const ttcd_fw_desc* desc);

ttcd_status ttcd_fastweight_decode_append(const ttcd_fw_desc* desc,
                                          const void* z_teacher, const void* z_student,
                                          void* hist_t, void* hist_s,
                                          const void* conv_t, const void* conv_s,
                                          const void* m,
                                          void* r_out, int64_t r_stride,
                                          void* k_out, int64_t k_stride,
                                          void* workspace, size_t workspace_bytes,
                                          void* stream);

/* ------------------------------------------------------------------------
 * Fold low-rank chunk lists into a dense fast weight (decode set-up):
 *   state_out[b] = W_down0 + sum_{j < n_chunks} beta_list[b,j] R_j^T K_j
 * with R_j = r_list[b, j*chunk:(j+1)*chunk], K_j likewise (the prefix sum of
 * the papernotes.org notes, key design 2, evaluated once).
 * desc->seq is ignored; desc->in_dtype is the list/weight type.
 * ---------------------------------------------------------------------- */
size_t ttcd_fastweight_fold_workspace_size(const ttcd_fw_desc* desc, int32_t n_chunks);

ttcd_status ttcd_fastweight_fold(const ttcd_fw_desc* desc, const void* w_down0,
                                 const void* r_list, const void* k_list,
                                 const float* beta_list, int32_t n_chunks,
                                 float* state_out,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Human-readable name of a status code (static storage). */
const char* ttcd_status_string(ttcd_status status);

/* Detail of the last failing call on this thread ("" if none). */
const char* ttcd_last_error(void);

/* Library version string, e.g. "0.1.0 gfx950". */
const char* ttcd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TTCD_H */
