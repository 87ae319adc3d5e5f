// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ttcd {

enum DType { F32 = 0, BF16 = 1 };

inline size_t dsize(int dt) { return dt == BF16 ? 2 : 4; }

// ---------------------------------------------------------------- attention
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* vt;           // workspace: V transposed [B][Hkv][D][vt_ld] (bf16 path)
  int vt_ld;
  void* o_t;
  void* o_s;
  float* lse_t;
  float* lse_s;
  int B, Tq, Tk, kv_rows, q_pos0, Hq, Hkv, D, wT, wS;
  float scale;
  int in_dt, out_dt;
};
// Returns hipSuccess or the launch error.
hipError_t launch_dual_window_attn(const AttnArgs& a, hipStream_t s);
// The same outputs through the LSE-combination path (student call, shifted
// far-band call, exact merge); o_far, lse_far, lse_tmp are fp32 workspace.
hipError_t launch_dual_window_attn_lse_split(const AttnArgs& a, float* o_far, float* lse_far,
                                             float* lse_tmp, hipStream_t s);
size_t attn_vt_bytes(int B, int Hkv, int D, int Tk, int in_dt);

// ---------------------------------------------------------------- decode attention
struct DecodeAttnArgs {
  const void* q;      // [B, 1, Hq, D]
  const void* k;      // [B, kv_rows, Hkv, D]
  const void* v;
  void* o_t;          // [B, 1, Hq, D] out_dt
  void* o_s;
  float* lse_t;       // [B, Hq]
  float* lse_s;
  float* part;        // workspace partials
  int B, pos, kv_rows, Hq, Hkv, D, wT, wS;
  float scale;
  int in_dt, out_dt;
  int nsplit, split_len;
};
void decode_attn_plan(int wT, int* nsplit, int* split_len);
size_t decode_attn_part_bytes(int B, int Hq, int D, int nsplit);
hipError_t launch_decode_attn(const DecodeAttnArgs& a, hipStream_t s);

// ---------------------------------------------------------------- GEMM (C = A B^T)
// A [M, K] (row stride lda), B [N, K] (row stride ldb), both K-contiguous.
enum Epi {
  EPI_STORE = 0,        // C = acc (* colscale[n] if given)
  EPI_RESIDUAL = 1,     // C(f32) = acc + res[(m % res_rows) * ldr + n]
  EPI_SWIGLU = 2,       // C = silu(A Bg^T) * (A Bu^T); B2 = Bu, N = f
                        //   (with rowscale: silu(s_m A Bg^T) * (s_m A Bu^T))
  EPI_SWIGLU_RS = 4,    // (kernel selection only: EPI_SWIGLU with rowscale)
  EPI_RESNORM = 3,      // EPI_RESIDUAL, and also U(bf16) = C * gamma[n] and the
                        //   sum over each 64-column group of C^2 into
                        //   rowss[(n / 64) * M + m]; the 256 x 256 tile only,
                        //   full tiles only, batch 1, bf16 operands
};
struct GemmArgs {
  const void* A; long lda;
  const void* B; long ldb;
  const void* B2;                 // second B (swiglu up) or NULL
  void* C; long ldc;
  int M, N, K;
  int in_dt;                      // A, B dtype
  int out_dt;                     // C dtype
  int epi;
  const float* colscale;          // EPI_STORE: per-column scale (or NULL)
  const void* res; long ldr; int res_rows; int res_dt;   // EPI_RESIDUAL
  // batching over blockIdx.z: pointer strides in elements
  int batch; long sA, sB, sC, sRes, sScale;
  // chunked B (fast-weight apply): rows [c*chunk, (c+1)*chunk) of each batch
  // use B = (c == 0 ? B : Bchunks + (c-1) * sBchunk); 0 disables
  int chunk; const void* Bchunks; long sBchunk; long sBchunksBatch;
  // optional fp32 workspace for the few-row (M <= 32) split-K path; NULL
  // disables it (gemm_skinny_ws_floats gives the size it needs)
  float* ws; size_t ws_floats;
  // EPI_RESNORM outputs (U [M, ldc] bf16; gamma [N] bf16 or NULL for ones;
  // rowss [N / 64, M] fp32) and the EPI_SWIGLU row scale (NULL: none)
  void* U; const void* gamma; float* rowss;
  const float* rowscale;
};
hipError_t launch_gemm(const GemmArgs& g, hipStream_t s);
size_t gemm_skinny_ws_floats(int M, int N, int K, int epi);
// Whether launch_gemm runs g on the 256 x 256 tile with every tile full, the
// condition for EPI_RESNORM and for a SwiGLU row scale.
bool gemm_wide_full(const GemmArgs& g);
// RMSNorm row scale from the EPI_RESNORM partials:
//   rs[m] = 1 / sqrt(sum_j rowss[j * M + m] / N + eps), j < N / 64.
hipError_t launch_rms_rowscale(const float* rowss, int M, int N, float eps, float* rs,
                               hipStream_t s);

// Fast-weight prefix states:
//   acc = W0 (fp32); for i in [0, nstates): acc += A_i B_i^T over tokens of
//   chunk i; states[i] = acc  (state i = weight after chunk i's write).
// A = Rs^T [d, T] (lda = T), B = Zb^T [f, T] (ldb = T).
// Causal prefix of the chunk writes (papernotes.org notes, key design 2):
//   S_{j+1} = W0 + sum_{i <= j} dW_i, kept in fp32 while walking j;
//   states[b, j] = S_{j+1} (st_dt) for j < nstates, final_out[b] = S_{nwrites}.
//   dw [B, dw_chunks, n] in st_dt (the first nwrites chunks of each batch element
//   are read), w0 [n] w0_dt, states [B, nstates, n], final_out [B, n], n = d * f.
hipError_t launch_state_prefix(const void* dw, long dw_chunks, const void* w0, void* states,
                               float* final_out, long n, int nstates, int nwrites, int batch,
                               int w0_dt, int st_dt, hipStream_t s);

// ---------------------------------------------------------------- elementwise / stream
// u = rmsnorm(h) * gamma, h fp32 [rows, d] -> u [rows, d] out_dt
hipError_t launch_rmsnorm(const float* h, const void* gamma, void* u, int rows, int d,
                          float eps, int in_dt, int out_dt, hipStream_t s);

// fast-weight stream: conv, difference, key norms.
//   dbar [B, T, f] = conv_t(zt) - conv_s(zs)   (in_dt)
//   zbt  [B, f, T] = conv_s(zs) transposed      (in_dt)
//   sc   [B, T]    = beta[b, t / chunk] / max(||conv_s(zs)[t]||, eps)
struct StreamArgs {
  const void* zt; const void* zs;
  const void* conv_t; const void* conv_s;
  const float* beta;
  void* dbar; void* zbt; float* sc;
  float* inv;                     // [B, Tpad] 1 / max(key norm, eps), or NULL
  float* part;                    // workspace: partial key norms (fw_stream_part_bytes)
  int B, T, f, kc, chunk, nchunks;
  float eps;
  int in_dt;
  int raw_keys;                   // 1: sc = beta (keys not normalised)
};
hipError_t launch_fw_stream(const StreamArgs& a, hipStream_t s);
// k_out [B, T, f] = zbt [B, f, Tpad]^T scaled per token by inv [B, Tpad]
hipError_t launch_unit_keys(const void* zbt, const float* inv, void* k_out, int B, int T, int f,
                            int dt, hipStream_t s);

// One generated token: convs over the history and the token, dbar, the unit
// key (to k_out + b * k_stride), and the history advanced by one row.
struct DecodeAppendArgs {
  const void* zt; const void* zs;       // [B, f]
  void* hist_t; void* hist_s;           // [B, kc-1, f], updated in place
  const void* conv_t; const void* conv_s;
  void* dbar;                           // [B, f] workspace
  void* k_out; long k_stride;
  int B, f, kc;
  float eps;
  int in_dt;
};
hipError_t launch_fw_decode_append(const DecodeAppendArgs& a, hipStream_t s);
// on-policy recurrence: s32 = float(w0); per chunk s32 += dw, s16 = s32 (dt)
hipError_t launch_state_init(const void* w0, float* s32, long n, int dt, hipStream_t s);
hipError_t launch_fill(void* p, long n, float v, int dt, hipStream_t s);
// a strided 2-D region: p[b * bstride + r * ld + c] = v, r < rows, c < width,
// b < nbatch (a no-op for an empty region)
hipError_t launch_fill2d(void* p, long rows, long width, long ld, int nbatch, long bstride,
                         float v, int dt, hipStream_t s);
hipError_t launch_splitk_reduce(const float* part, int nsplit, long zstride, int ldp,
                                const float* colscale, void* out, long ldo, int M, int N, int dt,
                                hipStream_t s);
hipError_t launch_state_step(const float* dw, int nsplit, float* s32, void* s16, long n, int dt,
                             hipStream_t s);
size_t fw_stream_part_bytes(int B, int T, int f);

// out [cols, rows] = in [rows, cols]^T (per batch), 2- or 4-byte elements
// out[z][c][r] = in[z][r][c] * (scale ? scale[z * s_scale + c / scale_div] : 1)
//                            * (rscale ? rscale[z * s_rscale + r / rscale_div] : 1)
// for r < in_rows, c < in_cols (dtypes in_dt -> out_dt), one rounding to the
// output type; output columns in_rows <= r < out_cols are written as zero
hipError_t launch_transpose64(const void* in, int in_dt, long ld_in, long s_in, int in_rows,
                              int in_cols, void* out, int out_dt, long ld_out, long s_out,
                              int out_cols, int batch, const float* scale, long s_scale,
                              int scale_div, hipStream_t s, const float* rscale = nullptr,
                              long s_rscale = 0, int rscale_div = 1);
hipError_t launch_transpose(const void* in, void* out, int rows, int cols, long ld_in,
                            long ld_out, int batch, long s_in, long s_out, int esize,
                            hipStream_t s);
// V [B, kv_rows, Hkv, D] (bf16) -> vt [B, Hkv, D, vt_ld]: keys in [jlo, Tk), the
// keys of each 16-group permuted for the attention kernel's MFMA operand reads

// ------------------------------------------------------- attention backward
struct AttnBwdArgs {
  const void *q, *k, *v;            // [B,T,Hq,D], [B,T,Hkv,D] x2, in_dt
  const void *o_t, *o_s;            // [B,T,Hq,D] in_dt (the forward's outputs)
  const float *lse_t, *lse_s;       // [B,Hq,T] natural log
  const void *do_t, *do_s;          // [B,T,Hq,D] in_dt
  void *dq, *dk, *dv;               // out_dt
  int B, T, Hq, Hkv, D, wT, wS;
  float scale;
  int in_dt, out_dt;
};
struct AttnBwdBufs {
  float* meta;                      // per query row: LSE_T, LSE_S (log2), D_T, D_S
  void *qT, *dotT, *dosT, *kT;      // transposed copies (bf16 MFMA path)
};
// 32-row blocks of the row data per (batch, kv group), one of them padding
int attn_bwd_meta_blocks(int T, int G);
long attn_bwd_key_ld(int T);
size_t attn_bwd_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int in_dt);
void attn_bwd_plan(const AttnBwdArgs& a, char* ws, AttnBwdBufs& w);
hipError_t launch_dual_window_attn_backward(const AttnBwdArgs& a, const AttnBwdBufs& w,
                                            hipStream_t s);

// ---------------------------------------------------------------- backward
// token-major [B, rows, F] (the first T rows of each sequence) ->
// feature-major [F, B * TC], zero for T <= t < TC
hipError_t launch_to_feature_major(const void* in, void* out, int B, int T, int rows, int TC,
                                   int F, int dt, hipStream_t s);
// feature-major [F, B * TC] -> token-major [B, T, F], each token scaled by
// scale[b * n + t / chunk] when scale is given
hipError_t launch_to_token_major(const void* in, int in_dt, void* out, int out_dt, int B, int T,
                                 int TC, int F, const float* scale, int chunk, int n,
                                 hipStream_t s);
// out [B, d, Tpad] = R^T [d, B * TC] (fp32) times s[b * Tpad + t], zero for
// t >= T (the forward's write-scaled residual, from the unscaled fp32 one)
hipError_t launch_scaled_rt(const float* rt, const float* sc, void* out, int out_dt, int d, int T,
                            int TC, int Tpad, int B, hipStream_t s);
// x [rows, B * TC] *= s[b * Tpad + t] (zero for t >= T)
hipError_t launch_scale_token_cols(void* x, const float* sc, int rows, int B, int T, int TC,
                                   int Tpad, int dt, hipStream_t s);
// G [B, nch, n] = exclusive suffix sums of ds (fp32) over the chunks, stored
// in dt as g and, for bf16, the remainder g_lo = G - g (NULL: not wanted);
// total [n] fp32 = sum over sequences and chunks of ds
hipError_t launch_chunk_suffix(const float* ds, void* g, void* g_lo, float* total, long n,
                               int nch, int B, int dt, hipStream_t s);
// out [n] = sum over z < S of parts [S, n] (n % 4 == 0)
hipError_t launch_sum_slices(const float* parts, float* out, long n, int S, hipStream_t s);
// out[i] = sum over the S slices parts[z][i] (n % 4 == 0), stored as out_dt
hipError_t launch_sum_slices_to(const float* parts, void* out, long n, int S, int out_dt,
                                hipStream_t s);
// x fp32 [n] -> hi = bf16(x), lo = bf16(x - hi)
hipError_t launch_split_bf16(const float* x, void* hi, void* lo, long n, hipStream_t s);
// dbeta [B, nch] = per-chunk <R^T, P^T>; P^T *= beta (in place); rt, pt fp32 [d, B * TC]
size_t dbeta_part_floats(int B, int nch, int d);
hipError_t launch_dbeta(const float* rt, const float* pt, const float* beta, float* part,
                        float* dbeta, void* drt, int drt_dt, int B, int d, int chunk, int T,
                        int TC, int nch, hipStream_t s);
// kd [B * T] = beta_{c(t)} (khat_t . dk_t)
hipError_t launch_key_dot(const void* khat, const float* dk, const float* beta, float* kd, int B,
                          int T, int f, int chunk, int nch, int dt, hipStream_t s);
struct StreamBwdArgs {
  const void* zt; const void* zs; const void* conv_t; const void* conv_s;   // in_dt
  const float* dk;       // [B*T, f] G_j^T r_t (beta not applied)
  const float* ddbar;    // [B*T, f]
  const float* kd;       // [B*T] beta (k . dK)
  const float* inv;      // [B, Tpad] 1 / max(|zbar_S|, eps)
  const float* beta;     // [B, nch]
  void* dzt; void* dzs;  // [B, T, f] out_dt
  float* dconv_t; float* dconv_s;   // [f, kc]
  float* part;           // stream_bwd_part_floats
  int B, T, f, kc, chunk, nch;
  float eps;
  int in_dt, out_dt;
};
size_t stream_bwd_part_floats(int B, int T, int f, int kc);
hipError_t launch_stream_bwd(const StreamBwdArgs& a, hipStream_t s);

// decode fast-weight apply from low-rank lists:
//   c[b, t]  = k_list[b, t] . z[b]          (t < n*chunk)
//   y[b]    += sum_j beta[b, j] sum_{t in j} c[b, t] r_list[b, t]
struct ListApplyArgs {
  const void* z;          // [B, f] in_dt
  const void* r_list;     // [B, n*C, d]
  const void* k_list;     // [B, n*C, f]
  const float* beta;      // [B, n]
  float* cbuf;            // workspace [B, n*C]
  float* y;               // [B, d] fp32, accumulated into
  int B, d, f, chunk, n;
  int in_dt;
};
hipError_t launch_list_apply(const ListApplyArgs& a, hipStream_t s);
// y[b] (+)= S[b] z[b], S fp32 [B, d, f]
hipError_t launch_dense_apply(const float* S, const void* z, float* y, int B, int d, int f,
                              int in_dt, int accumulate, hipStream_t s);
// out[i] = a[i] + b[i] (fp32)
hipError_t launch_add(const float* a, const float* b, float* out, long n, hipStream_t s);
// out[b][i] = float(in[i]) for every b < batch
hipError_t launch_widen_repeat(const void* in, float* out, long n, int batch, int in_dt,
                               hipStream_t s);
// convert fp32 -> dt
hipError_t launch_convert(const float* in, void* out, long n, int out_dt, hipStream_t s);

}  // namespace ttcd
