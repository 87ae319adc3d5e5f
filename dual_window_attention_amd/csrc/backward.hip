// Backward pass of the chunk-wise fast-weight update (off-policy rule) on
// gfx950: the layout, reduction and per-token kernels around the backward
// GEMMs.  With S_i the weight in force for chunk i, y_t = S_{c(t)} z_main[t],
// S_{i+1} = S_i + beta_i R_i^T K_i, r_t = M dbar_t (M = W_down0 W_proj),
// k_t = Zbar_S[t] / max(|Zbar_S[t]|, eps), the gradient given dy is
//   dS_i = dY_i^T Z_main,i,   G_j = sum_{i > j} dS_i (exclusive suffix),
//   dr_t = beta_j G_j k_t,    dk_t = beta_j G_j^T r_t,
//   dbeta_j = sum_{t in C_j} r_t . (G_j k_t),
// then the residual projection, the l2 and the conv backward per token (the
// chain rule of the papernotes.org notes' key design 3 update; the pages
// state the training cost of the method, not its gradient).
#include "common.hpp"
#include "kernels.hpp"

namespace ttcd {

namespace {

// out[f_i][b * TC + t] = in[b][t][f_i] for t < T, 0 for T <= t < TC:
// token-major [B, rows, F] (rows >= T per sequence) -> feature-major
// [F, B * TC], zero padded.
template <typename T>
__global__ void __launch_bounds__(256)
to_feature_major_kernel(const T* __restrict__ in, T* __restrict__ out, int Tn, int rows, int TC,
                        int F) {
  __shared__ float tile[32][33];
  const int b = blockIdx.z;
  const int t0 = blockIdx.x * 32, f0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    const int t = t0 + i, fi = f0 + tx;
    tile[i][tx] = (t < Tn && fi < F) ? ldf(in + ((size_t)b * rows + t) * F + fi) : 0.f;
  }
  __syncthreads();
  const size_t ld = (size_t)gridDim.z * TC;
  for (int i = ty; i < 32; i += 8) {
    const int fi = f0 + i, t = t0 + tx;
    if (fi < F && t < TC) stf(out + (size_t)fi * ld + (size_t)b * TC + t, tile[tx][i]);
  }
}

// out[b][t][f_i] = in[f_i][b * TC + t] * (scale ? scale[b * n + t / chunk] : 1)
// for t < T: feature-major -> token-major, optionally scaled per token.
template <typename TI, typename TO>
__global__ void __launch_bounds__(256)
to_token_major_kernel(const TI* __restrict__ in, TO* __restrict__ out, int Tn, int TC, int F,
                      const float* __restrict__ scale, int chunk, int n) {
  __shared__ float tile[32][33];
  const int b = blockIdx.z;
  const int t0 = blockIdx.x * 32, f0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const size_t ld = (size_t)gridDim.z * TC;
  for (int i = ty; i < 32; i += 8) {
    const int fi = f0 + i, t = t0 + tx;
    tile[i][tx] = (fi < F && t < Tn) ? ldf(in + (size_t)fi * ld + (size_t)b * TC + t) : 0.f;
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int t = t0 + i, fi = f0 + tx;
    if (t < Tn && fi < F) {
      float v = tile[tx][i];
      if (scale) v *= scale[(size_t)b * n + t / chunk];
      stf(out + ((size_t)b * Tn + t) * F + fi, v);
    }
  }
}

// x[a][b * TC + t] *= s[b * Tpad + t] for t < T (0 beyond): the write scale
// beta / |Zbar_S| folded into the residual columns.
template <typename T>
__global__ void __launch_bounds__(256)
scale_token_cols_kernel(T* __restrict__ x, const float* __restrict__ s, int rows, int Tn, int TC,
                        int Tpad, int B) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const long ld = (long)B * TC;
  if (i >= (long)rows * ld) return;
  const long col = i % ld;
  const int b = (int)(col / TC), t = (int)(col % TC);
  const float v = t < Tn ? ldf(x + i) * s[(size_t)b * Tpad + t] : 0.f;
  stf(x + i, v);
}

// Exclusive suffix sums of the chunk gradients, per sequence:
//   G_j = sum_{i > j} dS_i  (element type),  total += sum_i dS_i  (fp32,
// summed over the batch).  Each thread owns 4 consecutive entries and walks
// the chunks from the last, the running sum in fp32.  dS arrives in fp32;
// G is stored as g (the operand dtype) and, for bf16, also as the remainder
// g_lo = bf16(G - g), so that a product with g + g_lo carries G to about
// fp32 accuracy.
template <typename T>
__global__ void __launch_bounds__(256)
chunk_suffix_kernel(const float* __restrict__ ds, T* __restrict__ g, T* __restrict__ g_lo,
                    float* __restrict__ total, long n, int nch, int B) {
  const long e = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= n) return;
  float tot[4] = {0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < B; ++b) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = nch - 1; j >= 0; --j) {
      const size_t off = ((size_t)b * nch + j) * n + e;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        T hv;
        stf(&hv, acc[i]);
        g[off + i] = hv;
        if (g_lo) stf(g_lo + off + i, acc[i] - ldf(&hv));
      }
      const f32x4 v = *reinterpret_cast<const f32x4*>(ds + off);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += v[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) tot[i] += acc[i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) total[e + i] = tot[i];
}

// x -> hi = bf16(x), lo = bf16(x - hi)
__global__ void __launch_bounds__(256)
split_bf16_kernel(const float* __restrict__ x, bf16_t* __restrict__ hi, bf16_t* __restrict__ lo,
                  long n) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float v = x[i];
  const bf16_t h = f2bf(v);
  hi[i] = h;
  lo[i] = f2bf(v - bf2f(h));
}

// dbeta partials and the scaled residual gradient: for sequence b, chunk j
// and a group of 16 rows a of P^T [d, B * TC] (P_j = G_j K_j^T, unscaled):
//   part[b][j][group] = sum_{a in group} sum_{t in C_j} R^T[a][t] P^T[a][t]
//   dR^T[a][t] = beta_j P^T[a][t]   (in place)
__global__ void __launch_bounds__(256)
dbeta_part_kernel(const float* __restrict__ rt, float* __restrict__ pt,
                  const float* __restrict__ beta, float* __restrict__ part, int d, int chunk,
                  int Tn, int TC, int nch) {
  const int grp = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const size_t ld = (size_t)gridDim.z * TC;
  const float bj = beta[(size_t)b * nch + j];
  float s = 0.f;
  for (int rr = 0; rr < 16; ++rr) {
    const int a = grp * 16 + rr;
    if (a >= d) break;
    for (int c = threadIdx.x; c < chunk; c += 256) {
      const int t = j * chunk + c;
      if (t >= Tn) break;
      const size_t i = (size_t)a * ld + (size_t)b * TC + t;
      const float p = pt[i];
      s = __builtin_fmaf(rt[i], p, s);
      pt[i] = bj * p;
    }
  }
  __shared__ float red[4];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0)
    part[((size_t)b * nch + j) * gridDim.x + grp] = (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ void __launch_bounds__(64)
dbeta_sum_kernel(const float* __restrict__ part, float* __restrict__ dbeta, int ngrp, int total) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= total) return;
  float s = 0.f;
  for (int g = 0; g < ngrp; ++g) s += part[(size_t)i * ngrp + g];
  dbeta[i] = s;
}

// kd[b * T + t] = beta_{t / chunk} * (k_t . dK_t): the projection term of the
// l2 backward (dK holds G_j^T r_t unscaled).  One wave per token.
template <typename T>
__global__ void __launch_bounds__(256)
key_dot_kernel(const T* __restrict__ khat, const float* __restrict__ dk,
               const float* __restrict__ beta, float* __restrict__ kd, int Tn, int f, int chunk,
               int nch, long rows) {
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const T* kr = khat + row * f;
  const float* dr = dk + row * f;
  float s = 0.f;
  for (int c = lane; c < f; c += 64) s = __builtin_fmaf(ldf(kr + c), dr[c], s);
  s = wave_sum(s);
  const int b = (int)(row / Tn), t = (int)(row % Tn);
  if (lane == 0) kd[row] = beta[(size_t)b * nch + t / chunk] * s;
}

// The per-token end of the backward, one 64-token x 64-feature tile per
// workgroup, one feature and 16 tokens per thread:
//   zbar_S[tau] = conv_S(z_s) (recomputed), k = zbar_S * inv,
//   dzbar_S = (beta dK - k kd) inv - ddbar   (|zbar_S| > eps)
//           = beta dK inv - ddbar             (otherwise; inv = 1/eps)
//   dzbar_T = ddbar
//   dz_p[t] = sum_i taps_p[i] dzbar_p[t + kc-1-i],  dtaps_p[i] += dzbar_p[t] z_p[t-(kc-1)+i]
// kd already holds beta (k . dK).  The tile's dtaps partial sums go to
// part[b][tile][2][f][kc] (teacher, student).
constexpr int SB_TOK = 16, SB_GRP = 4, SB_TT = SB_TOK * SB_GRP, SB_FF = 64;

template <typename T, typename OutT, int KC>
__global__ void __launch_bounds__(256)
stream_bwd_kernel(const T* __restrict__ zt, const T* __restrict__ zs,
                  const T* __restrict__ conv_t, const T* __restrict__ conv_s,
                  const float* __restrict__ dk, const float* __restrict__ ddbar,
                  const float* __restrict__ kd, const float* __restrict__ inv,
                  const float* __restrict__ beta, OutT* __restrict__ dzt, OutT* __restrict__ dzs,
                  float* __restrict__ part, int Tn, int Tpad, int f, int chunk, int nch,
                  float inv_eps) {
  constexpr int H = KC - 1;
  const int b = blockIdx.z;
  const int tile = blockIdx.x;
  const int fl = threadIdx.x % SB_FF, grp = threadIdx.x / SB_FF;
  const int c = blockIdx.y * SB_FF + fl;
  const bool fok = c < f;
  const int t0 = tile * SB_TT + grp * SB_TOK;          // this thread's first token
  const size_t rowb = (size_t)b * Tn;
  float wt[KC], ws[KC];
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    wt[i] = fok ? ldf(conv_t + (size_t)c * KC + i) : 0.f;
    ws[i] = fok ? ldf(conv_s + (size_t)c * KC + i) : 0.f;
  }
  // inputs of rows t0 - H .. t0 + SB_TOK + H - 1 (zero outside [0, T))
  constexpr int NR = SB_TOK + 2 * H;
  float xt[NR], xs[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int tau = t0 - H + r;
    const bool in = fok && tau >= 0 && tau < Tn;
    xt[r] = in ? ldf(zt + (rowb + tau) * f + c) : 0.f;
    xs[r] = in ? ldf(zs + (rowb + tau) * f + c) : 0.f;
  }
  // dzbar of rows t0 .. t0 + SB_TOK + H - 1 (rows >= T are zero)
  constexpr int ND = SB_TOK + H;
  float gt[ND], gs[ND];
#pragma unroll
  for (int r = 0; r < ND; ++r) {
    const int tau = t0 + r;
    float a = 0.f, s_ = 0.f;
    if (fok && tau < Tn) {
      float zb = 0.f;
#pragma unroll
      for (int i = 0; i < KC; ++i) zb = __builtin_fmaf(ws[i], xs[r + i], zb);
      const size_t ti = rowb + tau;
      const float iv = inv[(size_t)b * Tpad + tau];
      const float bj = beta[(size_t)b * nch + tau / chunk];
      const float g = dk[ti * f + c];
      const float dd = ddbar[ti * f + c];
      const float kv = zb * iv;
      float dz;
      if (iv < inv_eps)
        dz = (bj * g - kv * kd[ti]) * iv;       // (dk - k (k . dk)) / |zbar|, dk = beta dK
      else
        dz = bj * g * iv;                        // dk / eps
      s_ = dz - dd;
      a = dd;
    }
    gt[r] = a;
    gs[r] = s_;
  }
  float dtap_t[KC], dtap_s[KC];
#pragma unroll
  for (int i = 0; i < KC; ++i) dtap_t[i] = dtap_s[i] = 0.f;
#pragma unroll
  for (int r = 0; r < SB_TOK; ++r) {
    const int t = t0 + r;
    float at = 0.f, as = 0.f;
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      // zbar[t + H - i] takes z[t] through tap i
      at = __builtin_fmaf(wt[i], gt[r + H - i], at);
      as = __builtin_fmaf(ws[i], gs[r + H - i], as);
      // dtaps[i] += dzbar[t] z[t - H + i]
      dtap_t[i] = __builtin_fmaf(gt[r], xt[r + i], dtap_t[i]);
      dtap_s[i] = __builtin_fmaf(gs[r], xs[r + i], dtap_s[i]);
    }
    if (fok && t < Tn) {
      stf(dzt + (rowb + t) * f + c, at);
      stf(dzs + (rowb + t) * f + c, as);
    }
  }
  // reduce the tap partials over the token groups of the tile
  __shared__ float red[SB_GRP][SB_FF][2 * KC];
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    red[grp][fl][i] = dtap_t[i];
    red[grp][fl][KC + i] = dtap_s[i];
  }
  __syncthreads();
  if (grp == 0 && fok) {
    const int ntile = gridDim.x;
    for (int i = 0; i < 2 * KC; ++i) {
      float s = 0.f;
      for (int g2 = 0; g2 < SB_GRP; ++g2) s += red[g2][fl][i];
      const int p = i / KC, tap = i % KC;
      part[((((size_t)b * ntile + tile) * 2 + p) * f + c) * KC + tap] = s;
    }
  }
}

// dconv_p[c][i] = sum over sequences and tiles of the partials
__global__ void __launch_bounds__(256)
dtaps_sum_kernel(const float* __restrict__ part, float* __restrict__ dconv_t,
                 float* __restrict__ dconv_s, int f, int kc, int ntile, int B) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int n = 2 * f * kc;
  if (i >= n) return;
  const int p = i / (f * kc), e = i % (f * kc);
  float s = 0.f;
  for (int b = 0; b < B; ++b)
    for (int tl = 0; tl < ntile; ++tl) s += part[(((size_t)b * ntile + tl) * 2 + p) * f * kc + e];
  (p == 0 ? dconv_t : dconv_s)[e] = s;
}

}  // namespace

hipError_t launch_to_feature_major(const void* in, void* out, int B, int T, int rows, int TC,
                                   int F, int dt, hipStream_t s) {
  dim3 grid((TC + 31) / 32, (F + 31) / 32, B);
  if (dt == BF16)
    hipLaunchKernelGGL(to_feature_major_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)in,
                       (bf16_t*)out, T, rows, TC, F);
  else
    hipLaunchKernelGGL(to_feature_major_kernel<float>, grid, dim3(256), 0, s, (const float*)in,
                       (float*)out, T, rows, TC, F);
  return hipGetLastError();
}

hipError_t launch_to_token_major(const void* in, int in_dt, void* out, int out_dt, int B, int T,
                                 int TC, int F, const float* scale, int chunk, int n,
                                 hipStream_t s) {
  dim3 grid((T + 31) / 32, (F + 31) / 32, B);
#define TTCD_TTM(TI, TO)                                                                         \
  hipLaunchKernelGGL((to_token_major_kernel<TI, TO>), grid, dim3(256), 0, s, (const TI*)in,    \
                     (TO*)out, T, TC, F, scale, chunk, n)
  if (in_dt == BF16 && out_dt == BF16) TTCD_TTM(bf16_t, bf16_t);
  else if (in_dt == BF16) TTCD_TTM(bf16_t, float);
  else if (out_dt == BF16) TTCD_TTM(float, bf16_t);
  else TTCD_TTM(float, float);
#undef TTCD_TTM
  return hipGetLastError();
}

hipError_t launch_scale_token_cols(void* x, const float* sc, int rows, int B, int T, int TC,
                                   int Tpad, int dt, hipStream_t s) {
  const long n = (long)rows * B * TC;
  dim3 grid((unsigned)((n + 255) / 256));
  if (dt == BF16)
    hipLaunchKernelGGL(scale_token_cols_kernel<bf16_t>, grid, dim3(256), 0, s, (bf16_t*)x, sc, rows,
                       T, TC, Tpad, B);
  else
    hipLaunchKernelGGL(scale_token_cols_kernel<float>, grid, dim3(256), 0, s, (float*)x, sc, rows, T,
                       TC, Tpad, B);
  return hipGetLastError();
}

hipError_t launch_chunk_suffix(const float* ds, void* g, void* g_lo, float* total, long n,
                               int nch, int B, int dt, hipStream_t s) {
  if (n % 4) return hipErrorInvalidValue;
  dim3 grid((unsigned)((n / 4 + 255) / 256));
  if (dt == BF16)
    hipLaunchKernelGGL(chunk_suffix_kernel<bf16_t>, grid, dim3(256), 0, s, ds, (bf16_t*)g,
                       (bf16_t*)g_lo, total, n, nch, B);
  else
    hipLaunchKernelGGL(chunk_suffix_kernel<float>, grid, dim3(256), 0, s, ds, (float*)g,
                       (float*)nullptr, total, n, nch, B);
  return hipGetLastError();
}

hipError_t launch_split_bf16(const float* x, void* hi, void* lo, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(split_bf16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x,
                     (bf16_t*)hi, (bf16_t*)lo, n);
  return hipGetLastError();
}

size_t dbeta_part_floats(int B, int nch, int d) { return (size_t)B * nch * ((d + 15) / 16); }

hipError_t launch_dbeta(const float* rt, float* pt, const float* beta, float* part, float* dbeta,
                        int B, int d, int chunk, int T, int TC, int nch, hipStream_t s) {
  const int ngrp = (d + 15) / 16;
  hipLaunchKernelGGL(dbeta_part_kernel, dim3(ngrp, nch, B), dim3(256), 0, s, rt, pt, beta, part,
                     d, chunk, T, TC, nch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int total = B * nch;
  hipLaunchKernelGGL(dbeta_sum_kernel, dim3((total + 63) / 64), dim3(64), 0, s, part, dbeta, ngrp,
                     total);
  return hipGetLastError();
}

hipError_t launch_key_dot(const void* khat, const float* dk, const float* beta, float* kd, int B,
                          int T, int f, int chunk, int nch, int dt, hipStream_t s) {
  const long rows = (long)B * T;
  dim3 grid((unsigned)((rows + 3) / 4));
  if (dt == BF16)
    hipLaunchKernelGGL(key_dot_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)khat, dk, beta,
                       kd, T, f, chunk, nch, rows);
  else
    hipLaunchKernelGGL(key_dot_kernel<float>, grid, dim3(256), 0, s, (const float*)khat, dk, beta,
                       kd, T, f, chunk, nch, rows);
  return hipGetLastError();
}

size_t stream_bwd_part_floats(int B, int T, int f, int kc) {
  const int ntile = (T + SB_TT - 1) / SB_TT;
  return (size_t)B * ntile * 2 * f * kc;
}

hipError_t launch_stream_bwd(const StreamBwdArgs& a, hipStream_t s) {
  const int ntile = (a.T + SB_TT - 1) / SB_TT;
  dim3 grid(ntile, (a.f + SB_FF - 1) / SB_FF, a.B);
  const int Tpad = (a.T + 63) / 64 * 64;
  const float inv_eps = 1.f / a.eps;
#define TTCD_SBW(T_, O_, K)                                                                      \
  hipLaunchKernelGGL((stream_bwd_kernel<T_, O_, K>), grid, dim3(256), 0, s, (const T_*)a.zt,     \
                     (const T_*)a.zs, (const T_*)a.conv_t, (const T_*)a.conv_s, a.dk, a.ddbar,    \
                     a.kd, a.inv, a.beta, (O_*)a.dzt, (O_*)a.dzs, a.part, a.T, Tpad, a.f,          \
                     a.chunk, a.nch, inv_eps)
#define TTCD_SBW_KC(K)                                                                           \
  case K:                                                                                        \
    if (a.in_dt == BF16 && a.out_dt == BF16) TTCD_SBW(bf16_t, bf16_t, K);                        \
    else if (a.in_dt == BF16) TTCD_SBW(bf16_t, float, K);                                        \
    else if (a.out_dt == BF16) TTCD_SBW(float, bf16_t, K);                                       \
    else TTCD_SBW(float, float, K);                                                              \
    break;
  switch (a.kc) {
    TTCD_SBW_KC(1) TTCD_SBW_KC(2) TTCD_SBW_KC(3) TTCD_SBW_KC(4)
    TTCD_SBW_KC(5) TTCD_SBW_KC(6) TTCD_SBW_KC(7) TTCD_SBW_KC(8)
    default: return hipErrorInvalidValue;
  }
#undef TTCD_SBW_KC
#undef TTCD_SBW
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n = 2 * a.f * a.kc;
  hipLaunchKernelGGL(dtaps_sum_kernel, dim3((n + 255) / 256), dim3(256), 0, s, a.part, a.dconv_t,
                     a.dconv_s, a.f, a.kc, ntile, a.B);
  return hipGetLastError();
}

}  // namespace ttcd
