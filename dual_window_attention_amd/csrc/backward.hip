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

// out[b][a][t] = R^T[a][b * TC + t] * s[b * Tpad + t] for t < T, 0 for
// T <= t < Tpad: the forward's write-scaled R~^T (one row of d per
// workgroup column) from the unscaled fp32 R^T
template <typename T>
__global__ void __launch_bounds__(256)
scaled_rt_kernel(const float* __restrict__ rt, const float* __restrict__ s, T* __restrict__ out,
                 int Tn, int TC, int Tpad, int B) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= Tpad) return;
  const int a = blockIdx.y, b = blockIdx.z;
  const float v = t < Tn ? rt[((size_t)a * B + b) * TC + t] * s[(size_t)b * Tpad + t] : 0.f;
  stf(out + ((size_t)b * gridDim.y + a) * Tpad + t, v);
}

// Exclusive suffix sums of the chunk gradients, per sequence:
//   G_j = sum_{i > j} dS_i  (element type),  total += sum_i dS_i  (fp32,
// summed over the batch).  Each thread owns 4 consecutive entries and walks
// the chunks from the last, 8 loads in flight at a time, the running sum in
// fp32.  dS arrives in fp32; G is stored as g (the operand dtype) and, for
// bf16, also as the remainder g_lo = bf16(G - g), so that a product with
// g + g_lo carries G to about fp32 accuracy.  Each 4-entry group is written
// with one access.
template <typename T>
__global__ void __launch_bounds__(256)
chunk_suffix_kernel(const float* __restrict__ ds, T* __restrict__ g, T* __restrict__ g_lo,
                    float* __restrict__ total, long n, int nch, int B) {
  typedef T T4 __attribute__((ext_vector_type(4)));
  const long e = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= n) return;
  float tot[4] = {0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < B; ++b) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = nch - 1; j0 >= 0; j0 -= 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 - u;
        if (j >= 0) v[u] = *reinterpret_cast<const f32x4*>(ds + ((size_t)b * nch + j) * n + e);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 - u;
        if (j < 0) break;
        const size_t off = ((size_t)b * nch + j) * n + e;
        T4 hv, lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          T h;
          stf(&h, acc[i]);
          hv[i] = h;
          if (g_lo) {
            T l;
            stf(&l, acc[i] - ldf(&h));
            lo[i] = l;
          }
        }
        *reinterpret_cast<T4*>(g + off) = hv;
        if (g_lo) *reinterpret_cast<T4*>(g_lo + off) = lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += v[u][i];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) tot[i] += acc[i];
  }
  *reinterpret_cast<f32x4*>(total + e) = f32x4{tot[0], tot[1], tot[2], tot[3]};
}

// out[i] = sum_z parts[z][i], z in a fixed order (the K slices of a product)
__global__ void __launch_bounds__(256)
sum_slices_kernel(const float* __restrict__ parts, float* __restrict__ out, long n, int S) {
  const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 acc = *reinterpret_cast<const f32x4*>(parts + i);
  for (int z = 1; z < S; ++z) acc += *reinterpret_cast<const f32x4*>(parts + (size_t)z * n + i);
  *reinterpret_cast<f32x4*>(out + i) = acc;
}

// out[i] = sum_z parts[z][i] in the element type of out (fixed slice order)
template <typename OutT>
__global__ void __launch_bounds__(256)
sum_slices_to_kernel(const float* __restrict__ parts, OutT* __restrict__ out, long n, int S) {
  const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 acc = *reinterpret_cast<const f32x4*>(parts + i);
  for (int z = 1; z < S; ++z) acc += *reinterpret_cast<const f32x4*>(parts + (size_t)z * n + i);
#pragma unroll
  for (int e = 0; e < 4; ++e) stf(out + i + e, acc[e]);
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
//   dR^T[a][t] = beta_j P^T[a][t], written in the gradient's type (OutT)
template <typename OutT>
__global__ void __launch_bounds__(256)
dbeta_part_kernel(const float* __restrict__ rt, const float* __restrict__ pt,
                  const float* __restrict__ beta, float* __restrict__ part,
                  OutT* __restrict__ drt, int d, int chunk, int Tn, int TC, int nch) {
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
      stf(drt + i, bj * p);
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

// The per-token end of the backward.  Each wave walks 64 consecutive tokens
// (plus the kc-1 after them) for V consecutive features per lane, keeping
// the last kc rows of z_T, z_S and of dzbar_T, dzbar_S in registers:
//   zbar_S[tau] = conv_S(z_s) (recomputed), k = zbar_S * inv,
//   dzbar_S = (beta dK - k kd) inv - ddbar   (|zbar_S| > eps)
//           = beta dK inv - ddbar             (otherwise; inv = 1/eps)
//   dzbar_T = ddbar
//   dz_p[t] = sum_i taps_p[i] dzbar_p[t + kc-1-i],  dtaps_p[i] += dzbar_p[t] z_p[t-(kc-1)+i]
// kd already holds beta (k . dK).  A workgroup is four waves over 256
// consecutive tokens; its dtaps partial sums go to part[b][tile][2][f][kc]
// (teacher, student).
constexpr int SB_L = 64, SB_W = 4, SB_TT = SB_L * SB_W;
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int V, typename T>
TTCD_DEV void ldv(const T* p, float* o) {
  if constexpr (sizeof(T) == 2) {
    if constexpr (V == 4) {
      const u32x2 u = *reinterpret_cast<const u32x2*>(p);
      o[0] = __uint_as_float(u[0] << 16); o[1] = __uint_as_float(u[0] & 0xffff0000u);
      o[2] = __uint_as_float(u[1] << 16); o[3] = __uint_as_float(u[1] & 0xffff0000u);
    } else {
      const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
      o[0] = __uint_as_float(u << 16); o[1] = __uint_as_float(u & 0xffff0000u);
    }
  } else {
    if constexpr (V == 4) {
      const f32x4 u = *reinterpret_cast<const f32x4*>(p);
      o[0] = u[0]; o[1] = u[1]; o[2] = u[2]; o[3] = u[3];
    } else {
      const f32x2 u = *reinterpret_cast<const f32x2*>(p);
      o[0] = u[0]; o[1] = u[1];
    }
  }
}

template <int V, typename T>
TTCD_DEV void stv(T* p, const float* v) {
  if constexpr (sizeof(T) == 2) {
    if constexpr (V == 4)
      *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    else
      *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(v[0], v[1]);
  } else {
    if constexpr (V == 4)
      *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    else
      *reinterpret_cast<f32x2*>(p) = f32x2{v[0], v[1]};
  }
}

template <typename T, typename OutT, int KC, int V>
__global__ void __launch_bounds__(256)
stream_bwd_kernel(const T* __restrict__ zt, const T* __restrict__ zs,
                  const T* __restrict__ conv_t, const T* __restrict__ conv_s,
                  const float* __restrict__ dk, const float* __restrict__ ddbar,
                  const float* __restrict__ kd, const float* __restrict__ inv,
                  const float* __restrict__ beta, OutT* __restrict__ dzt, OutT* __restrict__ dzs,
                  float* __restrict__ part, int Tn, int Tpad, int f, int chunk, int nch,
                  float inv_eps) {
  constexpr int H = KC - 1;
  constexpr int NSTEP = SB_L + H;
  const int b = blockIdx.z;
  const int tile = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = (blockIdx.y * 64 + lane) * V;
  const bool fok = c < f;
  const int t0 = tile * SB_TT + wv * SB_L;             // this wave's first token
  const size_t rowb = (size_t)b * Tn;
  float wt[KC][V], ws[KC][V];
#pragma unroll
  for (int e = 0; e < V; ++e)
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      wt[i][e] = fok ? ldf(conv_t + (size_t)(c + e) * KC + i) : 0.f;
      ws[i][e] = fok ? ldf(conv_s + (size_t)(c + e) * KC + i) : 0.f;
    }
  // rings: slot j holds row tau - H + j (slot H the newest)
  float xt[KC][V], xs[KC][V], gt[KC][V], gs[KC][V];
  float dtt[KC][V], dts[KC][V];
#pragma unroll
  for (int j = 0; j < KC; ++j)
#pragma unroll
    for (int e = 0; e < V; ++e) {
      xt[j][e] = xs[j][e] = gt[j][e] = gs[j][e] = 0.f;
      dtt[j][e] = dts[j][e] = 0.f;
    }
#pragma unroll
  for (int j = 1; j < KC; ++j) {     // rows t0 - H .. t0 - 1 into slots 0 .. H-1 (after a shift)
    const int tau = t0 - KC + j;
    if (fok && tau >= 0 && tau < Tn) {
      ldv<V>(zt + (rowb + tau) * f + c, xt[j]);
      ldv<V>(zs + (rowb + tau) * f + c, xs[j]);
    }
  }
  for (int s0 = 0; s0 < NSTEP; s0 += KC) {
#pragma unroll
    for (int u = 0; u < KC; ++u) {
      const int st = s0 + u;
      const int tau = t0 + st;
      const bool row = st < NSTEP && tau < Tn;
#pragma unroll
      for (int j = 0; j < H; ++j)
#pragma unroll
        for (int e = 0; e < V; ++e) {
          xt[j][e] = xt[j + 1][e];
          xs[j][e] = xs[j + 1][e];
          gt[j][e] = gt[j + 1][e];
          gs[j][e] = gs[j + 1][e];
        }
      float nt[V], ns[V], gk[V], dd[V];
#pragma unroll
      for (int e = 0; e < V; ++e) nt[e] = ns[e] = gk[e] = dd[e] = 0.f;
      float iv = 0.f, bj = 0.f, kdv = 0.f;
      if (row) {
        const size_t ti = rowb + tau;
        if (fok) {
          ldv<V>(zt + ti * f + c, nt);
          ldv<V>(zs + ti * f + c, ns);
          ldv<V>(dk + ti * f + c, gk);
          ldv<V>(ddbar + ti * f + c, dd);
        }
        iv = inv[(size_t)b * Tpad + tau];
        bj = beta[(size_t)b * nch + tau / chunk];
        kdv = kd[ti];
      }
#pragma unroll
      for (int e = 0; e < V; ++e) {
        xt[H][e] = nt[e];
        xs[H][e] = ns[e];
        float zb = 0.f;
#pragma unroll
        for (int i = 0; i < KC; ++i) zb = __builtin_fmaf(ws[i][e], xs[i][e], zb);
        float dz;
        if (iv < inv_eps)
          dz = (bj * gk[e] - zb * iv * kdv) * iv;   // (dk - k (k . dk)) / |zbar|, dk = beta dK
        else
          dz = bj * gk[e] * iv;                      // dk / eps
        gt[H][e] = row ? dd[e] : 0.f;
        gs[H][e] = row ? dz - dd[e] : 0.f;
      }
      if (row && st < SB_L) {
#pragma unroll
        for (int i = 0; i < KC; ++i)
#pragma unroll
          for (int e = 0; e < V; ++e) {
            dtt[i][e] = __builtin_fmaf(gt[H][e], xt[i][e], dtt[i][e]);
            dts[i][e] = __builtin_fmaf(gs[H][e], xs[i][e], dts[i][e]);
          }
      }
      const int t = tau - H;
      if (st >= H && st < NSTEP && t < Tn && fok) {
        float at[V], as[V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
          at[e] = as[e] = 0.f;
#pragma unroll
          for (int i = 0; i < KC; ++i) {
            at[e] = __builtin_fmaf(wt[i][e], gt[H - i][e], at[e]);
            as[e] = __builtin_fmaf(ws[i][e], gs[H - i][e], as[e]);
          }
        }
        stv<V>(dzt + (rowb + t) * f + c, at);
        stv<V>(dzs + (rowb + t) * f + c, as);
      }
    }
  }
  // the workgroup's tap partials: sum over its four waves, one path at a time
  __shared__ float red[SB_W][64][KC * V];
  const int ntile = gridDim.x;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int i = 0; i < KC; ++i)
#pragma unroll
      for (int e = 0; e < V; ++e) red[wv][lane][e * KC + i] = p == 0 ? dtt[i][e] : dts[i][e];
    __syncthreads();
    if (wv == 0 && fok) {
      float* dst = part + (((size_t)b * ntile + tile) * 2 + p) * f * KC + (size_t)c * KC;
#pragma unroll
      for (int q = 0; q < KC * V; ++q) {
        float s_ = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < SB_W; ++w2) s_ += red[w2][lane][q];
        dst[q] = s_;
      }
    }
    __syncthreads();
  }
}

// dconv_p[c][i] = sum over sequences and tiles of the partials: 64 outputs
// per workgroup, each wave summing every fourth partial row, then the four
// sums in a fixed order
__global__ void __launch_bounds__(256)
dtaps_sum_kernel(const float* __restrict__ part, float* __restrict__ dconv_t,
                 float* __restrict__ dconv_s, int f, int kc, int nrows) {
  const int n = 2 * f * kc;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + lane;
  float s = 0.f;
  if (i < n)
    for (int r = wv; r < nrows; r += 4) s += part[(size_t)r * n + i];
  __shared__ float red[4][64];
  red[wv][lane] = s;
  __syncthreads();
  if (wv == 0 && i < n) {
    const float tot = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
    const int p = i / (f * kc), e = i % (f * kc);
    (p == 0 ? dconv_t : dconv_s)[e] = tot;
  }
}

}  // namespace

hipError_t launch_to_feature_major(const void* in, void* out, int B, int T, int rows, int TC,
                                   int F, int dt, hipStream_t s) {
  // out[f][b * TC + t] = in[b][t][f] (t < T), zero for T <= t < TC
  return launch_transpose64(in, dt, F, (long)rows * F, T, F, out, dt, (long)B * TC, TC, TC, B,
                            nullptr, 0, 1, s);
}

hipError_t launch_to_token_major(const void* in, int in_dt, void* out, int out_dt, int B, int T,
                                 int TC, int F, const float* scale, int chunk, int n,
                                 hipStream_t s) {
  // out[b][t][f] = in[f][b * TC + t] * (scale ? scale[b * n + t / chunk] : 1)
  return launch_transpose64(in, in_dt, (long)B * TC, TC, F, T, out, out_dt, F, (long)T * F, F, B,
                            scale, n, scale ? chunk : 1, s);
}

hipError_t launch_scaled_rt(const float* rt, const float* sc, void* out, int out_dt, int d, int T,
                            int TC, int Tpad, int B, hipStream_t s) {
  if (d <= 0 || B <= 0 || Tpad <= 0) return hipSuccess;
  const dim3 grid((unsigned)((Tpad + 255) / 256), (unsigned)d, (unsigned)B);
  if (out_dt == BF16)
    hipLaunchKernelGGL(scaled_rt_kernel<bf16_t>, grid, dim3(256), 0, s, rt, sc, (bf16_t*)out, T, TC,
                       Tpad, B);
  else
    hipLaunchKernelGGL(scaled_rt_kernel<float>, grid, dim3(256), 0, s, rt, sc, (float*)out, T, TC,
                       Tpad, B);
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

hipError_t launch_sum_slices(const float* parts, float* out, long n, int S, hipStream_t s) {
  if (n % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sum_slices_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s,
                     parts, out, n, S);
  return hipGetLastError();
}

hipError_t launch_sum_slices_to(const float* parts, void* out, long n, int S, int out_dt,
                                hipStream_t s) {
  if (n % 4) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((n / 4 + 255) / 256));
  if (out_dt == BF16)
    hipLaunchKernelGGL(sum_slices_to_kernel<bf16_t>, grid, dim3(256), 0, s, parts, (bf16_t*)out,
                       n, S);
  else
    hipLaunchKernelGGL(sum_slices_to_kernel<float>, grid, dim3(256), 0, s, parts, (float*)out, n,
                       S);
  return hipGetLastError();
}

hipError_t launch_split_bf16(const float* x, void* hi, void* lo, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(split_bf16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x,
                     (bf16_t*)hi, (bf16_t*)lo, n);
  return hipGetLastError();
}

size_t dbeta_part_floats(int B, int nch, int d) { return (size_t)B * nch * ((d + 15) / 16); }

hipError_t launch_dbeta(const float* rt, const float* pt, const float* beta, float* part,
                        float* dbeta, void* drt, int drt_dt, int B, int d, int chunk, int T,
                        int TC, int nch, hipStream_t s) {
  const int ngrp = (d + 15) / 16;
  if (drt_dt == BF16)
    hipLaunchKernelGGL(dbeta_part_kernel<bf16_t>, dim3(ngrp, nch, B), dim3(256), 0, s, rt, pt,
                       beta, part, (bf16_t*)drt, d, chunk, T, TC, nch);
  else
    hipLaunchKernelGGL(dbeta_part_kernel<float>, dim3(ngrp, nch, B), dim3(256), 0, s, rt, pt,
                       beta, part, (float*)drt, d, chunk, T, TC, nch);
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
  if (a.f % 8) return hipErrorInvalidValue;
  const int ntile = (a.T + SB_TT - 1) / SB_TT;
  const int Tpad = (a.T + 63) / 64 * 64;
  const float inv_eps = 1.f / a.eps;
#define TTCD_SBW(T_, O_, K, V)                                                                   \
  hipLaunchKernelGGL((stream_bwd_kernel<T_, O_, K, V>),                                          \
                     dim3(ntile, (a.f / V + 63) / 64, a.B), dim3(256), 0, s, (const T_*)a.zt,    \
                     (const T_*)a.zs, (const T_*)a.conv_t, (const T_*)a.conv_s, a.dk, a.ddbar,    \
                     a.kd, a.inv, a.beta, (O_*)a.dzt, (O_*)a.dzs, a.part, a.T, Tpad, a.f,          \
                     a.chunk, a.nch, inv_eps)
#define TTCD_SBW_KC(K)                                                                           \
  case K: {                                                                                      \
    constexpr int V = K <= 4 ? 4 : 2;                                                            \
    if (a.in_dt == BF16 && a.out_dt == BF16) TTCD_SBW(bf16_t, bf16_t, K, V);                     \
    else if (a.in_dt == BF16) TTCD_SBW(bf16_t, float, K, V);                                     \
    else if (a.out_dt == BF16) TTCD_SBW(float, bf16_t, K, V);                                    \
    else TTCD_SBW(float, float, K, V);                                                           \
    break;                                                                                       \
  }
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
  hipLaunchKernelGGL(dtaps_sum_kernel, dim3((n + 63) / 64), dim3(256), 0, s, a.part, a.dconv_t,
                     a.dconv_s, a.f, a.kc, a.B * ntile);
  return hipGetLastError();
}

}  // namespace ttcd
