// Bandwidth-bound kernels of the IP-TTCD layer on gfx950:
//   * the fast-weight stream (papernotes.org notes on "Learning What to
//     Remember", key design 3): depthwise short causal convs of both paths,
//     their difference, and the per-token l2 norm of the student keys;
//   * RMSNorm of the residual stream (the declared pre-norm glue);
//   * layout transposes that turn token-major tensors into the
//     token-contiguous operands of the chunk-write contraction.
#include "common.hpp"
#include "kernels.hpp"

namespace ttcd {

namespace {

// --------------------------------------------------------------- fw stream
constexpr int ST_T = 64;     // tokens per workgroup
constexpr int ST_F = 64;     // features per slab
constexpr int MAXK = 8;      // max conv taps

template <typename T>
struct Vec16;
template <>
struct Vec16<bf16_t> {
  static constexpr int N = 8;
  static TTCD_DEV void load(const bf16_t* p, float* out) {
    u32x4 v = ld16(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(v[i] << 16);
      out[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
  }
  static TTCD_DEV void store(bf16_t* p, const float* in) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(in[2 * i], in[2 * i + 1]);
    st16(p, v);
  }
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  static TTCD_DEV void load(const float* p, float* out) {
    f32x4 v = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = v[i];
  }
  static TTCD_DEV void store(float* p, const float* in) {
    *reinterpret_cast<f32x4*>(p) = f32x4{in[0], in[1], in[2], in[3]};
  }
};

template <typename T>
__global__ void __launch_bounds__(256)
fw_stream_kernel(const T* __restrict__ zt, const T* __restrict__ zs,
                 const T* __restrict__ conv_t, const T* __restrict__ conv_s,
                 const float* __restrict__ beta, T* __restrict__ dbar, T* __restrict__ zbt,
                 float* __restrict__ sc, int T_, int Tpad, int f, int kc, int chunk,
                 int nchunks, float eps) {
  constexpr int VN = Vec16<T>::N;
  __shared__ float zts[ST_T + MAXK - 1][ST_F + 1];
  __shared__ float zss[ST_T + MAXK - 1][ST_F + 1];
  __shared__ float tap_t[ST_F][MAXK];
  __shared__ float tap_s[ST_F][MAXK];
  __shared__ float zbT[ST_F][ST_T + 1];

  const int b = blockIdx.y;
  const int t0 = blockIdx.x * ST_T;
  const int tid = threadIdx.x;
  const int tok = tid >> 2, fq = tid & 3;      // compute mapping
  const int t = t0 + tok;
  const int halo = kc - 1;
  const int nrows = ST_T + halo;
  const size_t zoff = (size_t)b * T_ * f;
  const T* ztb = zt + zoff;
  const T* zsb = zs + zoff;
  float ssq = 0.f;

  for (int c0 = 0; c0 < f; c0 += ST_F) {
    __syncthreads();
    // stage the slab (rows t0-halo .. t0+63) of both paths
    constexpr int CPR = ST_F / VN;   // vector chunks per row
    for (int e = tid; e < nrows * CPR; e += 256) {
      const int row = e / CPR, cc = e % CPR;
      const int tt = t0 - halo + row;
      const int c = c0 + cc * VN;
      float a[VN], bb[VN];
      if (tt >= 0 && tt < T_ && c < f) {
        Vec16<T>::load(ztb + (size_t)tt * f + c, a);
        Vec16<T>::load(zsb + (size_t)tt * f + c, bb);
      } else {
#pragma unroll
        for (int i = 0; i < VN; ++i) a[i] = bb[i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < VN; ++i) {
        zts[row][cc * VN + i] = a[i];
        zss[row][cc * VN + i] = bb[i];
      }
    }
    for (int e = tid; e < ST_F * kc; e += 256) {
      const int cc = e / kc, k = e % kc;
      const int c = c0 + cc;
      tap_t[cc][k] = c < f ? ldf(conv_t + (size_t)c * kc + k) : 0.f;
      tap_s[cc][k] = c < f ? ldf(conv_s + (size_t)c * kc + k) : 0.f;
    }
    __syncthreads();

    // conv of 16 features of one token
    float dv[16];
    const bool tok_ok = t < T_;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int cc = fq * 16 + i;
      float at = 0.f, as = 0.f;
      for (int k = 0; k < kc; ++k) {
        at = __builtin_fmaf(tap_t[cc][k], zts[tok + k][cc], at);
        as = __builtin_fmaf(tap_s[cc][k], zss[tok + k][cc], as);
      }
      if (!tok_ok) at = as = 0.f;
      dv[i] = at - as;
      zbT[cc][tok] = as;
      ssq = __builtin_fmaf(as, as, ssq);
    }
    if (t < Tpad) {
      T* dp = dbar + ((size_t)b * Tpad + t) * f + c0 + fq * 16;
#pragma unroll
      for (int i = 0; i < 16; i += VN)
        if (c0 + fq * 16 + i < f) Vec16<T>::store(dp + i, dv + i);
    }
    __syncthreads();
    // transposed write: feature row fr, 16 tokens per thread
    {
      const int fr = tid >> 2, tq = tid & 3;
      const int c = c0 + fr;
      if (c < f) {
        T* zp = zbt + ((size_t)b * f + c) * Tpad + t0 + tq * 16;
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = zbT[fr][tq * 16 + i];
#pragma unroll
        for (int i = 0; i < 16; i += VN)
          if (t0 + tq * 16 + i < Tpad) Vec16<T>::store(zp + i, v + i);
      }
    }
  }
  // per-token norm -> scale beta_i / max(||zbar_s||, eps)
  ssq += __shfl_xor(ssq, 1, 64);
  ssq += __shfl_xor(ssq, 2, 64);
  if (fq == 0 && t < Tpad) {
    float v = 0.f;
    if (t < T_) {
      const int ci = min(t / chunk, nchunks - 1);
      v = beta[(size_t)b * nchunks + ci] / fmaxf(sqrtf(ssq), eps);
    }
    sc[(size_t)b * Tpad + t] = v;
  }
}

// --------------------------------------------------------------- rmsnorm
template <typename GT, typename OutT>
__global__ void __launch_bounds__(256)
rmsnorm_kernel(const float* __restrict__ h, const GT* __restrict__ gamma, OutT* __restrict__ u,
               int rows, int d, float eps) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + wave;
  if (row >= rows) return;
  const float* hr = h + row * d;
  float ss = 0.f;
  for (int i = lane * 4; i < d; i += 256) {
    f32x4 v = *reinterpret_cast<const f32x4*>(hr + i);
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = wave_sum(ss);
  const float rs = 1.f / sqrtf(ss / d + eps);
  OutT* ur = u + row * d;
  for (int i = lane * 4; i < d; i += 256) {
    f32x4 v = *reinterpret_cast<const f32x4*>(hr + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float gm = gamma ? ldf(gamma + i + e) : 1.f;
      stf(ur + i + e, v[e] * rs * gm);
    }
  }
}

// --------------------------------------------------------------- transposes
template <typename E>
__global__ void __launch_bounds__(256)
transpose_kernel(const E* __restrict__ in, E* __restrict__ out, int rows, int cols, long ld_in,
                 long ld_out, long s_in, long s_out) {
  __shared__ E tile[32][33];
  const int z = blockIdx.z;
  const long r0 = (long)blockIdx.x * 32, c0 = (long)blockIdx.y * 32;
  const E* ip = in + z * s_in;
  E* op = out + z * s_out;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    const long r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < rows && c < cols) ? ip[r * ld_in + c] : E(0);
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const long c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows) op[c * ld_out + r] = tile[tx][i];
  }
}

// V [B, kv_rows, Hkv, D] -> vt [B, Hkv, D, vt_ld] (bf16), the keys of every
// aligned group of 16 stored in the order that makes the 8 keys one MFMA lane
// needs contiguous (bits 2 and 3 of the key index swapped).  Only keys in
// [jlo, Tk) are read; the other columns are zero.
__global__ void __launch_bounds__(256)
v_transpose_kernel(const uint16_t* __restrict__ v, uint16_t* __restrict__ vt, int Tk, int jlo,
                   int kv_rows, int Hkv, int D, int vt_ld) {
  __shared__ uint16_t tile[64][65];
  const int bg = blockIdx.z;
  const int b = bg / Hkv, g = bg % Hkv;
  const long j0 = (long)blockIdx.x * 64;
  const int d0 = blockIdx.y * 64;
  const uint16_t* vp = v + ((size_t)b * kv_rows * Hkv + g) * D;
  uint16_t* op = vt + (size_t)bg * D * vt_ld;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const long j = j0 + i;
    const int d = d0 + tx;
    tile[i][tx] = (j >= jlo && j < Tk && d < D) ? vp[j * Hkv * D + d] : (uint16_t)0;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int d = d0 + i;
    const int col = tx;                                   // storage column within the tile
    const int key = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1);
    if (d < D && j0 + col < vt_ld) op[(size_t)d * vt_ld + j0 + col] = tile[key][i];
  }
}

// out[b][c][r] = in[b][r][c] * (scale ? scale[b * nscale + r / rows_per_scale] : 1)
template <typename T>
__global__ void __launch_bounds__(256)
transpose_scale_kernel(const T* __restrict__ in, T* __restrict__ out, int rows, int cols,
                       const float* __restrict__ scale, int rows_per_scale, int nscale) {
  __shared__ float tile[32][33];
  const int z = blockIdx.z;
  const long r0 = (long)blockIdx.x * 32, c0 = (long)blockIdx.y * 32;
  const T* ip = in + (size_t)z * rows * cols;
  T* op = out + (size_t)z * rows * cols;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    const long r = r0 + i, c = c0 + tx;
    float v = 0.f;
    if (r < rows && c < cols) {
      v = ldf(ip + r * cols + c);
      if (scale) v *= scale[(size_t)z * nscale + r / rows_per_scale];
    }
    tile[i][tx] = v;
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const long c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows) stf(op + c * rows + r, tile[tx][i]);
  }
}

// --------------------------------------------------------------- small helpers
__global__ void add_kernel(const float* a, const float* b, float* o, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) o[i] = a[i] + b[i];
}

template <typename InT>
__global__ void widen_repeat_kernel(const InT* in, float* out, long n, int batch) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = ldf(in + i);
  for (int b = 0; b < batch; ++b) out[(size_t)b * n + i] = v;
}

template <typename OutT>
__global__ void convert_kernel(const float* in, OutT* out, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) stf(out + i, in[i]);
}

}  // namespace

hipError_t launch_fw_stream(const StreamArgs& a, hipStream_t s) {
  const int Tpad = (a.T + 63) / 64 * 64;
  dim3 grid(Tpad / ST_T, a.B);
  if (a.in_dt == BF16)
    hipLaunchKernelGGL(fw_stream_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)a.zt,
                       (const bf16_t*)a.zs, (const bf16_t*)a.conv_t, (const bf16_t*)a.conv_s,
                       a.beta, (bf16_t*)a.dbar, (bf16_t*)a.zbt, a.sc, a.T, Tpad, a.f, a.kc,
                       a.chunk, a.nchunks, a.eps);
  else
    hipLaunchKernelGGL(fw_stream_kernel<float>, grid, dim3(256), 0, s, (const float*)a.zt,
                       (const float*)a.zs, (const float*)a.conv_t, (const float*)a.conv_s,
                       a.beta, (float*)a.dbar, (float*)a.zbt, a.sc, a.T, Tpad, a.f, a.kc,
                       a.chunk, a.nchunks, a.eps);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* h, const void* gamma, void* u, int rows, int d, float eps,
                          int in_dt, int out_dt, hipStream_t s) {
  dim3 grid((rows + 3) / 4);
  if (in_dt == BF16) {
    if (out_dt == BF16)
      hipLaunchKernelGGL((rmsnorm_kernel<bf16_t, bf16_t>), grid, dim3(256), 0, s, h,
                         (const bf16_t*)gamma, (bf16_t*)u, rows, d, eps);
    else
      hipLaunchKernelGGL((rmsnorm_kernel<bf16_t, float>), grid, dim3(256), 0, s, h,
                         (const bf16_t*)gamma, (float*)u, rows, d, eps);
  } else {
    if (out_dt == BF16)
      hipLaunchKernelGGL((rmsnorm_kernel<float, bf16_t>), grid, dim3(256), 0, s, h,
                         (const float*)gamma, (bf16_t*)u, rows, d, eps);
    else
      hipLaunchKernelGGL((rmsnorm_kernel<float, float>), grid, dim3(256), 0, s, h,
                         (const float*)gamma, (float*)u, rows, d, eps);
  }
  return hipGetLastError();
}

hipError_t launch_transpose(const void* in, void* out, int rows, int cols, long ld_in,
                            long ld_out, int batch, long s_in, long s_out, int esize,
                            hipStream_t s) {
  dim3 grid((rows + 31) / 32, (cols + 31) / 32, batch > 0 ? batch : 1);
  if (esize == 2)
    hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)in,
                       (uint16_t*)out, rows, cols, ld_in, ld_out, s_in, s_out);
  else
    hipLaunchKernelGGL(transpose_kernel<uint32_t>, grid, dim3(256), 0, s, (const uint32_t*)in,
                       (uint32_t*)out, rows, cols, ld_in, ld_out, s_in, s_out);
  return hipGetLastError();
}

hipError_t launch_v_transpose(const void* v, void* vt, int B, int Tk, int jlo, int kv_rows, int Hkv,
                              int D, int vt_ld, hipStream_t s) {
  dim3 grid(vt_ld / 64, (D + 63) / 64, B * Hkv);
  hipLaunchKernelGGL(v_transpose_kernel, grid, dim3(256), 0, s, (const uint16_t*)v, (uint16_t*)vt,
                     Tk, jlo, kv_rows, Hkv, D, vt_ld);
  return hipGetLastError();
}

hipError_t launch_transpose_scale(const void* in, void* out, int rows, int cols, int batch,
                                  const float* scale, int rows_per_scale, int nscale, int dt,
                                  hipStream_t s) {
  dim3 grid((rows + 31) / 32, (cols + 31) / 32, batch);
  if (dt == BF16)
    hipLaunchKernelGGL(transpose_scale_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)in,
                       (bf16_t*)out, rows, cols, scale, rows_per_scale, nscale);
  else
    hipLaunchKernelGGL(transpose_scale_kernel<float>, grid, dim3(256), 0, s, (const float*)in,
                       (float*)out, rows, cols, scale, rows_per_scale, nscale);
  return hipGetLastError();
}

hipError_t launch_add(const float* a, const float* b, float* out, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(add_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, b, out, n);
  return hipGetLastError();
}

hipError_t launch_widen_repeat(const void* in, float* out, long n, int batch, int in_dt,
                               hipStream_t s) {
  if (n <= 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256));
  if (in_dt == BF16)
    hipLaunchKernelGGL(widen_repeat_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)in, out,
                       n, batch);
  else
    hipLaunchKernelGGL(widen_repeat_kernel<float>, grid, dim3(256), 0, s, (const float*)in, out, n,
                       batch);
  return hipGetLastError();
}

hipError_t launch_convert(const float* in, void* out, long n, int out_dt, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256));
  if (out_dt == BF16)
    hipLaunchKernelGGL(convert_kernel<bf16_t>, grid, dim3(256), 0, s, in, (bf16_t*)out, n);
  else
    hipLaunchKernelGGL(convert_kernel<float>, grid, dim3(256), 0, s, in, (float*)out, n);
  return hipGetLastError();
}

}  // namespace ttcd
