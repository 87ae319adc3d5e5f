// One decode step of the IP-TTCD layer on gfx950 (bandwidth-bound):
//   * dual-window attention of one new query per sequence over the last
//     w_T cached keys, split over the keys (each split keeps a student-band
//     and a far-band online-softmax state) and merged exactly through the
//     log-sum-exp (the README's LSE-combination identity);
//   * the fast-weight MLP output y = W_down^(0) z + sum_j beta_j R_j^T (K_j z)
//     read straight from the low-rank chunk lists, or S z from a dense
//     folded weight (papernotes.org notes, key design 3).
// Keys outside [pos - w_T + 1, pos] are never read.
#include "common.hpp"
#include "kernels.hpp"

namespace ttcd {

namespace {

constexpr float NEG_INF = -__builtin_inff();
constexpr int GMAX = 4;

struct St {
  float m, l;
};

TTCD_DEV void merge_into(float& m, float& l, float* acc, float m2, float l2, const float* acc2,
                         int n) {
  const float mn = fmaxf(m, m2);
  const float a1 = (m == NEG_INF) ? 0.f : fast_exp2(m - mn);
  const float a2 = (m2 == NEG_INF) ? 0.f : fast_exp2(m2 - mn);
  l = l * a1 + l2 * a2;
  for (int i = 0; i < n; ++i) acc[i] = acc[i] * a1 + acc2[i] * a2;
  m = mn;
}

// G: query heads per kv head (the per-head states are sized for it, so
// fewer registers and more resident waves when G is small)
template <typename T, int D, int G>
__global__ void __launch_bounds__(256)
decode_attn_split(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                  float* __restrict__ part, int pos, int kv_rows, int Hq, int Hkv, int wT,
                  int wS, float c, int nsplit, int split_len) {
  static_assert(G >= 1 && G <= GMAX, "query heads per kv head");
  constexpr int LPK = D / 8;           // lanes per key
  constexpr int KPW = 64 / LPK;        // keys per wave step
  constexpr int PS = D + 2;            // floats per partial state
  __shared__ float red[4][G][2][PS];
  // the kv heads of one split run next to each other in dispatch order:
  // together they read whole cache rows (all heads of a token)
  const uint32_t flat = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int g = (int)(flat % gridDim.y);
  const int s = (int)((flat / gridDim.y) % gridDim.x);
  const int b = (int)(flat / (gridDim.y * gridDim.x));
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int dc = lane % LPK, kg = lane / LPK;
  const int jlo = max(0, pos - wT + 1);
  const int ks = jlo + s * split_len;
  const int ke = min(ks + split_len, pos + 1);

  float qv[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const T* qp = q + ((size_t)b * Hq + g * G + hh) * D + dc * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[hh][e] = ldf(qp + e) * c;
  }
  float mS[G], lS[G], aS[G][8], mF[G], lF[G], aF[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    mS[hh] = mF[hh] = NEG_INF;
    lS[hh] = lF[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) aS[hh][e] = aF[hh][e] = 0.f;
  }

  const size_t rs = (size_t)Hkv * D;
  const T* kb = k + ((size_t)b * kv_rows * Hkv + g) * D + dc * 8;
  const T* vb = v + ((size_t)b * kv_rows * Hkv + g) * D + dc * 8;
  // this lane's 8 elements of key j's K and V rows (16-byte loads for bf16),
  // one key step loaded ahead of the one being used
  using Raw = u32x4[sizeof(T) == 2 ? 1 : 2];
  auto fetch = [&](int j, Raw& rk, Raw& rv) {
#pragma unroll
    for (int h2 = 0; h2 < (int)(sizeof(T) == 2 ? 1 : 2); ++h2) {
      rk[h2] = ld16(kb + (size_t)j * rs + h2 * 4);
      rv[h2] = ld16(vb + (size_t)j * rs + h2 * 4);
    }
  };
  auto unpack = [&](const Raw& r, float* o) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] = __uint_as_float(r[0][e] << 16);
        o[2 * e + 1] = __uint_as_float(r[0][e] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = __uint_as_float(r[e / 4][e % 4]);
    }
  };
  // Rows are fetched only from [ks, ke), which lies inside [0, pos] <
  // kv_rows; a split with no key (ks >= ke) fetches nothing and leaves the
  // empty states (m = -inf, l = 0, acc = 0), which merge exactly.  The host
  // launches no such split, but the kernel does not rely on it.
  // two key steps in flight: buffer A holds step i, B step i+1; each step,
  // once unpacked, refills its buffer with the step two ahead
  Raw ak, av, bk, bv;
  if (ks < ke) {
    const int j = ks + wave * KPW + kg;
    fetch(j < ke ? j : ks, ak, av);
    const int j2 = j + 4 * KPW;
    fetch(j2 < ke ? j2 : ks, bk, bv);
  }
  auto step = [&](int j0, Raw& rk, Raw& rv) __attribute__((always_inline)) {
    const int j = j0 + kg;
    const bool ok = j < ke;
    float kv[8], vv[8];
    unpack(rk, kv);
    unpack(rv, vv);
    {
      const int jn = j + 8 * KPW;
      fetch(jn < ke ? jn : ks, rk, rv);       // ks < ke inside the loop
    }
    if (!ok) {
#pragma unroll
      for (int e = 0; e < 8; ++e) kv[e] = vv[e] = 0.f;
    }
    const bool inS = pos - j < wS;
    auto upd = [&](float& m, float& l, float* acc, float sc) {
      const float mn = fmaxf(m, sc);
      const float al = (m == NEG_INF) ? 0.f : fast_exp2(m - mn);
      const float p = fast_exp2(sc - mn);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(p, vv[e], acc[e] * al);
      l = l * al + p;
      m = mn;
    };
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float sc = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) sc = __builtin_fmaf(qv[hh][e], kv[e], sc);
#pragma unroll
      for (int o = 1; o < LPK; o <<= 1) sc += __shfl_xor(sc, o, 64);
      if (!ok) continue;
      if (inS)
        upd(mS[hh], lS[hh], aS[hh], sc);
      else
        upd(mF[hh], lF[hh], aF[hh], sc);
    }
  };
  for (int j0 = ks + wave * KPW; j0 < ke; j0 += 8 * KPW) {
    step(j0, ak, av);
    if (j0 + 4 * KPW >= ke) break;
    step(j0 + 4 * KPW, bk, bv);
  }
  // merge the key groups inside the wave (lanes with equal dc)
  for (int o = LPK; o < 64; o <<= 1) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float m2 = __shfl_xor(mS[hh], o, 64), l2 = __shfl_xor(lS[hh], o, 64), a2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) a2[e] = __shfl_xor(aS[hh][e], o, 64);
      merge_into(mS[hh], lS[hh], aS[hh], m2, l2, a2, 8);
      m2 = __shfl_xor(mF[hh], o, 64);
      l2 = __shfl_xor(lF[hh], o, 64);
#pragma unroll
      for (int e = 0; e < 8; ++e) a2[e] = __shfl_xor(aF[hh][e], o, 64);
      merge_into(mF[hh], lF[hh], aF[hh], m2, l2, a2, 8);
    }
  }
  if (kg == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        red[wave][hh][0][2 + dc * 8 + e] = aS[hh][e];
        red[wave][hh][1][2 + dc * 8 + e] = aF[hh][e];
      }
      if (dc == 0) {
        red[wave][hh][0][0] = mS[hh];
        red[wave][hh][0][1] = lS[hh];
        red[wave][hh][1][0] = mF[hh];
        red[wave][hh][1][1] = lF[hh];
      }
    }
  }
  __syncthreads();
  // wave 0 merges the four waves: thread -> (head, state, d)
  for (int e = tid; e < G * 2 * D; e += 256) {
    const int hh = e / (2 * D), st = (e / D) % 2, d = e % D;
    float m = red[0][hh][st][0], l = red[0][hh][st][1], a = red[0][hh][st][2 + d];
    for (int w = 1; w < 4; ++w) merge_into(m, l, &a, red[w][hh][st][0], red[w][hh][st][1],
                                           &red[w][hh][st][2 + d], 1);
    float* pp = part + ((((size_t)b * Hq + g * G + hh) * nsplit + s) * 2 + st) * PS;
    pp[2 + d] = a;
    if (d == 0) {
      pp[0] = m;
      pp[1] = l;
    }
  }
}

template <typename OutT>
__global__ void __launch_bounds__(128)
decode_attn_combine(const float* __restrict__ part, OutT* __restrict__ o_t,
                    OutT* __restrict__ o_s, float* __restrict__ lse_t,
                    float* __restrict__ lse_s, int Hq, int D, int nsplit) {
  const int bh = blockIdx.x;   // b * Hq + h
  const int PS = D + 2;
  const float* pp = part + (size_t)bh * nsplit * 2 * PS;
  constexpr float LN2 = 0.69314718055994530942f;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float mS = NEG_INF, lS = 0.f, aS = 0.f, mF = NEG_INF, lF = 0.f, aF = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float* p0 = pp + (size_t)(s * 2 + 0) * PS;
      const float* p1 = pp + (size_t)(s * 2 + 1) * PS;
      merge_into(mS, lS, &aS, p0[0], p0[1], p0 + 2 + d, 1);
      merge_into(mF, lF, &aF, p1[0], p1[1], p1 + 2 + d, 1);
    }
    const float os = aS / lS;
    const bool far_empty = lF == 0.f;
    float mT = mS, lT = lS, aT = aS;
    if (!far_empty) merge_into(mT, lT, &aT, mF, lF, &aF, 1);
    const float ot = far_empty ? os : aT / lT;
    stf(o_s + (size_t)bh * D + d, os);
    stf(o_t + (size_t)bh * D + d, ot);
    if (d == 0) {
      const float ls = (mS + fast_log2(lS)) * LN2;
      if (lse_s) lse_s[bh] = ls;
      if (lse_t) lse_t[bh] = far_empty ? ls : (mT + fast_log2(lT)) * LN2;
    }
  }
}

// c[b, t] = beta[b, t / C] * (k_list[b, t] . z[b]) : one wave per list row
template <typename T>
__global__ void __launch_bounds__(256)
list_kdot(const T* __restrict__ klist, const T* __restrict__ z, const float* __restrict__ beta,
          float* __restrict__ cbuf, int rows, int f, int chunk, int n) {
  extern __shared__ float zs[];
  const int b = blockIdx.y;
  for (int i = threadIdx.x; i < f; i += 256) zs[i] = ldf(z + (size_t)b * f + i);
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int RPW = 4;
  for (int rr = 0; rr < RPW; ++rr) {
    const long t = ((long)blockIdx.x * 4 + wave) * RPW + rr;
    if (t >= rows) return;
    const T* kr = klist + ((size_t)b * rows + t) * f;
    float acc = 0.f;
    if (sizeof(T) == 2) {
      for (int c = lane * 8; c < f; c += 512) {
        u32x4 v = ld16(kr + c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc = __builtin_fmaf(__uint_as_float(v[e] << 16), zs[c + 2 * e], acc);
          acc = __builtin_fmaf(__uint_as_float(v[e] & 0xFFFF0000u), zs[c + 2 * e + 1], acc);
        }
      }
    } else {
      for (int c = lane; c < f; c += 64) acc = __builtin_fmaf(ldf(kr + c), zs[c], acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) cbuf[(size_t)b * rows + t] = acc * beta[(size_t)b * n + t / chunk];
  }
}

// ypart[b, seg, a] = sum_{t in seg} c[b, t] r_list[b, t, a]
constexpr int SEG = 1024;
template <typename T>
__global__ void __launch_bounds__(256)
list_raccum(const T* __restrict__ rlist, const float* __restrict__ cbuf, float* __restrict__ ypart,
            int rows, int d) {
  __shared__ float cs[SEG];
  const int seg = blockIdx.x, b = blockIdx.y;
  const long t0 = (long)seg * SEG;
  for (int i = threadIdx.x; i < SEG; i += 256) {
    const long t = t0 + i;
    cs[i] = t < rows ? cbuf[(size_t)b * rows + t] : 0.f;
  }
  __syncthreads();
  const int nseg = gridDim.x;
  for (int a0 = threadIdx.x * 4; a0 < d; a0 += 1024) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    const long tend = min((long)SEG, rows - t0);
    for (long i = 0; i < tend; ++i) {
      const T* rr = rlist + ((size_t)b * rows + t0 + i) * d + a0;
      const float cv = cs[i];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (a0 + e < d) acc[e] = __builtin_fmaf(cv, ldf(rr + e), acc[e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (a0 + e < d) ypart[((size_t)b * nseg + seg) * d + a0 + e] = acc[e];
  }
}

// bf16 fast paths of the two list passes.  K rows: z lives in registers (NCH
// 16-byte column chunks per lane), four rows' loads are in flight at once.
// R rows: 16-byte loads of 8 consecutive features, eight rows in flight per
// thread, the row groups of a workgroup summed through LDS.
template <int NCH>
__global__ void __launch_bounds__(256)
list_kdot_reg(const bf16_t* __restrict__ klist, const bf16_t* __restrict__ z,
              const float* __restrict__ beta, float* __restrict__ cbuf, int rows, int f,
              int chunk, int n) {
  constexpr int RG = 4;                     // rows in flight per wave
  const int b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float zr[NCH][8];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane * 8 + 512 * i;
    if (c < f) {
      const u32x4 v = ld16(z + (size_t)b * f + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        zr[i][2 * e] = __uint_as_float(v[e] << 16);
        zr[i][2 * e + 1] = __uint_as_float(v[e] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) zr[i][e] = 0.f;
    }
  }
  const long t0 = ((long)blockIdx.x * 4 + wave) * RG;
  u32x4 kv[RG][NCH];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const long t = t0 + r < rows ? t0 + r : rows - 1;
    const bf16_t* kr = klist + ((size_t)b * rows + t) * f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane * 8 + 512 * i;
      kv[r][i] = c < f ? ld16(kr + c) : u32x4{0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = __builtin_fmaf(__uint_as_float(kv[r][i][e] << 16), zr[i][2 * e], acc);
        acc = __builtin_fmaf(__uint_as_float(kv[r][i][e] & 0xFFFF0000u), zr[i][2 * e + 1], acc);
      }
    acc = wave_sum(acc);
    const long t = t0 + r;
    if (lane == 0 && t < rows) cbuf[(size_t)b * rows + t] = acc * beta[(size_t)b * n + t / chunk];
  }
}

__global__ void __launch_bounds__(256)
list_raccum_v(const bf16_t* __restrict__ rlist, const float* __restrict__ cbuf,
              float* __restrict__ ypart, int rows, int d) {
  __shared__ float cs[SEG];
  __shared__ float red[256 * 8];
  const int seg = blockIdx.x, b = blockIdx.y;
  const long t0 = (long)seg * SEG;
  for (int i = threadIdx.x; i < SEG; i += 256) {
    const long t = t0 + i;
    cs[i] = t < rows ? cbuf[(size_t)b * rows + t] : 0.f;
  }
  __syncthreads();
  const int nseg = gridDim.x;
  const int CH = d / 8;                              // 8-feature chunks (d % 8 == 0)
  const int CHP = CH < 256 ? CH : 256;               // threads per row group
  const int NRG = 256 / CHP;                         // row groups
  const int fc = threadIdx.x % CHP, rg = threadIdx.x / CHP;
  const int tend = (int)min((long)SEG, rows - t0);
  const int niter = (CH + CHP - 1) / CHP;            // the same for every thread (barriers)
  for (int it = 0; it < niter; ++it) {
    const int c0 = fc + it * CHP;
    const bool cok = c0 < CH;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    if (rg < NRG && cok) {
      const bf16_t* rb = rlist + ((size_t)b * rows + t0) * d + 8 * c0;
      int i = rg;
      for (; i + 7 * NRG < tend; i += 8 * NRG) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = ld16(rb + (size_t)(i + u * NRG) * d);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float cv = cs[i + u * NRG];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * e] = __builtin_fmaf(cv, __uint_as_float(v[u][e] << 16), acc[2 * e]);
            acc[2 * e + 1] = __builtin_fmaf(cv, __uint_as_float(v[u][e] & 0xFFFF0000u), acc[2 * e + 1]);
          }
        }
      }
      for (; i < tend; i += NRG) {
        const u32x4 v = ld16(rb + (size_t)i * d);
        const float cv = cs[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] = __builtin_fmaf(cv, __uint_as_float(v[e] << 16), acc[2 * e]);
          acc[2 * e + 1] = __builtin_fmaf(cv, __uint_as_float(v[e] & 0xFFFF0000u), acc[2 * e + 1]);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) red[threadIdx.x * 8 + e] = acc[e];
    __syncthreads();
    if (rg == 0 && cok) {
      for (int g2 = 1; g2 < NRG; ++g2)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += red[(g2 * CHP + fc) * 8 + e];
#pragma unroll
      for (int e = 0; e < 8; ++e) ypart[((size_t)b * nseg + seg) * d + 8 * c0 + e] = acc[e];
    }
  }
}

__global__ void __launch_bounds__(256)
list_reduce(const float* __restrict__ ypart, float* __restrict__ y, int nseg, int d) {
  const int b = blockIdx.y;
  const int a = blockIdx.x * 256 + threadIdx.x;
  if (a >= d) return;
  float acc = 0.f;
  for (int s = 0; s < nseg; ++s) acc += ypart[((size_t)b * nseg + s) * d + a];
  y[(size_t)b * d + a] += acc;
}

template <typename T>
__global__ void __launch_bounds__(256)
dense_apply(const float* __restrict__ S, const T* __restrict__ z, float* __restrict__ y, int d,
            int f, int accumulate) {
  extern __shared__ float zs[];
  const int b = blockIdx.y;
  for (int i = threadIdx.x; i < f; i += 256) zs[i] = ldf(z + (size_t)b * f + i);
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long a = (long)blockIdx.x * 4 + wave;
  if (a >= d) return;
  const float* sr = S + ((size_t)b * d + a) * f;
  float acc = 0.f;
  // four 16-byte reads of the row in flight per lane before they are used
  for (int c0 = lane * 4; c0 < f; c0 += 1024) {
    f32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + 256 * u;
      v[u] = c < f ? *reinterpret_cast<const f32x4*>(sr + c) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + 256 * u;
      if (c < f) acc += v[u][0] * zs[c] + v[u][1] * zs[c + 1] + v[u][2] * zs[c + 2] + v[u][3] * zs[c + 3];
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) {
    float* yp = y + (size_t)b * d + a;
    *yp = accumulate ? *yp + acc : acc;
  }
}

}  // namespace

void decode_attn_plan(int wT, int* nsplit, int* split_len) {
  int sl = 512;
  if (wT <= 2048) sl = 128;
  *split_len = sl;
  *nsplit = (wT + sl - 1) / sl;
}

// Splits that hold at least one key of query position pos: the window
// [max(0, pos - wT + 1), pos] has min(wT, pos + 1) keys.
int decode_attn_splits_used(int wT, int pos, int split_len) {
  const int keys = wT < pos + 1 ? wT : pos + 1;
  return (keys + split_len - 1) / split_len;
}

size_t decode_attn_part_bytes(int B, int Hq, int D, int nsplit) {
  return (size_t)B * Hq * nsplit * 2 * (D + 2) * sizeof(float);
}

template <typename T, int D>
void launch_split_g(const DecodeAttnArgs& a, int G, dim3 grid, float c, int ns, hipStream_t s) {
#define TTCD_SPLIT(GG)                                                                          \
  hipLaunchKernelGGL((decode_attn_split<T, D, GG>), grid, dim3(256), 0, s, (const T*)a.q,       \
                     (const T*)a.k, (const T*)a.v, a.part, a.pos, a.kv_rows, a.Hq, a.Hkv, a.wT, \
                     a.wS, c, ns, a.split_len)
  switch (G) {
    case 1: TTCD_SPLIT(1); break;
    case 2: TTCD_SPLIT(2); break;
    case 3: TTCD_SPLIT(3); break;
    default: TTCD_SPLIT(4); break;
  }
#undef TTCD_SPLIT
}

hipError_t launch_decode_attn(const DecodeAttnArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  if (G > GMAX) return hipErrorInvalidValue;
  const float c = a.scale * 1.4426950408889634f;
  // only the splits that hold keys (at most a.nsplit, the planned count)
  const int ns = decode_attn_splits_used(a.wT, a.pos, a.split_len);
  if (ns < 1 || ns > a.nsplit) return hipErrorInvalidValue;
  dim3 grid(ns, a.Hkv, a.B);
  if (a.in_dt == BF16) {
    if (a.D == 64)
      launch_split_g<bf16_t, 64>(a, G, grid, c, ns, s);
    else
      launch_split_g<bf16_t, 128>(a, G, grid, c, ns, s);
  } else {
    if (a.D == 64)
      launch_split_g<float, 64>(a, G, grid, c, ns, s);
    else
      launch_split_g<float, 128>(a, G, grid, c, ns, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(a.B * a.Hq);
  if (a.out_dt == BF16)
    hipLaunchKernelGGL(decode_attn_combine<bf16_t>, g2, dim3(128), 0, s, a.part,
                       (bf16_t*)a.o_t, (bf16_t*)a.o_s, a.lse_t, a.lse_s, a.Hq, a.D, ns);
  else
    hipLaunchKernelGGL(decode_attn_combine<float>, g2, dim3(128), 0, s, a.part, (float*)a.o_t,
                       (float*)a.o_s, a.lse_t, a.lse_s, a.Hq, a.D, ns);
  return hipGetLastError();
}

hipError_t launch_list_apply(const ListApplyArgs& a, hipStream_t s) {
  const int rows = a.n * a.chunk;
  if (rows <= 0) return hipSuccess;
  dim3 g1((rows + 15) / 16, a.B);
  const size_t zl = (size_t)a.f * sizeof(float);
  const int nseg = (rows + SEG - 1) / SEG;
  float* ypart = a.cbuf + (size_t)a.B * rows;
  const int nch = (a.f + 511) / 512;
  if (a.in_dt == BF16 && nch <= 8) {
    dim3 gk((rows + 15) / 16, a.B);               // 4 waves x 4 rows per workgroup
    switch (nch) {
#define TTCD_KDOT(N)                                                                          \
  case N:                                                                                     \
    hipLaunchKernelGGL(list_kdot_reg<N>, gk, dim3(256), 0, s, (const bf16_t*)a.k_list,        \
                       (const bf16_t*)a.z, a.beta, a.cbuf, rows, a.f, a.chunk, a.n);          \
    break;
      TTCD_KDOT(1) TTCD_KDOT(2) TTCD_KDOT(3) TTCD_KDOT(4)
      TTCD_KDOT(5) TTCD_KDOT(6) TTCD_KDOT(7) TTCD_KDOT(8)
#undef TTCD_KDOT
    }
    hipLaunchKernelGGL(list_raccum_v, dim3(nseg, a.B), dim3(256), 0, s, (const bf16_t*)a.r_list,
                       a.cbuf, ypart, rows, a.d);
  } else if (a.in_dt == BF16) {
    hipLaunchKernelGGL(list_kdot<bf16_t>, g1, dim3(256), zl, s, (const bf16_t*)a.k_list,
                       (const bf16_t*)a.z, a.beta, a.cbuf, rows, a.f, a.chunk, a.n);
    hipLaunchKernelGGL(list_raccum_v, dim3(nseg, a.B), dim3(256), 0, s, (const bf16_t*)a.r_list,
                       a.cbuf, ypart, rows, a.d);
  } else {
    hipLaunchKernelGGL(list_kdot<float>, g1, dim3(256), zl, s, (const float*)a.k_list,
                       (const float*)a.z, a.beta, a.cbuf, rows, a.f, a.chunk, a.n);
    hipLaunchKernelGGL(list_raccum<float>, dim3(nseg, a.B), dim3(256), 0, s,
                       (const float*)a.r_list, a.cbuf, ypart, rows, a.d);
  }
  hipLaunchKernelGGL(list_reduce, dim3((a.d + 255) / 256, a.B), dim3(256), 0, s, ypart, a.y, nseg,
                     a.d);
  return hipGetLastError();
}

hipError_t launch_dense_apply(const float* S, const void* z, float* y, int B, int d, int f,
                              int in_dt, int accumulate, hipStream_t s) {
  dim3 grid((d + 3) / 4, B);
  const size_t zl = (size_t)f * sizeof(float);
  if (in_dt == BF16)
    hipLaunchKernelGGL(dense_apply<bf16_t>, grid, dim3(256), zl, s, S, (const bf16_t*)z, y, d, f,
                       accumulate);
  else
    hipLaunchKernelGGL(dense_apply<float>, grid, dim3(256), zl, s, S, (const float*)z, y, d, f,
                       accumulate);
  return hipGetLastError();
}

}  // namespace ttcd
