// Dual-window causal sliding-window attention for gfx950.
//
// What is computed (papernotes.org notes on "Learning What to Remember",
// overall framework; podcast transcript, sliding-window cue): for the query
// at position t, the teacher attends to keys j with 0 <= t-j < w_T and the
// student to keys with 0 <= t-j < w_S, over one shared Q/K/V.  The README's
// "Fused inference kernels" section describes producing both in one pass
// over K/V; the LSE-combination variant merges a student-window result and
// a far-band result exactly through their log-sum-exp.
//
// Design here (CDNA4, bf16 MFMA 32x32x16):
//   * S^T = K Q^T and O^T = V^T P^T, so each lane owns ONE query (a column
//     of the MFMA output) and every softmax reduction over keys is in-lane
//     plus one swap between the two lane halves.
//   * One workgroup = 4 waves x 32 query rows of one (batch, kv head); the
//     rows are (position, q head) pairs of that kv group, so GQA heads share
//     every K/V tile staged in LDS.
//   * Two online-softmax states per row: the student band [t-w_S+1, t] and
//     the far band [t-w_T+1, t-w_S].  Each score belongs to exactly one of
//     them.  Tiles are walked newest to oldest; tiles outside a wave's
//     bands are skipped; masking only happens on edge sub-blocks.  The
//     teacher result is the exact LSE merge of the two states, and equals
//     the student result bit for bit when the far band is empty.
//   * Lazy rescaling: a state's running max only moves when a new score
//     exceeds it by more than 2^8, which keeps the fp32 accumulators exact
//     in value while skipping most rescales.
#include "common.hpp"
#include "kernels.hpp"

namespace ttcd {

namespace {

constexpr int BN = 64;          // keys per LDS tile
constexpr float TAU = 8.0f;     // lazy-rescale threshold (log2 domain)
constexpr float NEG_INF = -__builtin_inff();

template <int D, int NW>
struct AttnLds {
  static constexpr int KS = D + 8;     // K row stride (bf16)
  static constexpr int VS = BN + 4;    // V^T row stride (bf16)
  static constexpr int K_ELEMS = BN * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int BUF = K_ELEMS + V_ELEMS;
  static constexpr size_t BYTES = 2 * BUF * sizeof(bf16_t);
};

struct SoftState {
  float m;   // running max (log2 domain, scaled)
  float l;   // this lane's partial denominator
};

// One 32-key sub-block update of a state.  s: the 16 raw scores of this
// lane (MFMA output layout), msk: which of them belong to this state.
template <int NB, bool MASKED>
TTCD_DEV void state_update(SoftState& st, f32x16* acc, const f32x16& s, uint32_t msk,
                           float c, bf16x8& p0, bf16x8& p1) {
  float mx = NEG_INF;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float x = s[v] * c;
    if (MASKED) x = ((msk >> v) & 1u) ? x : NEG_INF;
    mx = fmaxf(mx, x);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const bool need = mx > st.m + TAU;
  if (__builtin_expect(__any(need), 0)) {
    const float mnew = need ? mx : st.m;
    const float alpha = (st.m == NEG_INF) ? 0.f : fast_exp2(st.m - mnew);
    st.l *= alpha;
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] *= alpha;
    st.m = mnew;
  }
  const float negm = -st.m;
  float p[16];
  float lsum = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float e = fast_exp2(__builtin_fmaf(s[v], c, negm));
    if (MASKED) e = ((msk >> v) & 1u) ? e : 0.f;
    p[v] = e;
    lsum += e;
  }
  st.l += lsum;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p0[j] = (__bf16)p[j];
    p1[j] = (__bf16)p[8 + j];
  }
}

template <int NB>
TTCD_DEV void pv_update(f32x16* acc, const bf16_t* vt_lds, int vs, int sb, int lane,
                        const bf16x8& p0, const bf16x8& p1) {
  const int h = lane >> 5;
  const int r = lane & 31;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const bf16_t* row = vt_lds + (32 * b + r) * vs + 32 * sb + 4 * h;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      u32x2 lo = *reinterpret_cast<const u32x2*>(row + 16 * m);
      u32x2 hi = *reinterpret_cast<const u32x2*>(row + 16 * m + 8);
      u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
      acc[b] = mfma32(as_bf16x8(w), m == 0 ? p0 : p1, acc[b]);
    }
  }
}

template <int D, int NW>
__global__ void __launch_bounds__(64 * NW, (D == 128 ? 1 : 2))
dual_window_attn_mfma(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                      const bf16_t* __restrict__ vt, int vt_ld,
                      void* __restrict__ o_t, void* __restrict__ o_s,
                      float* __restrict__ lse_t, float* __restrict__ lse_s,
                      int B, int Tq, int Tk, int kv_rows, int q_pos0, int Hq, int Hkv,
                      int wT, int wS, float c, int out_bf16, int nblk) {
  using L = AttnLds<D, NW>;
  constexpr int NB = D / 32;      // 32-wide d blocks of O^T
  constexpr int KSTEP = D / 16;   // k-steps of S^T
  constexpr int ROWS = 32 * NW;
  extern __shared__ __align__(16) bf16_t lds[];

  const int G = Hq / Hkv;
  const int R = Tq * G;
  const uint32_t total = (uint32_t)B * Hkv * nblk;
  const uint32_t lid = xcd_remap(blockIdx.x, total);
  const int blk = lid % nblk;
  const int bg = lid / nblk;
  const int g = bg % Hkv;
  const int b = bg / Hkv;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int h = lane >> 5;

  // ---- this lane's query row
  const int row0 = blk * ROWS;
  const int rw0 = row0 + 32 * wave;
  int r = rw0 + (lane & 31);
  const bool row_ok = r < R;
  r = row_ok ? r : R - 1;
  const int qi = r / G;
  const int qh = g * G + (r % G);
  const int t = q_pos0 + qi;

  // wave / workgroup position ranges
  const int wr_hi = min(rw0 + 31, R - 1);
  const int a_w = q_pos0 + min(rw0, R - 1) / G;
  const int b_w = q_pos0 + wr_hi / G;
  const int A = q_pos0 + row0 / G;
  const int Bp = q_pos0 + min(row0 + ROWS - 1, R - 1) / G;
  const int jlo = max(0, A - wT + 1);
  const int jhi = min(Bp, Tk - 1);

  // ---- Q fragments (B operand of S^T = K Q^T)
  bf16x8 qf[KSTEP];
  {
    const bf16_t* qp = q + ((size_t)(b * Tq + qi) * Hq + qh) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < KSTEP; ++s) qf[s] = as_bf16x8(ld16(qp + 16 * s));
  }

  f32x16 accS[NB], accF[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    accS[i] = zero16();
    accF[i] = zero16();
  }
  SoftState stS = {NEG_INF, 0.f}, stF = {NEG_INF, 0.f};

  // ---- tile loaders (registers -> LDS, double buffered)
  constexpr int KCH = BN * D / 8 / (64 * NW);   // 16B chunks per thread (K)
  constexpr int VCH = D * BN / 8 / (64 * NW);   // 16B chunks per thread (V^T)
  static_assert(KCH >= 1 && VCH >= 1, "tile too small for the workgroup");
  u32x4 kreg[KCH], vreg[VCH];
  const bf16_t* kbase = k + ((size_t)b * kv_rows * Hkv + g) * D;
  const size_t kstride = (size_t)Hkv * D;
  const bf16_t* vbase = vt + (size_t)(b * Hkv + g) * D * vt_ld;

  auto load_regs = [&](int n) {
    const int j0 = n * BN;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int cidx = tid + i * 64 * NW;
      const int key = cidx / (D / 8), dc = cidx % (D / 8);
      const int j = j0 + key;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (j >= jlo && j <= jhi) val = ld16(kbase + (size_t)j * kstride + dc * 8);
      kreg[i] = val;
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int cidx = tid + i * 64 * NW;
      const int d = cidx / (BN / 8), kc = cidx % (BN / 8);
      const int j = j0 + kc * 8;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (j + 7 >= jlo && j <= jhi) {
        val = ld16(vbase + (size_t)d * vt_ld + j);
        if (j < jlo || j + 7 > jhi) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int ja = j + 2 * e, jb = ja + 1;
            uint32_t w = val[e];
            if (ja < jlo || ja > jhi) w &= 0xFFFF0000u;
            if (jb < jlo || jb > jhi) w &= 0x0000FFFFu;
            val[e] = w;
          }
        }
      }
      vreg[i] = val;
    }
  };
  auto store_lds = [&](int buf) {
    bf16_t* kl = lds + buf * L::BUF;
    bf16_t* vl = kl + L::K_ELEMS;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int cidx = tid + i * 64 * NW;
      const int key = cidx / (D / 8), dc = cidx % (D / 8);
      st16(kl + key * L::KS + dc * 8, kreg[i]);
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int cidx = tid + i * 64 * NW;
      const int d = cidx / (BN / 8), kc = cidx % (BN / 8);
      u32x2* p = reinterpret_cast<u32x2*>(vl + d * L::VS + kc * 8);
      p[0] = u32x2{vreg[i][0], vreg[i][1]};
      p[1] = u32x2{vreg[i][2], vreg[i][3]};
    }
  };

  const int n_hi = jhi / BN, n_lo = jlo / BN;
  load_regs(n_hi);
  store_lds(0);
  __syncthreads();

  int it = 0;
  for (int n = n_hi; n >= n_lo; --n, ++it) {
    const int cur = it & 1;
    const bool has_next = n > n_lo;
    if (has_next) load_regs(n - 1);

    const bf16_t* kl = lds + cur * L::BUF;
    const bf16_t* vl = kl + L::K_ELEMS;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int j0 = n * BN + 32 * sb;
      const int j1 = j0 + 31;
      // wave-uniform classification of this 32-key sub-block
      if (j0 > b_w || j1 < a_w - wT + 1) continue;
      const bool anyS = (j0 <= b_w) && (j1 >= a_w - wS + 1);
      const bool anyF = (a_w - j1 <= wT - 1) && (b_w - j0 >= wS);
      const bool allS = (a_w - j1 >= 0) && (b_w - j0 <= wS - 1);
      const bool allF = (a_w - j1 >= wS) && (b_w - j0 <= wT - 1);

      f32x16 s = zero16();
      const bf16_t* krow = kl + (32 * sb + (lane & 31)) * L::KS + 8 * h;
#pragma unroll
      for (int ks = 0; ks < KSTEP; ++ks) s = mfma32(as_bf16x8(ld16(krow + 16 * ks)), qf[ks], s);

      bf16x8 p0, p1;
      if (allS) {
        state_update<NB, false>(stS, accS, s, 0xFFFFu, c, p0, p1);
        pv_update<NB>(accS, vl, L::VS, sb, lane, p0, p1);
      } else if (allF) {
        state_update<NB, false>(stF, accF, s, 0xFFFFu, c, p0, p1);
        pv_update<NB>(accF, vl, L::VS, sb, lane, p0, p1);
      } else {
        uint32_t mS = 0u, mF = 0u;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = j0 + 8 * (v >> 2) + 4 * h + (v & 3);
          const int dlt = t - j;
          if (dlt >= 0 && dlt < wS) mS |= 1u << v;
          if (dlt >= wS && dlt < wT) mF |= 1u << v;
        }
        if (anyS) {
          state_update<NB, true>(stS, accS, s, mS, c, p0, p1);
          pv_update<NB>(accS, vl, L::VS, sb, lane, p0, p1);
        }
        if (anyF) {
          state_update<NB, true>(stF, accF, s, mF, c, p0, p1);
          pv_update<NB>(accF, vl, L::VS, sb, lane, p0, p1);
        }
      }
    }

    if (has_next) store_lds(cur ^ 1);
    __syncthreads();
  }

  // ---- merge and store
  const float lS = stS.l + __shfl_xor(stS.l, 32, 64);
  const float lF = stF.l + __shfl_xor(stF.l, 32, 64);
  const float mT = fmaxf(stS.m, stF.m);
  const float aS = (stS.m == NEG_INF) ? 0.f : fast_exp2(stS.m - mT);
  const float aF = (stF.m == NEG_INF) ? 0.f : fast_exp2(stF.m - mT);
  const float lT = lS * aS + lF * aF;
  const bool far_empty = (lF == 0.f);
  const float invS = 1.f / lS;
  const float invT = 1.f / lT;
  constexpr float LN2 = 0.69314718055994530942f;

  if (row_ok) {
    const size_t obase = ((size_t)(b * Tq + qi) * Hq + qh) * D;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * bb + 8 * g4 + 4 * h;
        float os[4], ot[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float vs = accS[bb][4 * g4 + e];
          os[e] = vs * invS;
          ot[e] = far_empty ? os[e] : (vs * aS + accF[bb][4 * g4 + e] * aF) * invT;
        }
        if (out_bf16) {
          u32x2 ws = {pack_bf16x2(os[0], os[1]), pack_bf16x2(os[2], os[3])};
          u32x2 wt = {pack_bf16x2(ot[0], ot[1]), pack_bf16x2(ot[2], ot[3])};
          *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(o_s) + obase + d) = ws;
          *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(o_t) + obase + d) = wt;
        } else {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(o_s) + obase + d) =
              f32x4{os[0], os[1], os[2], os[3]};
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(o_t) + obase + d) =
              f32x4{ot[0], ot[1], ot[2], ot[3]};
        }
      }
    }
    if (h == 0) {
      const size_t li = (size_t)(b * Hq + qh) * Tq + qi;
      const float lseS = (stS.m + fast_log2(lS)) * LN2;
      if (lse_s) lse_s[li] = lseS;
      if (lse_t) lse_t[li] = far_empty ? lseS : (mT + fast_log2(lT)) * LN2;
    }
  }
}

// --------------------------------------------------------------------------
// Plain fp32 (or bf16-input) reference-grade kernel: one thread per query
// row, exact per-key online softmax, two states.  Used for fp32 inputs and
// head dims the MFMA kernel does not cover.
// --------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(64)
dual_window_attn_simple(const T* __restrict__ q, const T* __restrict__ k,
                        const T* __restrict__ v, void* __restrict__ o_t,
                        void* __restrict__ o_s, float* __restrict__ lse_t,
                        float* __restrict__ lse_s, int B, int Tq, int Tk, int kv_rows,
                        int q_pos0, int Hq, int Hkv, int wT, int wS, float scale,
                        int out_bf16, int nblk) {
  constexpr int TK = 32;
  __shared__ float ks[TK][D + 1];
  __shared__ float vs[TK][D + 1];
  const int G = Hq / Hkv;
  const int R = Tq * G;
  const int blk = blockIdx.x % nblk;
  const int bg = blockIdx.x / nblk;
  const int g = bg % Hkv, b = bg / Hkv;
  const int tid = threadIdx.x;
  int r = blk * 64 + tid;
  const bool row_ok = r < R;
  r = row_ok ? r : R - 1;
  const int qi = r / G, qh = g * G + r % G;
  const int t = q_pos0 + qi;
  const int A = q_pos0 + (blk * 64) / G;
  const int Bp = q_pos0 + min(blk * 64 + 63, R - 1) / G;
  const int jlo = max(0, A - wT + 1), jhi = min(Bp, Tk - 1);

  float qv[D];
  const T* qp = q + ((size_t)(b * Tq + qi) * Hq + qh) * D;
  for (int d = 0; d < D; ++d) qv[d] = ldf(qp + d) * scale;
  float aS[D], aF[D];
  for (int d = 0; d < D; ++d) aS[d] = aF[d] = 0.f;
  float mS = NEG_INF, lS = 0.f, mF = NEG_INF, lF = 0.f;

  for (int j0 = jhi; j0 >= jlo; j0 -= TK) {
    __syncthreads();
    for (int e = tid; e < TK * D; e += 64) {
      const int jj = e / D, d = e % D;
      const int j = j0 - jj;
      float kv = 0.f, vv = 0.f;
      if (j >= jlo) {
        const size_t off = ((size_t)(b * kv_rows + j) * Hkv + g) * D + d;
        kv = ldf(k + off);
        vv = ldf(v + off);
      }
      ks[jj][d] = kv;
      vs[jj][d] = vv;
    }
    __syncthreads();
    for (int jj = 0; jj < TK; ++jj) {
      const int j = j0 - jj;
      if (j < jlo) break;
      const int dlt = t - j;
      const bool inS = dlt >= 0 && dlt < wS;
      const bool inF = dlt >= wS && dlt < wT;
      if (!inS && !inF) continue;
      float s = 0.f;
      for (int d = 0; d < D; ++d) s = __builtin_fmaf(qv[d], ks[jj][d], s);
      if (inS) {
        const float mn = fmaxf(mS, s);
        const float al = (mS == NEG_INF) ? 0.f : expf(mS - mn);
        const float p = expf(s - mn);
        for (int d = 0; d < D; ++d) aS[d] = aS[d] * al + p * vs[jj][d];
        lS = lS * al + p;
        mS = mn;
      } else {
        const float mn = fmaxf(mF, s);
        const float al = (mF == NEG_INF) ? 0.f : expf(mF - mn);
        const float p = expf(s - mn);
        for (int d = 0; d < D; ++d) aF[d] = aF[d] * al + p * vs[jj][d];
        lF = lF * al + p;
        mF = mn;
      }
    }
  }
  if (!row_ok) return;
  const float mT = fmaxf(mS, mF);
  const float eS = (mS == NEG_INF) ? 0.f : expf(mS - mT);
  const float eF = (mF == NEG_INF) ? 0.f : expf(mF - mT);
  const float lT = lS * eS + lF * eF;
  const bool far_empty = lF == 0.f;
  const size_t obase = ((size_t)(b * Tq + qi) * Hq + qh) * D;
  for (int d = 0; d < D; ++d) {
    const float os = aS[d] / lS;
    const float ot = far_empty ? os : (aS[d] * eS + aF[d] * eF) / lT;
    if (out_bf16) {
      reinterpret_cast<bf16_t*>(o_s)[obase + d] = f2bf(os);
      reinterpret_cast<bf16_t*>(o_t)[obase + d] = f2bf(ot);
    } else {
      reinterpret_cast<float*>(o_s)[obase + d] = os;
      reinterpret_cast<float*>(o_t)[obase + d] = ot;
    }
  }
  const size_t li = (size_t)(b * Hq + qh) * Tq + qi;
  const float lseS = mS + logf(lS);
  if (lse_s) lse_s[li] = lseS;
  if (lse_t) lse_t[li] = far_empty ? lseS : mT + logf(lT);
}

template <int D>
hipError_t launch_mfma(const AttnArgs& a, hipStream_t s) {
  constexpr int NW = 4;
  using L = AttnLds<D, NW>;
  const int G = a.Hq / a.Hkv;
  const int R = a.Tq * G;
  const int nblk = (R + 32 * NW - 1) / (32 * NW);
  const long total = (long)a.B * a.Hkv * nblk;
  const float c = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((dual_window_attn_mfma<D, NW>), dim3((unsigned)total), dim3(64 * NW),
                     L::BYTES, s, (const bf16_t*)a.q, (const bf16_t*)a.k,
                     (const bf16_t*)a.vt, a.vt_ld, a.o_t, a.o_s, a.lse_t, a.lse_s, a.B, a.Tq,
                     a.Tk, a.kv_rows, a.q_pos0, a.Hq, a.Hkv, a.wT, a.wS, c,
                     a.out_dt == BF16 ? 1 : 0, nblk);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_simple(const AttnArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int R = a.Tq * G;
  const int nblk = (R + 63) / 64;
  const long total = (long)a.B * a.Hkv * nblk;
  hipLaunchKernelGGL((dual_window_attn_simple<T, D>), dim3((unsigned)total), dim3(64), 0, s,
                     (const T*)a.q, (const T*)a.k, (const T*)a.v, a.o_t, a.o_s, a.lse_t,
                     a.lse_s, a.B, a.Tq, a.Tk, a.kv_rows, a.q_pos0, a.Hq, a.Hkv, a.wT, a.wS,
                     a.scale, a.out_dt == BF16 ? 1 : 0, nblk);
  return hipGetLastError();
}

}  // namespace

size_t attn_vt_bytes(int B, int Hkv, int D, int Tk, int in_dt) {
  if (in_dt != BF16) return 0;
  const size_t ld = ((size_t)Tk + 63) / 64 * 64;
  return (size_t)B * Hkv * D * ld * 2;
}

hipError_t launch_dual_window_attn(const AttnArgs& a, hipStream_t s) {
  if (a.in_dt == BF16 && (a.D == 64 || a.D == 128)) {
    static bool attr_set = false;
    if (!attr_set) {
      (void)hipFuncSetAttribute((const void*)dual_window_attn_mfma<64, 4>,
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)AttnLds<64, 4>::BYTES);
      (void)hipFuncSetAttribute((const void*)dual_window_attn_mfma<128, 4>,
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)AttnLds<128, 4>::BYTES);
      attr_set = true;
    }
    hipError_t e = launch_v_transpose(a.v, a.vt, a.B, a.Tk, a.kv_rows, a.Hkv, a.D, a.vt_ld, 2, s);
    if (e != hipSuccess) return e;
    return a.D == 64 ? launch_mfma<64>(a, s) : launch_mfma<128>(a, s);
  }
  if (a.in_dt == F32) {
    if (a.D == 64) return launch_simple<float, 64>(a, s);
    if (a.D == 128) return launch_simple<float, 128>(a, s);
  } else {
    if (a.D == 64) return launch_simple<bf16_t, 64>(a, s);
    if (a.D == 128) return launch_simple<bf16_t, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ttcd
