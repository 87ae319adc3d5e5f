// Dual-window causal sliding-window attention for gfx950.
//
// What is computed (papernotes.org notes on "Learning What to Remember",
// overall framework; podcast transcript, sliding-window cue): for the query
// at position t, the teacher attends to keys j with 0 <= t-j < w_T and the
// student to keys with 0 <= t-j < w_S, over one shared Q/K/V.  The README's
// "Fused inference kernels" section describes producing both in one pass
// over K/V with the student recovered through the online-softmax rescaling.
//
// Design here (CDNA4, bf16 MFMA 32x32x16, fp32 accumulate):
//   * S^T = K Q^T and O^T = V^T P^T, so each lane owns ONE query (a column
//     of the MFMA output) and every softmax reduction over keys is in-lane
//     plus one swap between the two lane halves.
//   * One workgroup = 8 waves x 32 query rows of one (batch, kv head); the
//     rows are (position, q head) pairs of that kv group, so all GQA heads
//     share every K/V tile staged in LDS.
//   * K/V tiles of 64 keys go straight from global memory into LDS
//     (global_load_lds_dwordx4) in a 3-deep ring, XOR-swizzled so that the
//     MFMA operand reads are free of bank conflicts.  V arrives
//     pre-transposed (d-major) with the keys of every 16-key group permuted
//     so that one 16-byte LDS read yields the 8 keys an MFMA lane needs.
//   * ONE online-softmax state per row, walked newest to oldest: first the
//     student band (masked only on edge sub-blocks); when a wave passes its
//     oldest student sub-block the student output is written, the far-band
//     part of the (at most two) edge sub-blocks is added -- they are still
//     in the LDS ring -- and the walk continues through the far band to the
//     teacher output.  Tiles outside a wave's bands are skipped.  Rows whose
//     far band is empty finish with bit-identical teacher and student
//     results.
//   * Lazy rescaling: the running max only moves when a new score exceeds
//     it by more than 2^8; the result is unchanged up to rounding.
#include "common.hpp"
#include "kernels.hpp"

namespace ttcd {

namespace {

constexpr int BN = 64;          // keys per LDS tile
constexpr int NBUF = 4;         // LDS ring depth: current, previous, two in flight
constexpr float TAU = 8.0f;     // lazy-rescale threshold (log2 domain)
constexpr float NEG_INF = -__builtin_inff();
constexpr float LN2 = 0.69314718055994530942f;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// 16 bytes per lane, global -> LDS; lane i lands at lds_wave_base + 16 i.
TTCD_DEV void g2l16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)lds_wave_base, 16, 0, 0);
}

// Workgroup barrier that does not drain this wave's in-flight tile fetches
// (a fenced barrier would wait for every outstanding memory operation).  LDS
// ordering: every wave waits for the tile it needs with wait_vm first, and
// all LDS reads of a buffer are consumed by MFMAs before the barrier that
// precedes the fetch overwriting it.
TTCD_DEV void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
TTCD_DEV void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int D>
struct Tile {
  static constexpr int CPR = D / 8;                 // 16B chunks per K row
  static constexpr int KPOS = BN * CPR;             // 16B positions, K region
  static constexpr int VPOS = D * (BN / 8);         // 16B positions, V^T region
  static constexpr int BYTES = (KPOS + VPOS) * 16;
  static TTCD_DEV int kswz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
  static TTCD_DEV int vswz(int d) { return (d >> 1) & 7; }
};

struct SoftState {
  float m;   // running max (log2 domain, scaled)
  float l;   // this lane's partial denominator
};

template <int D, int NW>
TTCD_DEV void issue_tile(char* buf, const bf16_t* kbase, size_t kstride, const bf16_t* vbase,
                         int vt_ld, int j0, int jlo, int jhi, int wave, int lane) {
  using TL = Tile<D>;
  static_assert(TL::KPOS % (64 * NW) == 0 && TL::VPOS % (64 * NW) == 0, "tile/wave split");
#pragma unroll
  for (int i = 0; i < TL::KPOS / (64 * NW); ++i) {
    const int p0 = (i * NW + wave) * 64;
    const int p = p0 + lane;
    const int row = p / TL::CPR, cp = p % TL::CPR;
    const int c = cp ^ TL::kswz(row);
    const int j = min(max(j0 + row, jlo), jhi);   // never read outside the band
    g2l16(kbase + (size_t)j * kstride + c * 8, buf + p0 * 16);
  }
  char* vb = buf + TL::KPOS * 16;
#pragma unroll
  for (int i = 0; i < TL::VPOS / (64 * NW); ++i) {
    const int p0 = (i * NW + wave) * 64;
    const int p = p0 + lane;
    const int d = p >> 3, cp = p & 7;
    const int c = cp ^ TL::vswz(d);
    g2l16(vbase + (size_t)d * vt_ld + j0 + 8 * c, vb + p0 * 16);
  }
}

// One 32-key sub-block: S^T = K Q^T, online-softmax update, O^T += V^T P^T.
// Operand fragments are read from LDS in groups ahead of their MFMAs so that
// one LDS latency covers eight MFMAs, and the V^T fragments are in flight
// while the softmax runs.  masked (wave-uniform): only keys with
// lo <= t - j < hi take part.
template <int D>
TTCD_DEV void process(const char* buf, int sb, int j0, int t, bool masked, int lo, int hi,
                      float c, const bf16x8* qf, SoftState& st, f32x16* acc, int lane) {
  using TL = Tile<D>;
  constexpr int NB = D / 32;
  constexpr int KSTEP = D / 16;
  const int h = lane >> 5, r = lane & 31;

  bf16x8 kf[KSTEP];
  {
    const int row = 32 * sb + r;
    const char* krow = buf + row * (TL::CPR * 16);
    const int sw = TL::kswz(row);
#pragma unroll
    for (int ks = 0; ks < KSTEP; ++ks) kf[ks] = as_bf16x8(ld16(krow + (((2 * ks + h) ^ sw) << 4)));
  }
  __builtin_amdgcn_sched_barrier(0);
  f32x16 s = zero16();
#pragma unroll
  for (int ks = 0; ks < KSTEP; ++ks) s = mfma32(kf[ks], qf[ks], s);

  bf16x8 vf[NB][2];
  {
    const char* vb = buf + TL::KPOS * 16;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int d = 32 * b + r;
      const char* vrow = vb + d * (BN * 2);
      const int sw = TL::vswz(d);
      vf[b][0] = as_bf16x8(ld16(vrow + (((4 * sb + 0 + h) ^ sw) << 4)));
      vf[b][1] = as_bf16x8(ld16(vrow + (((4 * sb + 2 + h) ^ sw) << 4)));
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  if (masked) {
    // lo <= t - j < hi  <=>  (unsigned)(t - j - lo) < (unsigned)(hi - lo)
    const uint32_t d0 = (uint32_t)(t - j0 - 4 * h - lo), span = (uint32_t)(hi - lo);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const uint32_t dl = d0 - (uint32_t)(8 * (v >> 2) + (v & 3));
      s[v] = dl < span ? s[v] : NEG_INF;
    }
  }
  // row max over the 32 keys (raw scores; c > 0): in-lane, then swap halves
  float mx = NEG_INF;
#pragma unroll
  for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[v]);
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                     false, false);
    mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c;
  }
  const bool need = mx > st.m + TAU;
  if (__builtin_expect(__any(need), 0)) {
    const float mnew = need ? mx : st.m;
    const float alpha = (st.m == NEG_INF) ? 0.f : fast_exp2(st.m - mnew);
    st.l *= alpha;
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] *= alpha;
    st.m = mnew;
  }
  // masked scores are -inf: exp2(-inf) = 0 (a row without any key here has
  // m = -inf only if it never had one, and then every score is -inf too)
  const float negm = st.m == NEG_INF ? 0.f : -st.m;
  bf16x8 p0, p1;
  float lsum = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const float e = fast_exp2(__builtin_fmaf(s[v], c, negm));
    lsum += e;
    if (v < 8) p0[v] = (__bf16)e;
    else p1[v - 8] = (__bf16)e;
  }
  st.l += lsum;

  // O^T += V^T P^T
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    acc[b] = mfma32(vf[b][0], p0, acc[b]);
    acc[b] = mfma32(vf[b][1], p1, acc[b]);
  }
}

// softmax step of one unmasked 32-key sub-block: lazy max update, p = 2^(s c - m)
template <int NB>
TTCD_DEV void softmax32(f32x16& s, float c, SoftState& st, f32x16* acc, bf16x8& p0, bf16x8& p1) {
  float mx = NEG_INF;
#pragma unroll
  for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[v]);
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                     false, false);
    mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c;
  }
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
  float lsum = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const float e = fast_exp2(__builtin_fmaf(s[v], c, negm));
    lsum += e;
    if (v < 8) p0[v] = (__bf16)e;
    else p1[v - 8] = (__bf16)e;
  }
  st.l += lsum;
}

// Both 32-key sub-blocks of a tile, no masking, software-pipelined so the
// MFMA pipe always has queued work while the VALU runs a softmax:
//   QK(1) | QK(0) + softmax(1) | PV(1) + softmax(0) | PV(0)
template <int D>
TTCD_DEV void process_pair(const char* buf, float c, const bf16x8* qf, SoftState& st,
                           f32x16* acc, int lane) {
  using TL = Tile<D>;
  constexpr int NB = D / 32;
  constexpr int KSTEP = D / 16;
  const int h = lane >> 5, r = lane & 31;
  const char* vb = buf + TL::KPOS * 16;
  bf16x8 kf[KSTEP];
  bf16x8 vf[NB][2];
  f32x16 s1 = zero16(), s0 = zero16();
  bf16x8 p0, p1;

  auto load_k = [&](int sb) {
    const int row = 32 * sb + r;
    const char* krow = buf + row * (TL::CPR * 16);
    const int sw = TL::kswz(row);
#pragma unroll
    for (int ks = 0; ks < KSTEP; ++ks) kf[ks] = as_bf16x8(ld16(krow + (((2 * ks + h) ^ sw) << 4)));
  };
  auto load_v = [&](int sb) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int d = 32 * b + r;
      const char* vrow = vb + d * (BN * 2);
      const int sw = TL::vswz(d);
      vf[b][0] = as_bf16x8(ld16(vrow + (((4 * sb + 0 + h) ^ sw) << 4)));
      vf[b][1] = as_bf16x8(ld16(vrow + (((4 * sb + 2 + h) ^ sw) << 4)));
    }
  };

  load_k(1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < KSTEP; ++ks) s1 = mfma32(kf[ks], qf[ks], s1);
  __builtin_amdgcn_sched_barrier(0);
  load_k(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < KSTEP; ++ks) s0 = mfma32(kf[ks], qf[ks], s0);
  __builtin_amdgcn_sched_barrier(0);
  load_v(1);
  __builtin_amdgcn_sched_barrier(0);
  softmax32<NB>(s1, c, st, acc, p0, p1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    acc[b] = mfma32(vf[b][0], p0, acc[b]);
    acc[b] = mfma32(vf[b][1], p1, acc[b]);
  }
  __builtin_amdgcn_sched_barrier(0);
  load_v(0);
  __builtin_amdgcn_sched_barrier(0);
  softmax32<NB>(s0, c, st, acc, p0, p1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    acc[b] = mfma32(vf[b][0], p0, acc[b]);
    acc[b] = mfma32(vf[b][1], p1, acc[b]);
  }
}

template <int NB>
TTCD_DEV void store_out(void* o, float* lse, int out_bf16, bool row_ok, size_t obase, size_t li,
                        const SoftState& st, const f32x16* acc, int h) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(st.l), __float_as_uint(st.l),
                                                   false, false);
  const float l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  const float inv = 1.f / l;
  if (!row_ok) return;
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = 32 * bb + 8 * g4 + 4 * h;
      float ov[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[e] = acc[bb][4 * g4 + e] * inv;
      if (out_bf16) {
        *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(o) + obase + d) =
            u32x2{pack_bf16x2(ov[0], ov[1]), pack_bf16x2(ov[2], ov[3])};
      } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(o) + obase + d) =
            f32x4{ov[0], ov[1], ov[2], ov[3]};
      }
    }
  }
  if (h == 0 && lse) lse[li] = (st.m + fast_log2(l)) * LN2;
}

template <int D, int NW>
__global__ void __launch_bounds__(64 * NW)
dual_window_attn_mfma(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                      const bf16_t* __restrict__ vt, int vt_ld,
                      void* __restrict__ o_t, void* __restrict__ o_s,
                      float* __restrict__ lse_t, float* __restrict__ lse_s,
                      int B, int Tq, int Tk, int kv_rows, int q_pos0, int Hq, int Hkv,
                      int wT, int wS, float c, int out_bf16, int nblk) {
  using TL = Tile<D>;
  constexpr int NB = D / 32;
  constexpr int KSTEP = D / 16;
  constexpr int ROWS = 32 * NW;
  extern __shared__ __align__(16) char lds[];

  const int G = Hq / Hkv;
  const int R = Tq * G;
  const uint32_t total = (uint32_t)B * Hkv * nblk;
  const uint32_t lid = xcd_remap(blockIdx.x, total);
  const int blk = lid % nblk;
  const int bg = lid / nblk;
  const int g = bg % Hkv;
  const int b = bg / Hkv;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63;
  const int h = lane >> 5;

  // ---- this lane's query row: (position, head) pair of the kv group
  const int row0 = blk * ROWS;
  const int rw0 = row0 + 32 * wave;
  int r = rw0 + (lane & 31);
  const bool row_ok = r < R;
  r = row_ok ? r : R - 1;
  const int qi = r / G;
  const int qh = g * G + (r % G);
  const int t = q_pos0 + qi;

  // wave / workgroup position ranges
  const int a_w = q_pos0 + min(rw0, R - 1) / G;
  const int b_w = q_pos0 + min(rw0 + 31, R - 1) / G;
  const int A = q_pos0 + row0 / G;
  const int Bp = q_pos0 + min(row0 + ROWS - 1, R - 1) / G;
  const int jlo = max(0, A - wT + 1);
  const int jhi = min(Bp, Tk - 1);
  const int sLo = a_w - wS + 1;                 // oldest key of any row's student band
  const int fLo = max(a_w - wT + 1, 0);         // oldest key of any row's teacher band
  const int j0_lastS = max(sLo, 0) & ~31;       // the wave's oldest student sub-block

  bf16x8 qf[KSTEP];
  {
    const bf16_t* qp = q + ((size_t)(b * Tq + qi) * Hq + qh) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < KSTEP; ++s) qf[s] = as_bf16x8(ld16(qp + 16 * s));
  }
  f32x16 acc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) acc[i] = zero16();
  SoftState st = {NEG_INF, 0.f};

  const bf16_t* kbase = k + ((size_t)b * kv_rows * Hkv + g) * D;
  const size_t kstride = (size_t)Hkv * D;
  const bf16_t* vbase = vt + (size_t)(b * Hkv + g) * D * vt_ld;
  const size_t obase = ((size_t)(b * Tq + qi) * Hq + qh) * D;
  const size_t li = (size_t)(b * Hq + qh) * Tq + qi;

  // tiles are fetched two ahead of the one being computed
  constexpr int LPW = (TL::KPOS + TL::VPOS) / (64 * NW);   // 16B loads per wave and tile
  const int n_hi = jhi / BN, n_lo = jlo / BN;
  issue_tile<D, NW>(lds + (n_hi % NBUF) * TL::BYTES, kbase, kstride, vbase, vt_ld, n_hi * BN,
                    jlo, jhi, wave, lane);
  if (n_hi - 1 >= n_lo) {
    issue_tile<D, NW>(lds + ((n_hi - 1) % NBUF) * TL::BYTES, kbase, kstride, vbase, vt_ld,
                      (n_hi - 1) * BN, jlo, jhi, wave, lane);
    wait_vm<LPW>();
  } else {
    wait_vm<0>();
  }
  ring_barrier();

  for (int n = n_hi; n >= n_lo; --n) {
    const bool fetch = n - 2 >= n_lo;
    if (fetch)
      issue_tile<D, NW>(lds + ((n - 2) % NBUF) * TL::BYTES, kbase, kstride, vbase, vt_ld,
                        (n - 2) * BN, jlo, jhi, wave, lane);
    const char* buf = lds + (n % NBUF) * TL::BYTES;
    // work items of this tile, newest first: sub-block 1, sub-block 0, and
    // right after the wave's oldest student sub-block the far part of its
    // (at most two) edge sub-blocks
    int sbq = 1, pend = 0;
    {
      // fast path: both sub-blocks inside one band for every row of the wave
      const int j0b = n * BN;                                 // sub-block 0
      const int j0a = j0b + 32;                               // sub-block 1 (newer)
      const bool a_in = !(j0a > b_w || j0a + 31 < fLo);
      const bool b_in = !(j0b > b_w || j0b + 31 < fLo);
      auto unmasked = [&](int j0) {
        return (j0 + 31 >= sLo) ? (j0 + 31 <= a_w && j0 >= b_w - wS + 1) : (j0 >= b_w - wT + 1);
      };
      if (a_in && b_in && j0a != j0_lastS && unmasked(j0a) && unmasked(j0b)) {
        process_pair<D>(buf, c, qf, st, acc, lane);
        sbq = -1;
        if (j0b == j0_lastS) {
          store_out<NB>(o_s, lse_s, out_bf16, row_ok, obase, li, st, acc, h);
          pend = wT > wS ? 2 : 0;
        }
      }
    }
#pragma unroll 1
    while (true) {
      int j0, lo, hi;
      bool masked, main_item;
      const char* b;
      if (pend > 0) {
        j0 = j0_lastS + 32 * (2 - pend);
        --pend;
        if (j0 > b_w - wS) continue;
        b = lds + ((j0 / BN) % NBUF) * TL::BYTES;
        masked = true;
        lo = wS;
        hi = wT;
        main_item = false;
      } else if (sbq >= 0) {
        j0 = n * BN + 32 * sbq;
        --sbq;
        const int j1 = j0 + 31;
        if (j0 > b_w || j1 < fLo) continue;      // outside every row's teacher band
        b = buf;
        main_item = true;
        if (j1 >= sLo) {                          // student band (and causal diagonal)
          masked = !(j1 <= a_w && j0 >= b_w - wS + 1);
          lo = 0;
          hi = wS;
        } else {                                  // far band: >= w_S behind every row
          masked = !(j0 >= b_w - wT + 1);
          lo = wS;
          hi = wT;
        }
      } else {
        break;
      }
      process<D>(b, (j0 >> 5) & 1, j0, t, masked, lo, hi, c, qf, st, acc, lane);
      if (main_item && j0 == j0_lastS) {
        // the student band is complete: write it, then add the far edge
        store_out<NB>(o_s, lse_s, out_bf16, row_ok, obase, li, st, acc, h);
        pend = wT > wS ? 2 : 0;
      }
    }
    // tile n-1 must be in LDS; tile n-2 may still be in flight
    if (fetch)
      wait_vm<LPW>();
    else
      wait_vm<0>();
    ring_barrier();
  }
  store_out<NB>(o_t, lse_t, out_bf16, row_ok, obase, li, st, acc, h);
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
  constexpr int NW = 8;
  const size_t lds = (size_t)NBUF * Tile<D>::BYTES;
  static hipError_t attr = hipFuncSetAttribute((const void*)dual_window_attn_mfma<D, NW>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)lds);
  if (attr != hipSuccess) return attr;
  const int G = a.Hq / a.Hkv;
  const int R = a.Tq * G;
  const int nblk = (R + 32 * NW - 1) / (32 * NW);
  const long total = (long)a.B * a.Hkv * nblk;
  const float c = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((dual_window_attn_mfma<D, NW>), dim3((unsigned)total), dim3(64 * NW), lds,
                     s, (const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.vt, a.vt_ld,
                     a.o_t, a.o_s, a.lse_t, a.lse_s, a.B, a.Tq, a.Tk, a.kv_rows, a.q_pos0, a.Hq,
                     a.Hkv, a.wT, a.wS, c, a.out_dt == BF16 ? 1 : 0, nblk);
  return hipGetLastError();
}

// V^T operand of the PV product: vt[b, g, d, c] = v[b, key(c), g, d], where
// storage column c holds key c with bits 2 and 3 swapped inside each group
// of 16, so that one 16-byte LDS read gives a lane the 8 keys of its MFMA
// operand.  Keys outside [jlo, Tk) are written as zero.  One workgroup per
// 64 keys x 64 dims, 16-byte loads and stores through an LDS tile.
__global__ void __launch_bounds__(256)
v_transpose_kernel(const uint16_t* __restrict__ v, uint16_t* __restrict__ vt, int Tk, int jlo,
                   int kv_rows, int Hkv, int D, int vt_ld) {
  __shared__ __align__(16) uint16_t tile[64][64 + 8];   // [key][dim]
  const int bg = blockIdx.z;
  const int b = bg / Hkv, g = bg % Hkv;
  const long j0 = (long)blockIdx.x * 64;
  const int d0 = blockIdx.y * 64;
  const uint16_t* vp = v + ((size_t)b * kv_rows * Hkv + g) * D + d0;
  uint16_t* op = vt + ((size_t)bg * D + d0) * vt_ld + j0;
  const int t = threadIdx.x;
  const int c = t & 7;                       // 16-byte piece of a 64-element row
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int i = (t >> 3) + 32 * it;        // key row of the tile
    const long j = j0 + i;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (j >= jlo && j < Tk) val = ld16(vp + j * Hkv * D + c * 8);
    *reinterpret_cast<u32x4*>(&tile[i][c * 8]) = val;
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int dd = (t >> 3) + 32 * it;       // dim row of the output
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int c0 = c * 8 + e, c1 = c0 + 1;
      const int k0 = (c0 & ~12) | ((c0 & 4) << 1) | ((c0 & 8) >> 1);
      const int k1 = (c1 & ~12) | ((c1 & 4) << 1) | ((c1 & 8) >> 1);
      o[e / 2] = (uint32_t)tile[k0][dd] | ((uint32_t)tile[k1][dd] << 16);
    }
    st16(op + (size_t)dd * vt_ld + c * 8, o);
  }
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
    // V^T with the keys every query may read: [max(0, q_pos0 - w_T + 1), Tk)
    const int jlo_all = a.q_pos0 - a.wT + 1 > 0 ? a.q_pos0 - a.wT + 1 : 0;
    // grid covers vt_ld (a multiple of 64) keys and D (64 or 128) dims
    hipLaunchKernelGGL(v_transpose_kernel, dim3(a.vt_ld / 64, a.D / 64, a.B * a.Hkv), dim3(256),
                       0, s, (const uint16_t*)a.v, (uint16_t*)a.vt, a.Tk, jlo_all, a.kv_rows,
                       a.Hkv, a.D, a.vt_ld);
    hipError_t e = hipGetLastError();
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
