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
//     (global_load_lds_dwordx4) in a 4-slot ring, XOR-swizzled so that the
//     MFMA operand reads are free of bank conflicts.  V arrives
//     pre-transposed (d-major) with the keys of every 16-key group permuted
//     so that one 16-byte LDS read yields the 8 keys an MFMA lane needs.
//   * The two groups of four waves (one wave of each per SIMD) run half a
//     step apart: while one wave of a SIMD issues the QK and PV products,
//     the other computes a softmax (see the kernel's comment).
//   * ONE online-softmax state per row, walked newest to oldest: first the
//     student band (masked only on edge sub-blocks); once the wave's oldest
//     student sub-block is in, the student output is written and the walk
//     continues through the far band.  The far part of the (at most two)
//     sub-blocks at the w_S edge is added at the end, from global memory.
//     Rows whose far band is empty finish with bit-identical teacher and
//     student results.
//   * Lazy rescaling: the running max only moves when a new score exceeds
//     it by more than 2^8; the result is unchanged up to rounding.  The
//     softmax segment does not sum its terms: the wave adds them to the
//     denominator in fp32 between its next MFMAs, and the rescale test is
//     one exponent bit of the packed bf16 terms.
#include "common.hpp"
#include "kernels.hpp"

namespace ttcd {

namespace {

constexpr int BN = 64;          // keys per LDS tile
constexpr float TAU = 8.0f;     // lazy-rescale threshold (log2 domain)
constexpr float NEG_INF = -__builtin_inff();
constexpr float LN2 = 0.69314718055994530942f;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4_t;

typedef __attribute__((address_space(3))) const char lds_char_t;
// 16-byte LDS read at a register byte address plus a constant byte offset,
// written as pointer arithmetic so that the offset lands in the read's
// offset field.  The MFMA kernel has no static LDS, so its dynamic LDS
// starts at address 0 and an offset into it is the address.
TTCD_DEV u32x4 lds16(uint32_t base, uint32_t off) {
  lds_char_t* p = reinterpret_cast<lds_char_t*>((size_t)base);
  return *reinterpret_cast<lds_u32x4_t*>(p + off);
}

// 16 bytes per lane, global -> LDS; lane i lands at lds_wave_base + 16 i.
// Written as inline asm rather than the compiler builtin: the compiler counts
// a builtin LDS DMA as an outstanding LDS operation of unknown order, and
// then waits for every LDS read of a chain (lgkmcnt 0) before the first MFMA
// that needs only the oldest.  The hardware counts the DMA in vmcnt alone,
// and the kernel orders it explicitly (wait_vm before the publishing barrier).
// M0 takes the LDS address (bound as an operand, so the compiler writes it);
// one wait state separates that write from the DMA.
TTCD_DEV void g2l16(const void* src, void* lds_wave_base) {
  const uint32_t m = (uint32_t)(size_t)(lds_void_t*)lds_wave_base;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(src), "{m0}"(m) : "memory");
}
// The same from a wave-uniform base (scalar registers) plus a per-lane byte
// offset, so that only scalar arithmetic moves the source from load to load.
TTCD_DEV void g2l16s(const void* sbase, uint32_t voff, void* lds_wave_base) {
  const uint32_t m = (uint32_t)(size_t)(lds_void_t*)lds_wave_base;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(voff), "s"(sbase), "{m0}"(m)
               : "memory");
}

// Workgroup barrier that does not drain this wave's in-flight tile fetches
// (a fenced barrier would wait for every outstanding memory operation).  LDS
// ordering: the waves that fetch a tile wait for it with wait_vm before the
// barrier that publishes it, and every wave's LDS reads of a slot are
// complete (lgkmcnt 0) before the barrier after which the slot is refilled.
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

// The running max m is held TAU - 1 above the scaled row max it was last
// raised to, so every term 2^(s c - m) starts at most 2^-(TAU-1); a term
// that reaches 2 (its score exceeds the row max by TAU) raises m.
struct SoftState {
  float m;          // running max plus TAU - 1 (log2 domain, scaled)
  float l, l2;      // this lane's partial denominator, two interleaved sums
  float negm;       // -m, or 0 while m = -inf (the exponent offset)
  uint32_t force;   // the exponent bits of a packed bf16 term >= 2 while
                    // m = -inf (forces the first raise), else 0
};

// O = acc / l and LSE = ln 2 (m + log2 l) of the lane's row; o or lse may be
// NULL (not wanted).  A row that saw no key (possible only for the shifted
// band of the LSE-combination path) gets O = 0 and LSE = -inf.
template <int NB>
TTCD_DEV void store_out(void* o, float* lse, int out_bf16, bool row_ok, size_t obase, size_t li,
                        const SoftState& st, const f32x16* acc, int h) {
  const float lp = st.l + st.l2;
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lp), __float_as_uint(lp),
                                                   false, false);
  const float l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (!row_ok) return;
  if (o) {
    // lane (r, h) holds dims 32 bb + 8 g4 + 4 h + e of its row
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
  }
  if (h == 0 && lse) lse[li] = l > 0.f ? (st.m + fast_log2(l)) * LN2 : NEG_INF;
}

// --------------------------------------------------------------------------
// Two groups of four waves, one wave of each group per SIMD.  Each wave
// walks the workgroup's sub-blocks of 32 keys (newest first) as alternating
// segments, every one ended by a workgroup barrier:
//   M(k): PV of sub-block k-1 with the K fragments of sub-block k loaded
//         behind it, then S(k) = K(k) Q^T with the V^T fragments of k loaded
//         behind it;
//   X(k): the mask of S(k), P(k) = 2^(S(k) c - m) and its sum on the
//         vector ALU, with the lazy rescale.
// Group 1 runs one segment behind group 0 (it passes one extra barrier at
// the start, group 0 one at the end), so on each SIMD one wave feeds the
// matrix cores while the other runs a softmax.
//
// Keys that are far (w_S <= t-j) for some rows but lie in the two sub-blocks
// at the w_S edge are walked with the student mask only; their far part is
// added after the walk, from global memory, once the student output is out.
//
// Tile ring (NBUF slots of 64 keys): group 0 fetches the K part of every
// tile, group 1 the V^T part.  Tile i is read in M(2i) and M(2i+1).  Each
// group issues its part of tile i+NBUF into the slot of tile i in its
// M(2i+3), between the two MFMA chains, after every wave's reads of tile i
// have completed (each wave drains its LDS reads at the end of every X
// segment), and waits for its part of tile i before the barrier that
// publishes it: group 0 at the end of X(2i-1), group 1 (one segment
// behind) at the end of its M(2i-1).
// --------------------------------------------------------------------------
template <int V>
struct Int {
  static constexpr int value = V;
};

template <int D>
struct MfmaCfg {
  static constexpr int NB = D / 32;
  static constexpr int KSTEP = D / 16;
  static constexpr int NW = 8;
  static constexpr int ROWS = 32 * NW;
  static constexpr int NBUF = 4;
  static constexpr int ISSUERS = 4;     // waves per group; group 0 fetches K, group 1 V^T
  static constexpr int LPT = Tile<D>::KPOS / (64 * ISSUERS);   // loads per wave per tile
  static_assert(Tile<D>::KPOS == Tile<D>::VPOS, "K and V^T parts of a tile are equal");
};

TTCD_DEV void lds_wait_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// vmcnt wait with a run-time count among {0, L, 2L, 3L}
template <int L>
TTCD_DEV void wait_vm_tiles(int ntiles) {
  if (ntiles >= 3)
    wait_vm<3 * L>();
  else if (ntiles == 2)
    wait_vm<2 * L>();
  else if (ntiles == 1)
    wait_vm<L>();
  else
    wait_vm<0>();
}

// row max of the raw scores of one 32-key sub-block
TTCD_DEV float row_max32(const f32x16& s) {
  float mx = NEG_INF;
#pragma unroll
  for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[v]);
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                   false, false);
  // the two halves' maxima; a plain v_max_f32 (fmaxf would first quiet
  // both operands, which come back from the swap as integers)
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(sw[0]), "v"(sw[1]));
  return r;
}

// keys with lo <= t - j < hi keep their score, the others become -inf
TTCD_DEV void mask32(f32x16& s, int t, int j0, int h, int lo, int hi) {
  const uint32_t d0 = (uint32_t)(t - j0 - 4 * h - lo), span = (uint32_t)(hi - lo);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const uint32_t dl = d0 - (uint32_t)(8 * (v >> 2) + (v & 3));
    s[v] = dl < span ? s[v] : NEG_INF;
  }
}

// 2^(s c + negm) of this lane's 16 scores (sixteen independent fma -> exp
// chains), and the terms packed to bf16 for the PV product
TTCD_DEV void exp_pack16(const f32x16& s, float c, float negm, f32x16& x, bf16x8& p0,
                         bf16x8& p1) {
#pragma unroll
  for (int v = 0; v < 16; ++v) x[v] = __builtin_fmaf(s[v], c, negm);
#pragma unroll
  for (int v = 0; v < 16; ++v) x[v] = fast_exp2(x[v]);
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    p0[v] = (__bf16)x[v];
    p1[v] = (__bf16)x[v + 8];
  }
}

// Whether some packed bf16 term is >= 2 (or +inf/NaN): the terms are not
// negative, so that is the top exponent bit of either half of some word.
TTCD_DEV bool any_ge2(const bf16x8& p0, const bf16x8& p1, uint32_t force) {
  const u32x4 a = __builtin_bit_cast(u32x4, p0), b = __builtin_bit_cast(u32x4, p1);
  const uint32_t o = (a[0] | a[1] | a[2]) | (a[3] | b[0] | b[1]) | (b[2] | b[3] | force);
  return (o & 0x40004000u) != 0u;
}

// P = 2^(s c - m) in bf16 for the PV product and in fp32 (x) for the
// denominator, against the running max m as it stands; the denominator sum
// is left to the matrix segment (den_add).  The rescale is lazy and needs no
// row max in the common case: only when some term of the wave reaches 2
// (a score more than 2^TAU above the max m was last raised for), or a lane
// has no finite max yet, does the wave raise m to the sub-block's row max
// plus TAU - 1, rescale its accumulators and recompute the terms.
template <int NB>
TTCD_DEV void softmax_p(const f32x16& s, float c, SoftState& st, f32x16* acc, f32x16& x,
                        bf16x8& p0, bf16x8& p1) {
  exp_pack16(s, c, st.negm, x, p0, p1);
  if (__builtin_expect(__any(any_ge2(p0, p1, st.force)), 0)) {
    const float mnew = fmaxf(st.m, row_max32(s) * c + (TAU - 1.f));
    const float alpha = (st.m == NEG_INF) ? 0.f : fast_exp2(st.m - mnew);
    st.l *= alpha;
    st.l2 *= alpha;
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] *= alpha;
    st.m = mnew;
    st.negm = mnew == NEG_INF ? 0.f : -mnew;
    st.force = mnew == NEG_INF ? 0x4000u : 0u;
    exp_pack16(s, c, st.negm, x, p0, p1);
  }
}

// Terms v0 .. v0+N-1 of a sub-block's fp32 P into the two denominator sums.
// The empty asm takes both sums as operands at this point, so the compiler
// keeps the adds here (between the MFMAs of the matrix segment) instead of
// sinking them towards their first use, in front of the next softmax.
template <int N>
TTCD_DEV void den_add(SoftState& st, const f32x16& x, int v0) {
#pragma unroll
  for (int j = 0; j < N; ++j) {
    if ((v0 + j) & 1)
      st.l2 += x[v0 + j];
    else
      st.l += x[v0 + j];
  }
  asm volatile("" : "+v"(st.l), "+v"(st.l2));
}

// How this wave takes the sub-block of 32 keys starting at j0 in the walk:
// not at all, or with keys lo <= t - j < hi for the student band (w_S edge
// blocks included: lo = 0, hi = w_S) or the far band (lo = w_S, hi = w_T),
// masked when some row of the wave sees only part of the sub-block.  All
// values are wave-uniform; selects, no branches.
struct Item {
  bool act, masked;
  int lo, hi;
};
struct Band {
  int a_w, b_w, sLo, fLo, wS, wT;
  TTCD_DEV Item item(int j0) const {
    const int j1 = j0 + 31;
    const bool stud = j1 >= sLo;
    Item it;
    it.act = j0 <= b_w && j1 >= fLo;
    it.masked = stud ? !(j1 <= a_w && j0 >= b_w - wS + 1) : !(j0 >= b_w - wT + 1);
    it.lo = stud ? 0 : wS;
    it.hi = stud ? wS : wT;
    return it;
  }
};

template <int D>
__global__ void __launch_bounds__(512)
dual_window_attn_mfma(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                    const bf16_t* __restrict__ vt, int vt_ld, void* __restrict__ o_t,
                    void* __restrict__ o_s, float* __restrict__ lse_t,
                    float* __restrict__ lse_s, int B, int Tq, int Tk, int kv_rows, int q_pos0,
                    int Hq, int Hkv, int wT, int wS, float c, int out_bf16, int nblk) {
  using TL = Tile<D>;
  using CF = MfmaCfg<D>;
  constexpr int NB = CF::NB;
  constexpr int KSTEP = CF::KSTEP;
  constexpr int ROWS = CF::ROWS;
  constexpr int NBUF = CF::NBUF;
  constexpr int LPT = CF::LPT;
  extern __shared__ __align__(16) char lds[];

  const int G = Hq / Hkv;
  const int R = Tq * G;
  const uint32_t total = (uint32_t)B * Hkv * nblk;
  const uint32_t lid = xcd_remap(blockIdx.x, total);
  // position blocks run newest first: the workgroups an XCD starts together
  // then have full windows of equal length, stay in step, and re-read each
  // other's K/V tiles from L2 a few tiles apart
  const int blk = nblk - 1 - (int)(lid % nblk);
  const int bg = lid / nblk;
  const int g = bg % Hkv;
  const int b = bg / Hkv;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool issuer = wave < CF::ISSUERS;        // group 0
  const int lane = tid & 63;
  const int h = lane >> 5, r32 = lane & 31;

  const int row0 = blk * ROWS;
  const int rw0 = row0 + 32 * wave;
  int r = rw0 + r32;
  const bool row_ok = r < R;
  r = row_ok ? r : R - 1;
  const int qi = r / G;
  const int qh = g * G + (r % G);
  const int t = q_pos0 + qi;

  Band bd;
  bd.a_w = q_pos0 + min(rw0, R - 1) / G;
  bd.b_w = q_pos0 + min(rw0 + 31, R - 1) / G;
  bd.sLo = bd.a_w - wS + 1;
  bd.fLo = max(bd.a_w - wT + 1, 0);
  bd.wS = wS;
  bd.wT = wT;
  const int A = q_pos0 + row0 / G;
  const int Bp = q_pos0 + min(row0 + ROWS - 1, R - 1) / G;
  const int jlo = max(0, A - wT + 1);
  const int jhi = min(Bp, Tk - 1);
  const int j0_lastS = max(bd.sLo, 0) & ~31;

  bf16x8 qf[KSTEP];
  {
    const bf16_t* qp = q + ((size_t)(b * Tq + qi) * Hq + qh) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < KSTEP; ++s) qf[s] = as_bf16x8(ld16(qp + 16 * s));
  }
  f32x16 acc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) acc[i] = zero16();
  SoftState st = {NEG_INF, 0.f, 0.f, 0.f, 0x4000u};

  const bf16_t* kbase = k + ((size_t)b * kv_rows * Hkv + g) * D;
  const size_t kstride = (size_t)Hkv * D;
  const bf16_t* vbase = vt + (size_t)(b * Hkv + g) * D * vt_ld;
  const size_t obase = ((size_t)(b * Tq + qi) * Hq + qh) * D;
  const size_t li = (size_t)(b * Hq + qh) * Tq + qi;

  const int n_hi = jhi / BN, n_lo = jlo / BN;
  const int NT = n_hi - n_lo + 1;            // tiles, newest first
  const int K = 2 * NT;                       // sub-blocks
  auto j0_of = [&](int x) { return (n_hi - (x >> 1)) * BN + ((x & 1) ? 0 : 32); };
  // the walk position of the oldest student sub-block
  const int kL = 2 * (n_hi - j0_lastS / BN) + (((j0_lastS >> 5) & 1) ? 0 : 1);

  // LDS operand addresses.  The swizzled chunk of a K row or V^T row is
  // (logical chunk) ^ (per-lane swizzle); the k-step, key-half and sub-block
  // parts of the logical chunk occupy address bits that no other part uses:
  //   K, sub-block x, k-step i:  ring(x) + 32 sb(x) CPR 16 + (klane ^ 32 i)
  //   V^T, MFMA i of PV:         ring(x) + KPOS 16 + 4096 (i/2)
  //                              + (vlane ^ (64 sb(x) + 32 (i%2)))
  // (klane stays below the 32-row block of KSB bytes, vlane below 4 KB).  The
  // registers kl and vl hold ring(x) plus each lane part; the key half and
  // the V^T region are immediate offsets of the LDS reads, so a fragment
  // address costs no vector ALU work, and the registers move to the next
  // ring slot once per tile.
  const uint32_t klane = (uint32_t)(r32 * (TL::CPR * 16) + ((h ^ TL::kswz(r32)) << 4));
  const uint32_t vlane = (uint32_t)(r32 * (BN * 2) + ((h ^ TL::vswz(r32)) << 4));
  constexpr int KSB = 32 * TL::CPR * 16;
  static_assert((KSB & (KSB - 1)) == 0 && TL::BYTES % KSB == 0 && 32 * KSTEP <= KSB &&
                (TL::KPOS * 16) % 4096 == 0 && 32 * BN * 2 <= 4096, "fragment address layout");
  static_assert(KSB < 65536 && TL::KPOS * 16 + 4096 * (NB - 1) < 65536, "16-bit read offsets");
  uint32_t kl[KSTEP], vl[2][2];
#pragma unroll
  for (int i = 0; i < KSTEP; ++i) kl[i] = klane ^ (uint32_t)(32 * i);
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
    for (int e = 0; e < 2; ++e) vl[sb][e] = vlane ^ (uint32_t)(64 * sb + 32 * e);
  }
  // K fragment i of the current tile's sub-block half sb (1: the newer keys)
  auto load_k1 = [&](int sb, int i, bf16x8& dst) __attribute__((always_inline)) {
    dst = as_bf16x8(lds16(kl[i], (uint32_t)(sb * KSB)));
  };
  // V^T fragment of MFMA i of the PV of the current tile's half sb
  auto load_v1 = [&](int sb, int i, bf16x8& dst) __attribute__((always_inline)) {
    dst = as_bf16x8(lds16(vl[sb][i & 1], (uint32_t)(TL::KPOS * 16 + 4096 * (i >> 1))));
  };

  // Tile fetch, 16 bytes per lane straight into LDS, by the four waves of a
  // group (w = wave % 4).  For K, load u of a wave covers rows
  // (u*4 + w) * 64/CPR + lane/CPR and its swizzled chunk does not depend on
  // u; for V^T, dims (u*4 + w) * 8 + lane/8.  Only the newest tile can reach
  // past the last key; its rows are clamped there (they are masked).
  constexpr int KRPL = 64 / TL::CPR;          // K rows per load instruction
  const int wv4 = wave & 3;
  const int krow_l = wv4 * KRPL + lane / TL::CPR;
  const int kchunk = (lane % TL::CPR) ^ TL::kswz(krow_l);
  const uint32_t koff_b = (uint32_t)(2 * (krow_l * kstride + kchunk * 8));
  const int vd_l = wv4 * 8 + lane / 8;
  const uint32_t voff_b = (uint32_t)(2 * (vd_l * vt_ld + 8 * ((lane % 8) ^ TL::vswz(vd_l))));
  // group 0 fetches the K part of tile i, group 1 its V^T part
  auto issue = [&](int i) {
    char* buf = lds + (i % NBUF) * TL::BYTES;
    const int j0 = (n_hi - i) * BN;
    if (issuer) {
      if (j0 + BN - 1 < Tk) {
        const char* tb = reinterpret_cast<const char*>(kbase + (size_t)j0 * kstride);
#pragma unroll
        for (int u = 0; u < LPT; ++u)
          g2l16s(tb + (size_t)u * CF::ISSUERS * KRPL * kstride * 2, koff_b,
                 buf + (u * CF::ISSUERS + wv4) * 64 * 16);
      } else {
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
          const int j = min(j0 + u * CF::ISSUERS * KRPL + krow_l, Tk - 1);
          g2l16(kbase + (size_t)j * kstride + kchunk * 8, buf + (u * CF::ISSUERS + wv4) * 64 * 16);
        }
      }
    } else {
      const char* tb = reinterpret_cast<const char*>(vbase + j0);
      char* vb = buf + TL::KPOS * 16;
#pragma unroll
      for (int u = 0; u < LPT; ++u)
        g2l16s(tb + (size_t)u * CF::ISSUERS * 8 * vt_ld * 2, voff_b,
               vb + (u * CF::ISSUERS + wv4) * 64 * 16);
    }
  };

  // ---- prologue: tiles 0 .. NBUF-1 in flight, tile 0 visible
  const int npro = min(NBUF, NT);
  for (int i = 0; i < npro; ++i) issue(i);
  wait_vm_tiles<LPT>(npro - 1);
  ring_barrier();

  bf16x8 vf[NB][2];        // V^T fragments of the sub-block whose PV comes next
  bf16x8 p0, p1;           // its P (zero when the wave skips it)
  f32x16 px = zero16();    // the same terms in fp32, for the denominator
#pragma unroll
  for (int v = 0; v < 8; ++v) p0[v] = p1[v] = (__bf16)0.f;
#pragma unroll
  for (int i = 0; i < NB; ++i) vf[i][0] = vf[i][1] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});

  // M(kk): PV(kk-1) with the K fragments of sub-block kk loaded behind it
  // and the terms of P(kk-1) added to the denominator between the MFMAs,
  // then QK(kk) with the V^T fragments of kk loaded behind it: each load
  // reuses the registers of the fragment the MFMA before it read and has a
  // whole MFMA chain to land.  Sub-blocks the wave skips go through the
  // same code (their P is zero and their scores are not used).
  // SBc: the half of the current tile that sub-block kk is (1: the newer)
  auto seg_m = [&](auto SBc, f32x16& s, int fill) __attribute__((always_inline)) {
    constexpr int SB = decltype(SBc)::value;
    // At head dim 128 this wave takes the issue slots first while it feeds
    // the matrix cores, and the other wave of the SIMD runs its softmax in
    // the gaps.  At head dim 64 the matrix segment is half as long and the
    // softmax wave goes first instead (measured: 6 % faster there, 6 %
    // slower at 128).
    if constexpr (D == 128) __builtin_amdgcn_s_setprio(2);
    bf16x8 kf[KSTEP];
#pragma unroll
    for (int i = 0; i < KSTEP; ++i) {
      acc[i >> 1] = mfma32(vf[i >> 1][i & 1], (i & 1) ? p1 : p0, acc[i >> 1]);
      __builtin_amdgcn_sched_barrier(0);
      load_k1(SB, i, kf[i]);
      den_add<16 / KSTEP>(st, px, i * (16 / KSTEP));
      __builtin_amdgcn_sched_barrier(0);
    }
    s = zero16();
#pragma unroll
    for (int i = 0; i < KSTEP; ++i) {
      s = mfma32(kf[i], qf[i], s);
      __builtin_amdgcn_sched_barrier(0);
      load_v1(SB, i, vf[i >> 1][i & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // each group refills its part of a ring slot here, behind the MFMA
    // chains (a branch before them would split the block and let the
    // compiler move the second chain behind its loads)
    if (fill >= 0) issue(fill);
    if constexpr (D == 128) __builtin_amdgcn_s_setprio(0);
  };
  // X(kk): the student output right after PV(kL) (P(kL+1) is not in yet),
  // then the mask, row max and softmax of S(kk) (here rather than at the
  // end of M, whose last MFMA result they would wait for)
  auto seg_x = [&](int kk, const Item& ic, f32x16& s) __attribute__((always_inline)) {
    if constexpr (D != 128) __builtin_amdgcn_s_setprio(2);
    if (kk - 1 == kL)
      store_out<NB>(o_s, lse_s, out_bf16, row_ok, obase, li, st, acc, h);
    if (ic.act) {
      if (ic.masked) mask32(s, t, j0_of(kk), h, ic.lo, ic.hi);
      softmax_p<NB>(s, c, st, acc, px, p0, p1);
    } else {
#pragma unroll
      for (int v = 0; v < 8; ++v) p0[v] = p1[v] = (__bf16)0.f;
      px = zero16();
    }
    if constexpr (D != 128) __builtin_amdgcn_s_setprio(0);
  };

  if (!issuer) ring_barrier();                 // group 1 runs one segment behind
  // tile it holds sub-blocks 2 it (newer half) and 2 it + 1
#pragma unroll 1
  for (int it = 0; it < NT; ++it) {
    const int k0 = 2 * it, k1 = k0 + 1;
    const Item i0 = bd.item(j0_of(k0)), i1 = bd.item(j0_of(k1));
    f32x16 s;
    seg_m(Int<1>{}, s, -1);
    ring_barrier();
    seg_x(k0, i0, s);
    lds_wait_all();
    ring_barrier();
    // every wave's reads of tile it - 1 completed before the last barrier:
    // each group refills its part of the slot with tile it - 1 + NBUF
    const int fill = it >= 1 && it - 1 + NBUF < NT ? it - 1 + NBUF : -1;
    seg_m(Int<0>{}, s, fill);
    // the operand registers move on to the next tile's ring slot
    {
      const uint32_t step = (it + 1) % NBUF == 0 ? (uint32_t)(-(NBUF - 1) * TL::BYTES)
                                                 : (uint32_t)TL::BYTES;
#pragma unroll
      for (int i = 0; i < KSTEP; ++i) kl[i] += step;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        vl[sb][0] += step;
        vl[sb][1] += step;
      }
    }
    // group 1 runs one segment behind, so the barrier after its M(k1) is the
    // one that publishes tile it + 1: its V^T part must have landed
    if (!issuer && it + 1 < NT) {
      if (it + NBUF - 1 < NT)
        wait_vm<(NBUF - 2) * LPT>();
      else
        wait_vm<0>();
    }
    ring_barrier();
    seg_x(k1, i1, s);
    // tile it + 1 is read first by the next M: group 0 waits for its K part
    // (the tiles issued after it may stay in flight, except near the end)
    if (issuer && it + 1 < NT) {
      if (it + NBUF - 1 < NT)
        wait_vm<(NBUF - 2) * LPT>();
      else
        wait_vm<0>();
    }
    lds_wait_all();
    ring_barrier();
  }
  // The far part of the (at most two) sub-blocks at the w_S edge comes from
  // global memory at the end (keys with w_S <= t - j < w_T that the walk
  // left out).  Their operand loads are issued early: the first edge
  // sub-block's right after the last PV product (before the closing
  // barriers), the second's before the first one's products, so that their
  // latency overlaps other work.
  const bool edge0 = wT > wS && j0_lastS <= bd.b_w - wS;
  const bool edge1 = wT > wS && j0_lastS + 32 <= bd.b_w - wS;
  auto load_edge_k = [&](int j0, bf16x8* kf) __attribute__((always_inline)) {
    const int j = min(max(j0 + r32, jlo), jhi);
    const bf16_t* kp = kbase + (size_t)j * kstride + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KSTEP; ++ks) kf[ks] = as_bf16x8(ld16(kp + 16 * ks));
  };
  auto load_edge_v = [&](int j0, bf16x8 (*ve)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const bf16_t* vp = vbase + (size_t)(32 * bb + r32) * vt_ld + j0 + 8 * h;
      ve[bb][0] = as_bf16x8(ld16(vp));
      ve[bb][1] = as_bf16x8(ld16(vp + 16));
    }
  };
  auto edge_qk = [&](const bf16x8* kf) __attribute__((always_inline)) {
    f32x16 s = zero16();
#pragma unroll
    for (int i = 0; i < KSTEP; ++i) s = mfma32(kf[i], qf[i], s);
    return s;
  };
  auto edge_pv = [&](int j0, f32x16& s, const bf16x8 (*ve)[2]) __attribute__((always_inline)) {
    mask32(s, t, j0, h, wS, wT);
    softmax_p<NB>(s, c, st, acc, px, p0, p1);
    den_add<16>(st, px, 0);
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      acc[bb] = mfma32(ve[bb][0], p0, acc[bb]);
      acc[bb] = mfma32(ve[bb][1], p1, acc[bb]);
    }
  };

  // M(K): the PV of the last sub-block
#pragma unroll
  for (int i = 0; i < KSTEP; ++i)
    acc[i >> 1] = mfma32(vf[i >> 1][i & 1], (i & 1) ? p1 : p0, acc[i >> 1]);
  den_add<16>(st, px, 0);
  bf16x8 kf0[KSTEP], ve0[NB][2];
  if (edge0) {
    load_edge_k(j0_lastS, kf0);
    load_edge_v(j0_lastS, ve0);
  }
  ring_barrier();
  if (issuer) ring_barrier();                  // group 0's extra barrier
  if (kL == K - 1) {
    // the oldest walked sub-block was the last student one
    store_out<NB>(o_s, lse_s, out_bf16, row_ok, obase, li, st, acc, h);
  }

  if (edge0) {
    // the second edge sub-block's K fragments load behind the first one's
    // QK product, its V^T fragments (into vf, free after the last PV)
    // behind the first one's softmax and PV
    f32x16 s = edge_qk(kf0);
    bf16x8 kf1[KSTEP];
    if (edge1) load_edge_k(j0_lastS + 32, kf1);
    edge_pv(j0_lastS, s, ve0);
    if (edge1) {
      load_edge_v(j0_lastS + 32, vf);
      s = edge_qk(kf1);
      edge_pv(j0_lastS + 32, s, vf);
    }
  }
  store_out<NB>(o_t, lse_t, out_bf16, row_ok, obase, li, st, acc, h);
}

template <int D>
hipError_t launch_mfma(const AttnArgs& a, hipStream_t s) {
  using CF = MfmaCfg<D>;
  const size_t lds = (size_t)CF::NBUF * Tile<D>::BYTES;
  static hipError_t attr = hipFuncSetAttribute((const void*)dual_window_attn_mfma<D>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)lds);
  if (attr != hipSuccess) return attr;
  const int G = a.Hq / a.Hkv;
  const int R = a.Tq * G;
  const int nblk = (R + CF::ROWS - 1) / CF::ROWS;
  const long total = (long)a.B * a.Hkv * nblk;
  const float c = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((dual_window_attn_mfma<D>), dim3((unsigned)total), dim3(64 * CF::NW), lds, s,
                     (const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.vt, a.vt_ld, a.o_t,
                     a.o_s, a.lse_t, a.lse_s, a.B, a.Tq, a.Tk, a.kv_rows, a.q_pos0, a.Hq, a.Hkv,
                     a.wT, a.wS, c, a.out_dt == BF16 ? 1 : 0, nblk);
  return hipGetLastError();
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
  // o_t or o_s may be NULL (not wanted); a row that saw no key (only in the
  // shifted band of the LSE-combination path) gets O = 0 and LSE = -inf
  for (int d = 0; d < D; ++d) {
    const float os = lS > 0.f ? aS[d] / lS : 0.f;
    const float ot = far_empty ? os : (aS[d] * eS + aF[d] * eF) / lT;
    if (out_bf16) {
      if (o_s) reinterpret_cast<bf16_t*>(o_s)[obase + d] = f2bf(os);
      if (o_t) reinterpret_cast<bf16_t*>(o_t)[obase + d] = f2bf(ot);
    } else {
      if (o_s) reinterpret_cast<float*>(o_s)[obase + d] = os;
      if (o_t) reinterpret_cast<float*>(o_t)[obase + d] = ot;
    }
  }
  const size_t li = (size_t)(b * Hq + qh) * Tq + qi;
  const float lseS = lS > 0.f ? mS + logf(lS) : NEG_INF;
  if (lse_s) lse_s[li] = lseS;
  if (lse_t) lse_t[li] = far_empty ? lseS : mT + logf(lT);
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

namespace {

bool mfma_path(const AttnArgs& a) { return a.in_dt == BF16 && (a.D == 64 || a.D == 128); }

// V^T with the keys every query may read: [max(0, q_pos0 - w_T + 1), Tk)
hipError_t launch_vt(const AttnArgs& a, hipStream_t s) {
  const int jlo_all = a.q_pos0 - a.wT + 1 > 0 ? a.q_pos0 - a.wT + 1 : 0;
  // grid covers vt_ld (a multiple of 64) keys and D (64 or 128) dims
  hipLaunchKernelGGL(v_transpose_kernel, dim3(a.vt_ld / 64, a.D / 64, a.B * a.Hkv), dim3(256), 0,
                     s, (const uint16_t*)a.v, (uint16_t*)a.vt, a.Tk, jlo_all, a.kv_rows, a.Hkv,
                     a.D, a.vt_ld);
  return hipGetLastError();
}

hipError_t launch_core(const AttnArgs& a, hipStream_t s) {
  if (mfma_path(a)) return a.D == 64 ? launch_mfma<64>(a, s) : launch_mfma<128>(a, s);
  if (a.in_dt == F32) {
    if (a.D == 64) return launch_simple<float, 64>(a, s);
    if (a.D == 128) return launch_simple<float, 128>(a, s);
  } else {
    if (a.D == 64) return launch_simple<bf16_t, 64>(a, s);
    if (a.D == 128) return launch_simple<bf16_t, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

// Teacher output and LSE from the student-window result and the far band
// (keys with w_S <= t - j < w_T), merged exactly through their log-sum-exps
// (README "Fused inference kernels", the LSE-combination variant): with
// L = log(e^LSE_S + e^LSE_far), O_T = e^(LSE_S - L) O_S + e^(LSE_far - L) O_far.
// lse_far == NULL means the far band is empty for every row (w_T == w_S).
// One thread per 4 head dims of a (row, head); O is [B, Tq, Hq, D], LSE is
// [B, Hq, Tq].
__global__ void __launch_bounds__(256)
lse_merge_kernel(const void* __restrict__ o_s, const float* __restrict__ o_far,
                 const float* __restrict__ lse_s, const float* __restrict__ lse_far,
                 void* __restrict__ o_t, float* __restrict__ lse_t, int Tq, int Hq, int D,
                 long total4, int out_bf16) {
  const long i4 = (long)blockIdx.x * 256 + threadIdx.x;
  if (i4 >= total4) return;
  const long e0 = 4 * i4;                              // first element of the four
  const int d = (int)(e0 % D);
  const long row = e0 / D;                             // (b, qi, qh) flattened
  const int qh = (int)(row % Hq);
  const long bq = row / Hq;                            // b * Tq + qi
  const int qi = (int)(bq % Tq);
  const long b = bq / Tq;
  const size_t li = ((size_t)b * Hq + qh) * Tq + qi;
  const float ls = lse_s[li];
  const float lf = lse_far ? lse_far[li] : NEG_INF;
  float os[4];
  if (out_bf16) {
    const u32x2 u = *reinterpret_cast<const u32x2*>(reinterpret_cast<const bf16_t*>(o_s) + e0);
    os[0] = __uint_as_float(u[0] << 16);
    os[1] = __uint_as_float(u[0] & 0xFFFF0000u);
    os[2] = __uint_as_float(u[1] << 16);
    os[3] = __uint_as_float(u[1] & 0xFFFF0000u);
  } else {
    const f32x4 v = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(o_s) + e0);
#pragma unroll
    for (int j = 0; j < 4; ++j) os[j] = v[j];
  }
  float ot[4], lt;
  if (lf == NEG_INF) {
#pragma unroll
    for (int j = 0; j < 4; ++j) ot[j] = os[j];
    lt = ls;
  } else {
    const f32x4 of = *reinterpret_cast<const f32x4*>(o_far + e0);
    const float mx = fmaxf(ls, lf);
    const float ws = expf(ls - mx), wf = expf(lf - mx);
    const float inv = 1.f / (ws + wf);
#pragma unroll
    for (int j = 0; j < 4; ++j) ot[j] = (ws * os[j] + wf * of[j]) * inv;
    lt = mx + logf(ws + wf);
  }
  if (out_bf16) {
    *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(o_t) + e0) =
        u32x2{pack_bf16x2(ot[0], ot[1]), pack_bf16x2(ot[2], ot[3])};
  } else {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(o_t) + e0) = f32x4{ot[0], ot[1], ot[2], ot[3]};
  }
  if (lse_t && d == 0) lse_t[li] = lt;
}

}  // namespace

hipError_t launch_dual_window_attn(const AttnArgs& a, hipStream_t s) {
  if (mfma_path(a)) {
    hipError_t e = launch_vt(a, s);
    if (e != hipSuccess) return e;
  }
  return launch_core(a, s);
}

// The LSE-combination path: a student-window call (w = w_S), a call over
// the far band (queries shifted back by w_S against a window of w_T - w_S:
// a query at t then sees exactly the keys with w_S <= t - j < w_T), and the
// exact merge.  o_far [B,Tq,Hq,D] fp32, lse_far and lse_tmp [B,Hq,Tq] fp32
// are workspace; lse_tmp holds LSE_S when the caller does not want it.
hipError_t launch_dual_window_attn_lse_split(const AttnArgs& a, float* o_far, float* lse_far,
                                             float* lse_tmp, hipStream_t s) {
  if (mfma_path(a)) {
    hipError_t e = launch_vt(a, s);
    if (e != hipSuccess) return e;
  }
  float* lse_s = a.lse_s ? a.lse_s : lse_tmp;
  AttnArgs st = a;
  st.wT = a.wS;
  st.o_t = nullptr;
  st.lse_t = nullptr;
  st.lse_s = lse_s;
  hipError_t e = launch_core(st, s);
  if (e != hipSuccess) return e;
  const bool far = a.wT > a.wS;
  if (far) {
    AttnArgs fa = a;
    fa.q_pos0 = a.q_pos0 - a.wS;
    fa.wT = fa.wS = a.wT - a.wS;
    fa.o_t = o_far;
    fa.lse_t = lse_far;
    fa.o_s = nullptr;
    fa.lse_s = nullptr;
    fa.out_dt = F32;
    e = launch_core(fa, s);
    if (e != hipSuccess) return e;
  }
  const long total4 = (long)a.B * a.Tq * a.Hq * a.D / 4;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)((total4 + 255) / 256)), dim3(256), 0, s,
                     a.o_s, o_far, lse_s, far ? lse_far : nullptr, a.o_t, a.lse_t, a.Tq, a.Hq,
                     a.D, total4, a.out_dt == BF16 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace ttcd
