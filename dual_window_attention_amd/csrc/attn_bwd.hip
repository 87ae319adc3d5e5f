// Backward of the dual-window attention for gfx950.
//
// What is computed (papernotes.org notes on "Learning What to Remember":
// the overall framework puts teacher and student windows on one shared
// Q/K/V; its limitations section prices training): both windows' outputs
// depend on the same q, k and v, so their gradients add.  Per window w with
// softmax weights P_w = exp(s - LSE_w) on its visible keys (0 <= t-j < w):
//   dV_j += sum_t P_tj dO_t,  dP_tj = dO_t . v_j,  D_t = dO_t . O_t,
//   dS_tj = P_tj (dP_tj - D_t),  dQ_t += c sum_j dS_tj k_j,  dK_j += c sum_t dS_tj q_t
// (c the score scale).  A key with t-j < w_S is in both windows; a key with
// w_S <= t-j < w_T only in the teacher's.
//
// Design here (bf16 MFMA 32x32x16, fp32 accumulate), two deterministic
// kernels that both recompute the scores from the forward's LSE (no atomics):
//   * dK/dV: a workgroup owns 128 keys of one (batch, kv head), 32 per wave,
//     and walks every 32-row query block that sees them.  S = Q K^T puts one
//     key per lane (a column of the MFMA output), so P and dS sit in the
//     lanes exactly as the A operand of dV += P^T dO and dK += dS^T Q wants
//     them, with the 16 query rows of each k-step in the order the output
//     layout gives (bits 2 and 3 of the row swapped).  The B operands of those
//     two products come from transposed copies of Q and dO whose columns are
//     stored in that same order.  K and V stay in registers as the B operands
//     of S and dP = dO V^T.
//   * dQ: a workgroup owns 128 query rows (32 per wave) and walks the 32-key
//     tiles of its window, S^T = K Q^T with one query row per lane (as the
//     forward), dQ^T += K^T dS^T with K^T from a transposed, key-permuted copy.
//   * Query rows are the (position, q head) pairs of a kv group, as in the
//     forward, so the q heads of a group share every tile.
//   * Tiles go global -> LDS directly (global_load_lds_dwordx4), two stages,
//     the next tile in flight while the current one is used.
#include "common.hpp"
#include "kernels.hpp"

namespace ttcd {

namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float POS_INF = __builtin_inff();

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4_t;

// 16-byte LDS read at a byte address of the kernel's dynamic LDS (the kernels
// here have no static LDS, so an offset is the address)
TTCD_DEV u32x4 lds_rd16(uint32_t addr) { return *reinterpret_cast<lds_u32x4_t*>((size_t)addr); }

// 16 bytes per lane, global -> LDS; lane i lands at lds_wave_base + 16 i.
// The DMA is counted in vmcnt only: each wave waits for its own fetches
// (vmcnt 0) before the barrier that publishes a stage.
TTCD_DEV void dma16(const void* src, void* lds_wave_base) {
  const uint32_t m = (uint32_t)(size_t)(lds_void_t*)lds_wave_base;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(src), "{m0}"(m) : "memory");
}

// all of this wave's memory operations complete, then the workgroup barrier
TTCD_DEV void stage_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// storage column of query row (or key) x inside its group of 16: bits 2 and
// 3 swapped, so that the 8 rows an MFMA lane takes for one k-step are 8
// consecutive columns (an involution: the same map goes back)
TTCD_DEV int perm16(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

template <int D>
struct BwdTile {
  static constexpr int NB = D / 32;        // 32-wide column blocks of a D row
  static constexpr int KSTEP = D / 16;     // k-steps of a product over D
  static constexpr int CPR = D / 8;        // 16-byte chunks per D row
  static constexpr int RBYTES = 32 * D * 2;   // a 32-row tile, row-major
  static constexpr int TBYTES = D * 32 * 2;   // a D x 32 transposed tile
  static_assert(RBYTES == TBYTES, "equal tile sizes");
  // swizzled chunk of a row-major tile row / of a transposed tile row
  static TTCD_DEV int rswz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
  static TTCD_DEV int tswz(int d) { return (d >> 2) & 3; }
  // byte address of the A-operand chunk (k-step s, lane half h) of row r
  static TTCD_DEV uint32_t rfrag(uint32_t base, int r, int s, int h) {
    return base + (uint32_t)(r * (CPR * 16) + (((2 * s + h) ^ rswz(r)) << 4));
  }
  // byte address of the operand chunk (k-step s of 2, lane half h) of
  // transposed row d
  static TTCD_DEV uint32_t tfrag(uint32_t base, int d, int s, int h) {
    return base + (uint32_t)(d * 64 + (((2 * s + h) ^ tswz(d)) << 4));
  }
};

// position of query row x of a kv group (rows are (position, q head) pairs)
TTCD_DEV int row_pos(int x, int G, int gshift) { return gshift >= 0 ? (x >> gshift) : x / G; }

// --------------------------------------------------------------------------
// Row data of every query row, in 32-row blocks per (batch, kv group):
//   meta[((b Hkv + g) nblk + blk) 128 + k 32 + i], k = 0: LSE_T log2 e,
//   1: LSE_S log2 e, 2: D_T = dO_T . O_T, 3: D_S = dO_S . O_S
// Rows past the last (padding) get LSE = +inf (their weights vanish) and D = 0.
// One wave per row.
template <typename T>
__global__ void __launch_bounds__(256)
attn_bwd_meta_kernel(const T* __restrict__ o_t, const T* __restrict__ o_s,
                     const T* __restrict__ do_t, const T* __restrict__ do_s,
                     const float* __restrict__ lse_t, const float* __restrict__ lse_s,
                     float* __restrict__ meta, int Tn, int Hq, int Hkv, int D, int nblk,
                     long nrows) {
  const long id = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (id >= nrows) return;
  const int G = Hq / Hkv;
  const int R = Tn * G;
  const long per = (long)nblk * 32;
  const int x = (int)(id % per);
  const int bg = (int)(id / per);
  const int g = bg % Hkv, b = bg / Hkv;
  float lt = POS_INF, ls = POS_INF, dt = 0.f, dsum = 0.f;
  if (x < R) {
    const int t = x / G, hq = g * G + x % G;
    const size_t off = ((size_t)(b * Tn + t) * Hq + hq) * D;
    for (int d = lane; d < D; d += 64) {
      dt = __builtin_fmaf(ldf(do_t + off + d), ldf(o_t + off + d), dt);
      dsum = __builtin_fmaf(ldf(do_s + off + d), ldf(o_s + off + d), dsum);
    }
    dt = wave_sum(dt);
    dsum = wave_sum(dsum);
    const size_t li = ((size_t)b * Hq + hq) * Tn + t;
    lt = lse_t[li] * LOG2E;
    ls = lse_s[li] * LOG2E;
  }
  if (lane == 0) {
    float* m = meta + ((size_t)bg * nblk + x / 32) * 128 + x % 32;
    m[0] = lt;
    m[32] = ls;
    m[64] = dt;
    m[96] = dsum;
  }
}

// The same row data for bf16 rows of D = 64 or 128: D / 8 lanes per row, one
// 16-byte load of each of O_T, O_S, dO_T, dO_S per lane, the dot products
// reduced over those lanes only; 64 / (D / 8) rows per wave.
template <int D>
__global__ void __launch_bounds__(256)
attn_bwd_meta_vec_kernel(const bf16_t* __restrict__ o_t, const bf16_t* __restrict__ o_s,
                         const bf16_t* __restrict__ do_t, const bf16_t* __restrict__ do_s,
                         const float* __restrict__ lse_t, const float* __restrict__ lse_s,
                         float* __restrict__ meta, int Tn, int Hq, int Hkv, int nblk,
                         long nrows) {
  constexpr int LPR = D / 8, RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPR;
  const long id = ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
  if (id >= nrows) return;                 // whole row groups: the lanes of a row agree
  const int G = Hq / Hkv;
  const int R = Tn * G;
  const long per = (long)nblk * 32;
  const int x = (int)(id % per);
  const int bg = (int)(id / per);
  const int g = bg % Hkv, b = bg / Hkv;
  float dt = 0.f, dsum = 0.f;
  size_t li = 0;
  if (x < R) {
    const int t = x / G, hq = g * G + x % G;
    const size_t off = ((size_t)(b * Tn + t) * Hq + hq) * D + 8 * sub;
    const u32x4 a = ld16(do_t + off), c = ld16(o_t + off);
    const u32x4 e = ld16(do_s + off), f = ld16(o_s + off);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dt = __builtin_fmaf(__uint_as_float(a[j] << 16), __uint_as_float(c[j] << 16), dt);
      dt = __builtin_fmaf(__uint_as_float(a[j] & 0xFFFF0000u),
                          __uint_as_float(c[j] & 0xFFFF0000u), dt);
      dsum = __builtin_fmaf(__uint_as_float(e[j] << 16), __uint_as_float(f[j] << 16), dsum);
      dsum = __builtin_fmaf(__uint_as_float(e[j] & 0xFFFF0000u),
                            __uint_as_float(f[j] & 0xFFFF0000u), dsum);
    }
    li = ((size_t)b * Hq + hq) * Tn + t;
  }
#pragma unroll
  for (int o = LPR / 2; o >= 1; o >>= 1) {
    dt += __shfl_xor(dt, o, 64);
    dsum += __shfl_xor(dsum, o, 64);
  }
  if (sub == 0) {
    float* m = meta + ((size_t)bg * nblk + x / 32) * 128 + x % 32;
    m[0] = x < R ? lse_t[li] * LOG2E : POS_INF;
    m[32] = x < R ? lse_s[li] * LOG2E : POS_INF;
    m[64] = dt;
    m[96] = dsum;
  }
}

// Transposed copy of a [B, T, H, D] array, per kv group: out[b][g][d][c] =
// in row perm16-stored (c) of the group, where row x = (position x / G, head
// g G + x % G); rows >= rows_valid are zero.  For K (G = 1, H = Hkv) the rows
// are the keys.  One 64 x 64 tile per workgroup, 16-byte reads and writes.
__global__ void __launch_bounds__(256)
rows_transpose_kernel(const uint16_t* __restrict__ in, uint16_t* __restrict__ out, int Tn, int H,
                      int Hkv, int D, int rows_valid, long ld) {
  __shared__ __align__(16) uint16_t tile[64][64 + 8];   // [row][dim]
  const int bg = blockIdx.z;
  const int b = bg / Hkv, g = bg % Hkv;
  const int G = H / Hkv;
  const long x0 = (long)blockIdx.x * 64;
  const int d0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  const int c = tid & 7;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int i = (tid >> 3) + 32 * it;
    const long x = x0 + i;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (x < rows_valid) {
      const long t = x / G;
      const int hh = (int)(x % G);
      val = ld16(in + ((size_t)(b * (long)Tn + t) * H + g * G + hh) * D + d0 + c * 8);
    }
    *reinterpret_cast<u32x4*>(&tile[i][c * 8]) = val;
  }
  __syncthreads();
  uint16_t* op = out + ((size_t)bg * D + d0) * ld + x0;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int dd = (tid >> 3) + 32 * it;
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int k0 = perm16(c * 8 + e), k1 = perm16(c * 8 + e + 1);
      o[e / 2] = (uint32_t)tile[k0][dd] | ((uint32_t)tile[k1][dd] << 16);
    }
    st16(op + (size_t)dd * ld + c * 8, o);
  }
}

// Masks of one 32 x 32 block: which of the wave's (row, key) pairs take part
struct BlockKind {
  bool act;      // some pair in the teacher window
  bool stud;     // some pair in the student window
  bool tmask;    // the teacher window cuts the block
  bool smask;    // the student window cuts the block
};
TTCD_DEV BlockKind block_kind(int dmin, int dmax, int wT, int wS) {
  BlockKind k;
  k.act = dmax >= 0 && dmin < wT;
  k.stud = dmax >= 0 && dmin < wS;
  k.tmask = dmin < 0 || dmax >= wT;
  k.smask = dmin < 0 || dmax >= wS;
  return k;
}

// --------------------------------------------------------------------------
// dK, dV.  Stage layout (bytes): Q, dO_T, dO_S row-major 32-row tiles, then
// Q^T, dO_T^T, dO_S^T (D x 32, rows perm16-ordered), then 1 KB of row data
// (this block's 512 bytes and the next block's).
template <int D>
struct DkdvCfg {
  using TL = BwdTile<D>;
  static constexpr int OFF_Q = 0, OFF_DOT = TL::RBYTES, OFF_DOS = 2 * TL::RBYTES;
  static constexpr int OFF_QT = 3 * TL::RBYTES, OFF_DOTT = 4 * TL::RBYTES;
  static constexpr int OFF_DOST = 5 * TL::RBYTES, OFF_META = 6 * TL::RBYTES;
  static constexpr int STAGE = 6 * TL::RBYTES + 1024;
  static constexpr int LQ = TL::CPR / 8;      // row-major tile loads per wave
  static constexpr int LT = D / 64;           // transposed tile loads per wave
};

// One 32-row query block of a wave in the dK/dV kernel: S = Q K^T,
// dP_T = dO_T V^T (and dP_S), the weights and dS on the vector ALU, then
// dV += P^T dO and dK += dS^T Q.  The LDS operands of each MFMA chain are
// read four ahead of their MFMA (sched barriers keep that order), so that a
// single wave per SIMD does not stall on every read.
template <int D, bool STUD, bool MASK>
TTCD_DEV void dkdv_block(uint32_t st, int r32, int h, const bf16x8* kf, const bf16x8* vf,
                         f32x16* dka, f32x16* dva, int sb, int key, int G, int gshift, int wT,
                         int wS, float c2, bool tmask, bool smask) {
  using TL = BwdTile<D>;
  using CF = DkdvCfg<D>;
  constexpr int KSTEP = TL::KSTEP, NB = TL::NB;
  constexpr int NA = (STUD ? 3 : 2) * KSTEP;
  auto aaddr = [&](int i) {
    const int c = i / KSTEP, ks = i % KSTEP;
    const int off = c == 0 ? CF::OFF_Q : (c == 1 ? CF::OFF_DOT : CF::OFF_DOS);
    return TL::rfrag(st + off, r32, ks, h);
  };
  f32x16 sacc[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) sacc[c] = zero16();
  bf16x8 fa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[i] = as_bf16x8(lds_rd16(aaddr(i)));
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int c = i / KSTEP, ks = i % KSTEP;
    sacc[c] = mfma32(fa[i & 3], c == 0 ? kf[ks] : vf[ks], sacc[c]);
    __builtin_amdgcn_sched_barrier(0);
    if (i + 4 < NA) fa[i & 3] = as_bf16x8(lds_rd16(aaddr(i + 4)));
    __builtin_amdgcn_sched_barrier(0);
  }
  // P_T, P_S and dS; lane (r32, h) holds key `key` and the rows
  // 4 h + 8 (v / 4) + v % 4 of the block
  bf16x8 pa[2], psa[2], da[2];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const uint32_t mo = st + CF::OFF_META + (uint32_t)((4 * h + 8 * q4) * 4);
    const f32x4 lt4 = __builtin_bit_cast(f32x4, lds_rd16(mo));
    const f32x4 dt4 = __builtin_bit_cast(f32x4, lds_rd16(mo + 256));
    f32x4 ls4 = {0.f, 0.f, 0.f, 0.f}, ds4 = {0.f, 0.f, 0.f, 0.f};
    if (STUD) {
      ls4 = __builtin_bit_cast(f32x4, lds_rd16(mo + 128));
      ds4 = __builtin_bit_cast(f32x4, lds_rd16(mo + 384));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int vv = 4 * q4 + e;
      int dl = 0;
      if (MASK) dl = row_pos(sb * 32 + 4 * h + 8 * q4 + e, G, gshift) - key;
      float pt = fast_exp2(__builtin_fmaf(sacc[0][vv], c2, -lt4[e]));
      if (MASK && tmask && !(dl >= 0 && dl < wT)) pt = 0.f;
      float dsv = pt * (sacc[1][vv] - dt4[e]);
      pa[vv >> 3][vv & 7] = (__bf16)pt;
      if (STUD) {
        float ps = fast_exp2(__builtin_fmaf(sacc[0][vv], c2, -ls4[e]));
        if (MASK && smask && !(dl >= 0 && dl < wS)) ps = 0.f;
        dsv = __builtin_fmaf(ps, sacc[2][vv] - ds4[e], dsv);
        psa[vv >> 3][vv & 7] = (__bf16)ps;
      }
      da[vv >> 3][vv & 7] = (__bf16)dsv;
    }
  }
  // dV += P^T dO (both windows), dK += dS^T Q: item i is k-step (i / PER) % 2
  // of column block i / (2 PER), kind i % PER
  constexpr int PER = STUD ? 3 : 2;
  constexpr int NBK = NB * 2 * PER;
  auto baddr = [&](int i) {
    const int grp = i / PER, kind = i % PER;
    const int nb = grp >> 1, ks = grp & 1;
    const int off = kind == 0 ? CF::OFF_DOTT : (STUD && kind == 1 ? CF::OFF_DOST : CF::OFF_QT);
    return TL::tfrag(st + off, 32 * nb + r32, ks, h);
  };
  bf16x8 fb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) fb[i] = as_bf16x8(lds_rd16(baddr(i)));
#pragma unroll
  for (int i = 0; i < NBK; ++i) {
    const int grp = i / PER, kind = i % PER;
    const int nb = grp >> 1, ks = grp & 1;
    if (kind == 0)
      dva[nb] = mfma32(pa[ks], fb[i & 3], dva[nb]);
    else if (STUD && kind == 1)
      dva[nb] = mfma32(psa[ks], fb[i & 3], dva[nb]);
    else
      dka[nb] = mfma32(da[ks], fb[i & 3], dka[nb]);
    __builtin_amdgcn_sched_barrier(0);
    if (i + 4 < NBK) fb[i & 3] = as_bf16x8(lds_rd16(baddr(i + 4)));
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D>
__global__ void __launch_bounds__(256)
attn_bwd_dkdv_mfma(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                   const bf16_t* __restrict__ v, const bf16_t* __restrict__ dot,
                   const bf16_t* __restrict__ dos, const bf16_t* __restrict__ qT,
                   const bf16_t* __restrict__ dotT, const bf16_t* __restrict__ dosT,
                   const float* __restrict__ meta, void* __restrict__ dk_out,
                   void* __restrict__ dv_out, int out_bf16, int Tn, int Hq, int Hkv, long ldT,
                   int nmeta, int wT, int wS, float c2, float scale, int nkb, int gshift) {
  using TL = BwdTile<D>;
  using CF = DkdvCfg<D>;
  constexpr int NB = TL::NB, KSTEP = TL::KSTEP, CPR = TL::CPR;
  extern __shared__ __align__(16) char lds[];
  const int G = Hq / Hkv;
  const int R = Tn * G;
  const uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int kb = (int)(lid % nkb);
  const int bg = (int)(lid / nkb);
  const int g = bg % Hkv, b = bg / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, r32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jb = kb * 128;
  const int j0 = jb + 32 * wave;
  const int jl = min(j0 + r32, Tn - 1);

  // K and V of this lane's key: the B operands of S = Q K^T and dP = dO V^T
  bf16x8 kf[KSTEP], vf[KSTEP];
  {
    const size_t off = ((size_t)(b * Tn + jl) * Hkv + g) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < KSTEP; ++s) {
      kf[s] = as_bf16x8(ld16(k + off + 16 * s));
      vf[s] = as_bf16x8(ld16(v + off + 16 * s));
    }
  }
  f32x16 dka[NB], dva[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) dka[i] = dva[i] = zero16();
  // drain those loads here, so that no wait for them (which would also wait
  // for the tile fetches in flight) lands inside the loop
  __builtin_amdgcn_s_waitcnt(0);

  // 32-row query blocks holding the positions [jb, jb + 127 + w_T - 1]
  const int pend = min(Tn, jb + 127 + wT);
  const int sb_lo = (int)(((long)jb * G) / 32);
  const int sb_hi = (int)(((long)pend * G + 31) / 32);
  const int nsb = sb_hi - sb_lo;

  // fetch geometry: row-major tiles, load u of this wave covers slots
  // (u * 4 + wave) * 64 + lane: row x, stored chunk sc, source chunk sc ^ swz
  int qx[CF::LQ], qgc[CF::LQ];
#pragma unroll
  for (int u = 0; u < CF::LQ; ++u) {
    const int p = (u * 4 + wave) * 64 + lane;
    qx[u] = p / CPR;
    qgc[u] = (p % CPR) ^ TL::rswz(qx[u]);
  }
  int td[CF::LT], tgc[CF::LT];
#pragma unroll
  for (int u = 0; u < CF::LT; ++u) {
    const int p = (u * 4 + wave) * 64 + lane;
    td[u] = p / 4;
    tgc[u] = (p % 4) ^ TL::tswz(td[u]);
  }
  const size_t tbase = (size_t)bg * D * ldT;
  const float* mbase = meta + (size_t)bg * nmeta * 128;

  auto stud_wg = [&](int sb) {
    const int tA = row_pos(sb * 32, G, gshift);
    return tA - (jb + 127) < wS;
  };
  auto issue = [&](int i) {
    const int sb = sb_lo + i;
    char* st = lds + (i & 1) * CF::STAGE;
    const bool stud = stud_wg(sb);
#pragma unroll
    for (int u = 0; u < CF::LQ; ++u) {
      const int x = min(sb * 32 + qx[u], R - 1);
      const int t = row_pos(x, G, gshift);
      const size_t off = ((size_t)(b * Tn + t) * Hq + g * G + (x - t * G)) * D + qgc[u] * 8;
      char* dst = st + (u * 4 + wave) * 1024;
      dma16(q + off, dst + CF::OFF_Q);
      dma16(dot + off, dst + CF::OFF_DOT);
      if (stud) dma16(dos + off, dst + CF::OFF_DOS);
    }
#pragma unroll
    for (int u = 0; u < CF::LT; ++u) {
      const size_t off = tbase + (size_t)td[u] * ldT + sb * 32 + tgc[u] * 8;
      char* dst = st + (u * 4 + wave) * 1024;
      dma16(qT + off, dst + CF::OFF_QT);
      dma16(dotT + off, dst + CF::OFF_DOTT);
      if (stud) dma16(dosT + off, dst + CF::OFF_DOST);
    }
    if (wave == 0) dma16(mbase + (size_t)sb * 128 + lane * 4, st + CF::OFF_META);
  };

  issue(0);
  stage_barrier();
#pragma unroll 1
  for (int i = 0; i < nsb; ++i) {
    if (i + 1 < nsb) issue(i + 1);
    const int sb = sb_lo + i;
    const uint32_t st = (uint32_t)((i & 1) * CF::STAGE);
    const int tA = row_pos(sb * 32, G, gshift);
    const int tB = row_pos(min(sb * 32 + 31, R - 1), G, gshift);
    const BlockKind bk = block_kind(tA - (j0 + 31), tB - j0, wT, wS);
    if (bk.act && j0 < Tn) {
#define TTCD_DKDV(S, M) \
  dkdv_block<D, S, M>(st, r32, h, kf, vf, dka, dva, sb, j0 + r32, G, gshift, wT, wS, c2, \
                      bk.tmask, bk.smask)
      const bool msk = bk.tmask || (bk.stud && bk.smask);
      if (bk.stud) {
        if (msk) TTCD_DKDV(true, true); else TTCD_DKDV(true, false);
      } else {
        if (msk) TTCD_DKDV(false, true); else TTCD_DKDV(false, false);
      }
#undef TTCD_DKDV
    }
    stage_barrier();
  }

  // lane (r32, h) holds dims 32 nb + r32 of keys j0 + 4 h + 8 (v / 4) + v % 4
#pragma unroll
  for (int vv = 0; vv < 16; ++vv) {
    const int j = j0 + 4 * h + 8 * (vv >> 2) + (vv & 3);
    if (j >= Tn) continue;
    const size_t off = ((size_t)(b * Tn + j) * Hkv + g) * D + r32;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float gk = dka[nb][vv] * scale, gv = dva[nb][vv];
      if (out_bf16) {
        reinterpret_cast<bf16_t*>(dk_out)[off + 32 * nb] = f2bf(gk);
        reinterpret_cast<bf16_t*>(dv_out)[off + 32 * nb] = f2bf(gv);
      } else {
        reinterpret_cast<float*>(dk_out)[off + 32 * nb] = gk;
        reinterpret_cast<float*>(dv_out)[off + 32 * nb] = gv;
      }
    }
  }
}

// --------------------------------------------------------------------------
// dQ.  Stage layout: K and V row-major 32-key tiles, K^T (D x 32, keys
// perm16-ordered).
template <int D>
struct DqCfg {
  using TL = BwdTile<D>;
  static constexpr int OFF_K = 0, OFF_V = TL::RBYTES, OFF_KT = 2 * TL::RBYTES;
  static constexpr int STAGE = 3 * TL::RBYTES;
  static constexpr int LQ = TL::CPR / 8;
  static constexpr int LT = D / 64;
};

// One 32-key tile of a wave in the dQ kernel: S^T = K Q^T, dP^T = V dO^T
// (both windows), dS^T on the vector ALU, dQ^T += K^T dS^T; LDS operands
// read four ahead of their MFMA, as in the dK/dV kernel.
template <int D, bool STUD, bool MASK>
TTCD_DEV void dq_block(uint32_t st, int r32, int h, const bf16x8* qf, const bf16x8* dtf,
                       const bf16x8* dsf, f32x16* acc, int t, int jt, float lt, float ls,
                       float dt, float dsum, int wT, int wS, float c2, bool tmask, bool smask) {
  using TL = BwdTile<D>;
  using CF = DqCfg<D>;
  constexpr int KSTEP = TL::KSTEP, NB = TL::NB;
  constexpr int NA = (STUD ? 3 : 2) * KSTEP;
  auto aaddr = [&](int i) {
    const int c = i / KSTEP, ks = i % KSTEP;
    return TL::rfrag(st + (c == 0 ? CF::OFF_K : CF::OFF_V), r32, ks, h);
  };
  f32x16 sacc[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) sacc[c] = zero16();
  bf16x8 fa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[i] = as_bf16x8(lds_rd16(aaddr(i)));
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int c = i / KSTEP, ks = i % KSTEP;
    sacc[c] = mfma32(fa[i & 3], c == 0 ? qf[ks] : (c == 1 ? dtf[ks] : dsf[ks]), sacc[c]);
    __builtin_amdgcn_sched_barrier(0);
    if (i + 4 < NA) fa[i & 3] = as_bf16x8(lds_rd16(aaddr(i + 4)));
    __builtin_amdgcn_sched_barrier(0);
  }
  // lane (r32, h) holds row t and keys jt + 4 h + 8 (v / 4) + v % 4
  bf16x8 da[2];
#pragma unroll
  for (int vv = 0; vv < 16; ++vv) {
    const int dl = t - (jt + 4 * h + 8 * (vv >> 2) + (vv & 3));
    float pt = fast_exp2(__builtin_fmaf(sacc[0][vv], c2, -lt));
    if (MASK && tmask && !(dl >= 0 && dl < wT)) pt = 0.f;
    float dsv = pt * (sacc[1][vv] - dt);
    if (STUD) {
      float ps = fast_exp2(__builtin_fmaf(sacc[0][vv], c2, -ls));
      if (MASK && smask && !(dl >= 0 && dl < wS)) ps = 0.f;
      dsv = __builtin_fmaf(ps, sacc[2][vv] - dsum, dsv);
    }
    da[vv >> 3][vv & 7] = (__bf16)dsv;
  }
  // dQ^T += K^T dS^T: item i = (column block i / 2, k-step i % 2)
  constexpr int NBK = NB * 2;
  auto baddr = [&](int i) { return TL::tfrag(st + CF::OFF_KT, 32 * (i >> 1) + r32, i & 1, h); };
  bf16x8 fb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) fb[i] = as_bf16x8(lds_rd16(baddr(i)));
#pragma unroll
  for (int i = 0; i < NBK; ++i) {
    acc[i >> 1] = mfma32(fb[i & 3], da[i & 1], acc[i >> 1]);
    __builtin_amdgcn_sched_barrier(0);
    if (i + 4 < NBK) fb[i & 3] = as_bf16x8(lds_rd16(baddr(i + 4)));
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D>
__global__ void __launch_bounds__(256)
attn_bwd_dq_mfma(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                 const bf16_t* __restrict__ v, const bf16_t* __restrict__ dot,
                 const bf16_t* __restrict__ dos, const bf16_t* __restrict__ kT,
                 const float* __restrict__ meta, void* __restrict__ dq_out, int out_bf16, int Tn,
                 int Hq, int Hkv, long ldK, int nmeta, int wT, int wS, float c2, float scale,
                 int nblk, int gshift) {
  using TL = BwdTile<D>;
  using CF = DqCfg<D>;
  constexpr int NB = TL::NB, KSTEP = TL::KSTEP, CPR = TL::CPR;
  extern __shared__ __align__(16) char lds[];
  const int G = Hq / Hkv;
  const int R = Tn * G;
  const uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int blk = nblk - 1 - (int)(lid % nblk);
  const int bg = (int)(lid / nblk);
  const int g = bg % Hkv, b = bg / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, r32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row0 = blk * 128;
  const int rw0 = row0 + 32 * wave;
  const int r = rw0 + r32;
  const bool row_ok = r < R;
  const int rc = min(r, R - 1);
  const int t = row_pos(rc, G, gshift);
  const int hq = g * G + (rc - t * G);

  // this lane's query row: the B operands of S^T = K Q^T and dP^T = V dO^T
  bf16x8 qf[KSTEP], dtf[KSTEP], dsf[KSTEP];
  {
    const size_t off = ((size_t)(b * Tn + t) * Hq + hq) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < KSTEP; ++s) {
      qf[s] = as_bf16x8(ld16(q + off + 16 * s));
      dtf[s] = as_bf16x8(ld16(dot + off + 16 * s));
      dsf[s] = as_bf16x8(ld16(dos + off + 16 * s));
    }
  }
  const float* mrow = meta + ((size_t)bg * nmeta + rc / 32) * 128 + rc % 32;
  const float lt = mrow[0], ls = mrow[32], dt = mrow[64], dsum = mrow[96];
  f32x16 acc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) acc[i] = zero16();
  // drain those loads here (see the dK/dV kernel)
  __builtin_amdgcn_s_waitcnt(0);

  // key tiles of the workgroup, oldest first
  const int A = row_pos(min(row0, R - 1), G, gshift);
  const int Bp = row_pos(min(row0 + 127, R - 1), G, gshift);
  const int jlo = max(0, A - wT + 1) & ~31;
  const int ntile = (Bp - jlo) / 32 + 1;
  const int a_w = row_pos(min(rw0, R - 1), G, gshift);
  const int b_w = row_pos(min(rw0 + 31, R - 1), G, gshift);

  int kx[CF::LQ], kgc[CF::LQ];
#pragma unroll
  for (int u = 0; u < CF::LQ; ++u) {
    const int p = (u * 4 + wave) * 64 + lane;
    kx[u] = p / CPR;
    kgc[u] = (p % CPR) ^ TL::rswz(kx[u]);
  }
  int td[CF::LT], tgc[CF::LT];
#pragma unroll
  for (int u = 0; u < CF::LT; ++u) {
    const int p = (u * 4 + wave) * 64 + lane;
    td[u] = p / 4;
    tgc[u] = (p % 4) ^ TL::tswz(td[u]);
  }
  const size_t tbase = (size_t)bg * D * ldK;
  auto issue = [&](int i) {
    const int jt = jlo + 32 * i;
    char* st = lds + (i & 1) * CF::STAGE;
#pragma unroll
    for (int u = 0; u < CF::LQ; ++u) {
      const int j = min(jt + kx[u], Tn - 1);
      const size_t off = ((size_t)(b * Tn + j) * Hkv + g) * D + kgc[u] * 8;
      char* dst = st + (u * 4 + wave) * 1024;
      dma16(k + off, dst + CF::OFF_K);
      dma16(v + off, dst + CF::OFF_V);
    }
#pragma unroll
    for (int u = 0; u < CF::LT; ++u)
      dma16(kT + tbase + (size_t)td[u] * ldK + jt + tgc[u] * 8,
            st + (u * 4 + wave) * 1024 + CF::OFF_KT);
  };

  issue(0);
  stage_barrier();
#pragma unroll 1
  for (int i = 0; i < ntile; ++i) {
    if (i + 1 < ntile) issue(i + 1);
    const int jt = jlo + 32 * i;
    const uint32_t st = (uint32_t)((i & 1) * CF::STAGE);
    const BlockKind bk = block_kind(a_w - (jt + 31), b_w - jt, wT, wS);
    if (bk.act) {
#define TTCD_DQ(S, M) \
  dq_block<D, S, M>(st, r32, h, qf, dtf, dsf, acc, t, jt, lt, ls, dt, dsum, wT, wS, c2, \
                    bk.tmask, bk.smask)
      const bool msk = bk.tmask || (bk.stud && bk.smask);
      if (bk.stud) {
        if (msk) TTCD_DQ(true, true); else TTCD_DQ(true, false);
      } else {
        if (msk) TTCD_DQ(false, true); else TTCD_DQ(false, false);
      }
#undef TTCD_DQ
    }
    stage_barrier();
  }

  if (!row_ok) return;
  // lane (r32, h) holds dims 32 nb + 8 g4 + 4 h + e of its row
  const size_t obase = ((size_t)(b * Tn + t) * Hq + hq) * D;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = 32 * nb + 8 * g4 + 4 * h;
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = acc[nb][4 * g4 + e] * scale;
      if (out_bf16)
        *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(dq_out) + obase + d) =
            u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      else
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(dq_out) + obase + d) =
            f32x4{o[0], o[1], o[2], o[3]};
    }
  }
}

// --------------------------------------------------------------------------
// Plain kernels (fp32 inputs, or head dims the MFMA kernels do not cover):
// one thread per query row for dQ, one per key for dK and dV, exact fp32.
template <typename T, int D>
__global__ void __launch_bounds__(64)
attn_bwd_dq_simple(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                   const T* __restrict__ dot, const T* __restrict__ dos,
                   const float* __restrict__ meta, void* __restrict__ dq_out, int out_bf16,
                   int Tn, int Hq, int Hkv, int nmeta, int wT, int wS, float c2, float scale) {
  const int G = Hq / Hkv;
  const int R = Tn * G;
  const long id = (long)blockIdx.x * 64 + threadIdx.x;
  const int bg = blockIdx.y;
  const int g = bg % Hkv, b = bg / Hkv;
  if (id >= R) return;
  const int x = (int)id;
  const int t = x / G, hq = g * G + x % G;
  const size_t off = ((size_t)(b * Tn + t) * Hq + hq) * D;
  const float* m = meta + ((size_t)bg * nmeta + x / 32) * 128 + x % 32;
  const float lt = m[0], ls = m[32], dt = m[64], dsum = m[96];
  float acc[D];
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  for (int j = max(0, t - wT + 1); j <= t; ++j) {
    const size_t ko = ((size_t)(b * Tn + j) * Hkv + g) * D;
    float s = 0.f, dpt = 0.f, dps = 0.f;
    for (int d = 0; d < D; ++d) {
      const float vv = ldf(v + ko + d);
      s = __builtin_fmaf(ldf(q + off + d), ldf(k + ko + d), s);
      dpt = __builtin_fmaf(ldf(dot + off + d), vv, dpt);
      dps = __builtin_fmaf(ldf(dos + off + d), vv, dps);
    }
    float ds = exp2f(s * c2 - lt) * (dpt - dt);
    if (t - j < wS) ds += exp2f(s * c2 - ls) * (dps - dsum);
    for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(ds, ldf(k + ko + d), acc[d]);
  }
  for (int d = 0; d < D; ++d) {
    if (out_bf16)
      reinterpret_cast<bf16_t*>(dq_out)[off + d] = f2bf(acc[d] * scale);
    else
      reinterpret_cast<float*>(dq_out)[off + d] = acc[d] * scale;
  }
}

template <typename T, int D>
__global__ void __launch_bounds__(64)
attn_bwd_dkdv_simple(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                     const T* __restrict__ dot, const T* __restrict__ dos,
                     const float* __restrict__ meta, void* __restrict__ dk_out,
                     void* __restrict__ dv_out, int out_bf16, int Tn, int Hq, int Hkv, int nmeta,
                     int wT, int wS, float c2, float scale) {
  const int G = Hq / Hkv;
  const long j = (long)blockIdx.x * 64 + threadIdx.x;
  const int bg = blockIdx.y;
  const int g = bg % Hkv, b = bg / Hkv;
  if (j >= Tn) return;
  const size_t ko = ((size_t)(b * Tn + j) * Hkv + g) * D;
  float gk[D], gv[D];
  for (int d = 0; d < D; ++d) gk[d] = gv[d] = 0.f;
  const int tend = (int)min((long)Tn, j + wT);
  for (int t = (int)j; t < tend; ++t) {
    for (int hh = 0; hh < G; ++hh) {
      const int x = t * G + hh;
      const size_t off = ((size_t)(b * Tn + t) * Hq + g * G + hh) * D;
      const float* m = meta + ((size_t)bg * nmeta + x / 32) * 128 + x % 32;
      float s = 0.f, dpt = 0.f, dps = 0.f;
      for (int d = 0; d < D; ++d) {
        const float vv = ldf(v + ko + d);
        s = __builtin_fmaf(ldf(q + off + d), ldf(k + ko + d), s);
        dpt = __builtin_fmaf(ldf(dot + off + d), vv, dpt);
        dps = __builtin_fmaf(ldf(dos + off + d), vv, dps);
      }
      const bool stud = t - j < wS;
      const float pt = exp2f(s * c2 - m[0]);
      const float ps = stud ? exp2f(s * c2 - m[32]) : 0.f;
      const float ds = pt * (dpt - m[64]) + ps * (dps - m[96]);
      for (int d = 0; d < D; ++d) {
        gv[d] = __builtin_fmaf(pt, ldf(dot + off + d), gv[d]);
        gv[d] = __builtin_fmaf(ps, ldf(dos + off + d), gv[d]);
        gk[d] = __builtin_fmaf(ds, ldf(q + off + d), gk[d]);
      }
    }
  }
  for (int d = 0; d < D; ++d) {
    if (out_bf16) {
      reinterpret_cast<bf16_t*>(dk_out)[ko + d] = f2bf(gk[d] * scale);
      reinterpret_cast<bf16_t*>(dv_out)[ko + d] = f2bf(gv[d]);
    } else {
      reinterpret_cast<float*>(dk_out)[ko + d] = gk[d] * scale;
      reinterpret_cast<float*>(dv_out)[ko + d] = gv[d];
    }
  }
}

int log2_exact(int G) {
  for (int s = 0; s < 31; ++s)
    if ((1 << s) == G) return s;
  return -1;
}

template <typename KERN>
hipError_t set_lds(KERN kern, size_t bytes) {
  return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

template <int D>
hipError_t launch_bwd_mfma(const AttnBwdArgs& a, const AttnBwdBufs& w, float c2, float scale,
                           int gshift, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const long R = (long)a.T * G;
  const int nmeta = attn_bwd_meta_blocks(a.T, G);
  const int out_bf16 = a.out_dt == BF16 ? 1 : 0;
  // transposed copies: Q, dO_T, dO_S per kv group (rows = query rows), K
  const long ldR = (long)(nmeta - 1) * 32;
  const long ldK = attn_bwd_key_ld(a.T);
  {
    dim3 grid((unsigned)(ldR / 64), a.D / 64, a.B * a.Hkv);
    hipLaunchKernelGGL(rows_transpose_kernel, grid, dim3(256), 0, s, (const uint16_t*)a.q,
                       (uint16_t*)w.qT, a.T, a.Hq, a.Hkv, a.D, (int)R, ldR);
    hipLaunchKernelGGL(rows_transpose_kernel, grid, dim3(256), 0, s, (const uint16_t*)a.do_t,
                       (uint16_t*)w.dotT, a.T, a.Hq, a.Hkv, a.D, (int)R, ldR);
    hipLaunchKernelGGL(rows_transpose_kernel, grid, dim3(256), 0, s, (const uint16_t*)a.do_s,
                       (uint16_t*)w.dosT, a.T, a.Hq, a.Hkv, a.D, (int)R, ldR);
    dim3 gk((unsigned)(ldK / 64), a.D / 64, a.B * a.Hkv);
    hipLaunchKernelGGL(rows_transpose_kernel, gk, dim3(256), 0, s, (const uint16_t*)a.k,
                       (uint16_t*)w.kT, a.T, a.Hkv, a.Hkv, a.D, a.T, ldK);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    using CF = DkdvCfg<D>;
    const size_t lds = 2 * (size_t)CF::STAGE;
    static hipError_t attr = set_lds(attn_bwd_dkdv_mfma<D>, lds);
    if (attr != hipSuccess) return attr;
    const int nkb = (a.T + 127) / 128;
    hipLaunchKernelGGL((attn_bwd_dkdv_mfma<D>), dim3((unsigned)((long)a.B * a.Hkv * nkb)),
                       dim3(256), lds, s, (const bf16_t*)a.q, (const bf16_t*)a.k,
                       (const bf16_t*)a.v, (const bf16_t*)a.do_t, (const bf16_t*)a.do_s,
                       (const bf16_t*)w.qT, (const bf16_t*)w.dotT, (const bf16_t*)w.dosT, w.meta,
                       a.dk, a.dv, out_bf16, a.T, a.Hq, a.Hkv, ldR, nmeta, a.wT, a.wS, c2, scale,
                       nkb, gshift);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    using CF = DqCfg<D>;
    const size_t lds = 2 * (size_t)CF::STAGE;
    static hipError_t attr = set_lds(attn_bwd_dq_mfma<D>, lds);
    if (attr != hipSuccess) return attr;
    const int nblk = (int)((R + 127) / 128);
    hipLaunchKernelGGL((attn_bwd_dq_mfma<D>), dim3((unsigned)((long)a.B * a.Hkv * nblk)),
                       dim3(256), lds, s, (const bf16_t*)a.q, (const bf16_t*)a.k,
                       (const bf16_t*)a.v, (const bf16_t*)a.do_t, (const bf16_t*)a.do_s,
                       (const bf16_t*)w.kT, w.meta, a.dq, out_bf16, a.T, a.Hq, a.Hkv, ldK, nmeta,
                       a.wT, a.wS, c2, scale, nblk, gshift);
    return hipGetLastError();
  }
}

template <typename T, int D>
hipError_t launch_bwd_simple(const AttnBwdArgs& a, const AttnBwdBufs& w, float c2, float scale,
                             hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const long R = (long)a.T * G;
  const int nmeta = attn_bwd_meta_blocks(a.T, G);
  const int out_bf16 = a.out_dt == BF16 ? 1 : 0;
  hipLaunchKernelGGL((attn_bwd_dq_simple<T, D>), dim3((unsigned)((R + 63) / 64), a.B * a.Hkv),
                     dim3(64), 0, s, (const T*)a.q, (const T*)a.k, (const T*)a.v,
                     (const T*)a.do_t, (const T*)a.do_s, w.meta, a.dq, out_bf16, a.T, a.Hq, a.Hkv,
                     nmeta, a.wT, a.wS, c2, scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dkdv_simple<T, D>), dim3((unsigned)((a.T + 63) / 64), a.B * a.Hkv),
                     dim3(64), 0, s, (const T*)a.q, (const T*)a.k, (const T*)a.v,
                     (const T*)a.do_t, (const T*)a.do_s, w.meta, a.dk, a.dv, out_bf16, a.T, a.Hq,
                     a.Hkv, nmeta, a.wT, a.wS, c2, scale);
  return hipGetLastError();
}

}  // namespace

int attn_bwd_meta_blocks(int T, int G) { return (int)(((long)T * G + 63) / 64 * 2) + 1; }

long attn_bwd_key_ld(int T) { return ((long)T + 63) / 64 * 64; }

size_t attn_bwd_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int in_dt) {
  const int G = Hq / Hkv;
  const int nmeta = attn_bwd_meta_blocks(T, G);
  size_t n = (size_t)B * Hkv * nmeta * 128 * sizeof(float);
  n = (n + 255) / 256 * 256;
  if (in_dt == BF16 && (D == 64 || D == 128)) {
    const size_t rows = (size_t)(nmeta - 1) * 32;
    n += 3 * ((size_t)B * Hkv * D * rows * 2 + 255) / 256 * 256;
    n += ((size_t)B * Hkv * D * attn_bwd_key_ld(T) * 2 + 255) / 256 * 256;
  }
  return n;
}

void attn_bwd_plan(const AttnBwdArgs& a, char* ws, AttnBwdBufs& w) {
  const int G = a.Hq / a.Hkv;
  const int nmeta = attn_bwd_meta_blocks(a.T, G);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = ws + off;
    off += (bytes + 255) / 256 * 256;
    return (void*)p;
  };
  w.meta = (float*)take((size_t)a.B * a.Hkv * nmeta * 128 * sizeof(float));
  w.qT = w.dotT = w.dosT = w.kT = nullptr;
  if (a.in_dt == BF16 && (a.D == 64 || a.D == 128)) {
    const size_t rows = (size_t)(nmeta - 1) * 32;
    w.qT = take((size_t)a.B * a.Hkv * a.D * rows * 2);
    w.dotT = take((size_t)a.B * a.Hkv * a.D * rows * 2);
    w.dosT = take((size_t)a.B * a.Hkv * a.D * rows * 2);
    w.kT = take((size_t)a.B * a.Hkv * a.D * attn_bwd_key_ld(a.T) * 2);
  }
}

hipError_t launch_dual_window_attn_backward(const AttnBwdArgs& a, const AttnBwdBufs& w,
                                            hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int nmeta = attn_bwd_meta_blocks(a.T, G);
  const float c2 = a.scale * LOG2E;
  {
    const long nrows = (long)a.B * a.Hkv * nmeta * 32;
    dim3 grid((unsigned)((nrows + 3) / 4));
    if (a.in_dt == BF16 && (a.D == 64 || a.D == 128)) {
      const int rows_per_block = 4 * (64 / (a.D / 8));
      const dim3 vgrid((unsigned)((nrows + rows_per_block - 1) / rows_per_block));
      if (a.D == 64)
        hipLaunchKernelGGL(attn_bwd_meta_vec_kernel<64>, vgrid, dim3(256), 0, s,
                           (const bf16_t*)a.o_t, (const bf16_t*)a.o_s, (const bf16_t*)a.do_t,
                           (const bf16_t*)a.do_s, a.lse_t, a.lse_s, w.meta, a.T, a.Hq, a.Hkv,
                           nmeta, nrows);
      else
        hipLaunchKernelGGL(attn_bwd_meta_vec_kernel<128>, vgrid, dim3(256), 0, s,
                           (const bf16_t*)a.o_t, (const bf16_t*)a.o_s, (const bf16_t*)a.do_t,
                           (const bf16_t*)a.do_s, a.lse_t, a.lse_s, w.meta, a.T, a.Hq, a.Hkv,
                           nmeta, nrows);
    } else if (a.in_dt == BF16)
      hipLaunchKernelGGL(attn_bwd_meta_kernel<bf16_t>, grid, dim3(256), 0, s,
                         (const bf16_t*)a.o_t, (const bf16_t*)a.o_s, (const bf16_t*)a.do_t,
                         (const bf16_t*)a.do_s, a.lse_t, a.lse_s, w.meta, a.T, a.Hq, a.Hkv, a.D,
                         nmeta, nrows);
    else
      hipLaunchKernelGGL(attn_bwd_meta_kernel<float>, grid, dim3(256), 0, s,
                         (const float*)a.o_t, (const float*)a.o_s, (const float*)a.do_t,
                         (const float*)a.do_s, a.lse_t, a.lse_s, w.meta, a.T, a.Hq, a.Hkv, a.D,
                         nmeta, nrows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.in_dt == BF16 && (a.D == 64 || a.D == 128)) {
    const int gshift = log2_exact(G);
    return a.D == 64 ? launch_bwd_mfma<64>(a, w, c2, a.scale, gshift, s)
                     : launch_bwd_mfma<128>(a, w, c2, a.scale, gshift, s);
  }
  if (a.in_dt == BF16)
    return a.D == 64 ? launch_bwd_simple<bf16_t, 64>(a, w, c2, a.scale, s)
                     : launch_bwd_simple<bf16_t, 128>(a, w, c2, a.scale, s);
  return a.D == 64 ? launch_bwd_simple<float, 64>(a, w, c2, a.scale, s)
                   : launch_bwd_simple<float, 128>(a, w, c2, a.scale, s);
}

}  // namespace ttcd
