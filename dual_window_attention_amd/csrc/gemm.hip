// Dense contractions of the IP-TTCD layer on gfx950:
//   C = A B^T with A [M, K] and B [N, K] both K-contiguous ("NT"), bf16 in,
//   fp32 MFMA accumulate, with fused epilogues (residual add, SwiGLU,
//   per-column scale, chunk-indexed weights).  The chunk writes of the fast
//   weight (papernotes.org notes on "Learning What to Remember", key design
//   3: dW_i = beta_i R_i K_i^T) are one batched call over the chunks.
#include <algorithm>
#include <cstdlib>

#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace ttcd {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LS = BK + 8;                     // LDS row stride (bf16)
constexpr int TILE = BM * LS;                  // one operand tile
constexpr size_t GEMM_LDS = 2 * 2 * TILE * sizeof(bf16_t);   // 2 stages x (A, B)
constexpr int NT = 256;

struct Tile {
  f32x16 acc[2][2];
};

// Loads one BK slice of a 128-row operand into registers.
// rows: [r0, r0+128) of src (row stride ld), k in [k0, k0+64) limited to
// [kbeg, kend); rows >= rlim are zero.  rowmap optionally redirects rows
// 64..127 to a second matrix (SwiGLU up-projection).
struct OpLoad {
  u32x4 v[4];
  TTCD_DEV void load(const bf16_t* src, const bf16_t* src2, long ld, long r0, long rlim,
                     long k0, long kend, int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * NT;
      const int row = c >> 3, kc = c & 7;
      const long k = k0 + kc * 8;
      u32x4 val = {0u, 0u, 0u, 0u};
      const bf16_t* s = src;
      long rr = r0 + row;
      if (src2 && row >= 64) {
        s = src2;
        rr = r0 + row - 64;
      }
      if (rr < rlim && k < kend) val = ld16(s + rr * ld + k);
      v[i] = val;
    }
  }
  TTCD_DEV void store(bf16_t* dst, int tid) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * NT;
      const int row = c >> 3, kc = c & 7;
      st16(dst + row * LS + kc * 8, v[i]);
    }
  }
};

// acc += A[m0:m0+128, kbeg:kend] * B[n0:n0+128, kbeg:kend]^T
// brow_of(bn) gives the LDS row block of B used for output block bn.
TTCD_DEV void mainloop(Tile& t, const bf16_t* A, long lda, long m0, long mlim,
                       const bf16_t* Bp, const bf16_t* Bp2, long ldb, long n0, long nlim,
                       long kbeg, long kend, bf16_t* lds, int brow0, int brow1) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1;
  const int h = lane >> 5, r = lane & 31;
  const int nk = (int)((kend - kbeg + BK - 1) / BK);
  if (nk <= 0) return;
  OpLoad la, lb;
  la.load(A, nullptr, lda, m0, mlim, kbeg, kend, tid);
  lb.load(Bp, Bp2, ldb, n0, nlim, kbeg, kend, tid);
  la.store(lds, tid);
  lb.store(lds + TILE, tid);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool nxt = kt + 1 < nk;
    if (nxt) {
      const long k0 = kbeg + (long)(kt + 1) * BK;
      la.load(A, nullptr, lda, m0, mlim, k0, kend, tid);
      lb.load(Bp, Bp2, ldb, n0, nlim, k0, kend, tid);
    }
    const bf16_t* al = lds + cur * 2 * TILE;
    const bf16_t* bl = al + TILE;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const bf16x8 a0 = as_bf16x8(ld16(al + (64 * wm + r) * LS + 16 * s + 8 * h));
      const bf16x8 a1 = as_bf16x8(ld16(al + (64 * wm + 32 + r) * LS + 16 * s + 8 * h));
      const bf16x8 b0 = as_bf16x8(ld16(bl + (brow0 + r) * LS + 16 * s + 8 * h));
      const bf16x8 b1 = as_bf16x8(ld16(bl + (brow1 + r) * LS + 16 * s + 8 * h));
      t.acc[0][0] = mfma32(a0, b0, t.acc[0][0]);
      t.acc[0][1] = mfma32(a0, b1, t.acc[0][1]);
      t.acc[1][0] = mfma32(a1, b0, t.acc[1][0]);
      t.acc[1][1] = mfma32(a1, b1, t.acc[1][1]);
    }
    if (nxt) {
      bf16_t* nl = lds + (cur ^ 1) * 2 * TILE;
      la.store(nl, tid);
      lb.store(nl + TILE, tid);
    }
    __syncthreads();
  }
}

// silu(a) = a / (1 + e^-a) with the hardware reciprocal (about 1 ulp)
// rather than the correctly rounded division sequence; e^-a -> inf for very
// negative a gives rcp = 0 and silu = -0
TTCD_DEV float silu(float a) {
  return a * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * a));
}

template <typename OutT>
__global__ void __launch_bounds__(NT, 2)
gemm_nt_mfma(GemmArgs g) {
  extern __shared__ __align__(16) bf16_t lds[];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, r = lane & 31;
  const int z = blockIdx.z;
  const int ncol_tiles = gridDim.y;
  const uint32_t tiles = gridDim.x * ncol_tiles;
  const uint32_t lid = xcd_remap(blockIdx.y * gridDim.x + blockIdx.x, tiles);
  const long m0 = (long)(lid / ncol_tiles) * BM;
  const bool swiglu = g.epi == EPI_SWIGLU;
  const long ncols_tile = swiglu ? 64 : BN;
  const long n0 = (long)(lid % ncol_tiles) * ncols_tile;

  const bf16_t* A = (const bf16_t*)g.A + z * g.sA;
  const bf16_t* Bm = (const bf16_t*)g.B + z * g.sB;
  const bf16_t* B2 = g.B2 ? (const bf16_t*)g.B2 + z * g.sB : nullptr;
  if (g.chunk > 0) {
    const long c = m0 / g.chunk;
    if (c > 0) Bm = (const bf16_t*)g.Bchunks + z * g.sBchunksBatch + (c - 1) * g.sBchunk;
  }
  int brow0, brow1;
  if (swiglu) {
    brow0 = 32 * wn;
    brow1 = 64 + 32 * wn;
  } else {
    brow0 = 64 * wn;
    brow1 = 64 * wn + 32;
  }
  Tile t;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) t.acc[i][j] = zero16();

  mainloop(t, A, g.lda, m0, g.M, Bm, B2, g.ldb, n0, g.N, 0, g.K, lds, brow0, brow1);

  OutT* C = (OutT*)g.C + z * g.sC;
  if (swiglu) {
    const long n = n0 + 32 * wn + r;
    if (n >= g.N) return;
#pragma unroll
    for (int bm = 0; bm < 2; ++bm)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const long m = m0 + 64 * wm + 32 * bm + 8 * (v >> 2) + 4 * h + (v & 3);
        if (m < g.M) stf(C + m * g.ldc + n, silu(t.acc[bm][0][v]) * t.acc[bm][1][v]);
      }
    return;
  }
#pragma unroll
  for (int bn = 0; bn < 2; ++bn) {
    const long n = n0 + 64 * wn + 32 * bn + r;
    if (n >= g.N) continue;
    float cs = 1.f;
    if (g.epi == EPI_STORE && g.colscale) cs = g.colscale[z * g.sScale + n];
#pragma unroll
    for (int bm = 0; bm < 2; ++bm)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const long m = m0 + 64 * wm + 32 * bm + 8 * (v >> 2) + 4 * h + (v & 3);
        if (m >= g.M) continue;
        float val = t.acc[bm][bn][v];
        if (g.epi == EPI_RESIDUAL) {
          const long rm = (m % g.res_rows) * g.ldr + n + z * g.sRes;
          val += g.res_dt == BF16 ? bf2f(((const bf16_t*)g.res)[rm]) : ((const float*)g.res)[rm];
        } else {
          val *= cs;
        }
        stf(C + m * g.ldc + n, val);
      }
  }
}

// --------------------------------------------------------------------------
// Plain tiled FMA kernels (fp32 inputs, shapes the MFMA path does not take)
// --------------------------------------------------------------------------
constexpr int SB = 64, SK = 16;

template <typename InT>
TTCD_DEV void simple_tile(float (&acc)[4][4], float (&acc2)[4][4], const InT* A, long lda,
                          long m0, long M, const InT* Bm, const InT* B2, long ldb, long n0,
                          long N, long kbeg, long kend) {
  __shared__ float As[SK][SB + 1];
  __shared__ float Bs[SK][SB + 1];
  __shared__ float B2s[SK][SB + 1];
  const int tid = threadIdx.x;
  const int tr = tid / 16, tc = tid % 16;
  for (long k0 = kbeg; k0 < kend; k0 += SK) {
    __syncthreads();
    for (int e = tid; e < SK * SB; e += 256) {
      const int row = e / SK, kk = e % SK;
      const long k = k0 + kk;
      const bool kok = k < kend;
      As[kk][row] = (m0 + row < M && kok) ? ldf(A + (m0 + row) * lda + k) : 0.f;
      Bs[kk][row] = (n0 + row < N && kok) ? ldf(Bm + (n0 + row) * ldb + k) : 0.f;
      if (B2) B2s[kk][row] = (n0 + row < N && kok) ? ldf(B2 + (n0 + row) * ldb + k) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < SK; ++kk) {
      float av[4], bv[4], b2v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = As[kk][tr * 4 + i];
        bv[i] = Bs[kk][tc * 4 + i];
        b2v[i] = B2 ? B2s[kk][tc * 4 + i] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
          if (B2) acc2[i][j] = __builtin_fmaf(av[i], b2v[j], acc2[i][j]);
        }
    }
  }
}

template <typename InT, typename OutT>
__global__ void __launch_bounds__(256) gemm_nt_simple(GemmArgs g) {
  const int z = blockIdx.z;
  const long m0 = (long)blockIdx.x * SB, n0 = (long)blockIdx.y * SB;
  const InT* A = (const InT*)g.A + z * g.sA;
  const InT* Bm = (const InT*)g.B + z * g.sB;
  const InT* B2 = g.B2 ? (const InT*)g.B2 + z * g.sB : nullptr;
  if (g.chunk > 0) {
    const long c = m0 / g.chunk;
    if (c > 0) Bm = (const InT*)g.Bchunks + z * g.sBchunksBatch + (c - 1) * g.sBchunk;
  }
  float acc[4][4] = {}, acc2[4][4] = {};
  simple_tile<InT>(acc, acc2, A, g.lda, m0, g.M, Bm, B2, g.ldb, n0, g.N, 0, g.K);
  OutT* C = (OutT*)g.C + z * g.sC;
  const int tr = threadIdx.x / 16, tc = threadIdx.x % 16;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long m = m0 + tr * 4 + i, n = n0 + tc * 4 + j;
      if (m >= g.M || n >= g.N) continue;
      float val = acc[i][j];
      if (g.epi == EPI_SWIGLU) {
        val = silu(acc[i][j]) * acc2[i][j];
      } else if (g.epi == EPI_RESIDUAL) {
        const long rm = (m % g.res_rows) * g.ldr + n + z * g.sRes;
        val += g.res_dt == BF16 ? bf2f(((const bf16_t*)g.res)[rm]) : ((const float*)g.res)[rm];
      } else if (g.colscale) {
        val *= g.colscale[z * g.sScale + n];
      }
      stf(C + m * g.ldc + n, val);
    }
}

// --------------------------------------------------------------------------
// Large-tile NT GEMM: 256 x 128 workgroup tile, 4 waves each owning a
// 128 x 64 block (8 MFMAs per 6 KB of LDS operand reads), BK = 32.  Operand
// tiles go straight from global memory into LDS (global_load_lds_dwordx4) in
// an XOR-swizzled layout that keeps the MFMA operand reads nearly free of
// bank conflicts; the ring (2 stages: three workgroups per CU, or 3) is
// fetched one stage less than its depth ahead.  Output tiles are visited in
// 8-row groups per XCD for L2 reuse.  Requires K % 32 == 0 and 16-byte
// aligned rows.
// --------------------------------------------------------------------------
namespace big {
constexpr int BM = 256, BN = 128, BK = 32, NW = 4, NTH = 64 * NW;
constexpr int AB = BM * BK * 2, BB = BN * BK * 2;   // operand bytes per stage
constexpr int STAGE = AB + BB;                       // 24 KB
constexpr size_t lds_bytes(int nst) { return (size_t)nst * STAGE; }
constexpr int ALD = BM * BK / 8 / (64 * NW);         // 16B loads per wave (A)
constexpr int BLD = BN * BK / 8 / (64 * NW);         // 16B loads per wave (B)
constexpr int LPW = ALD + BLD;
constexpr int EPS = 72;                              // epilogue slab row stride (floats)
static_assert(NW * 32 * EPS * 4 <= 3 * STAGE, "epilogue slabs fit in the operand ring");

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// 16 bytes per lane, global -> LDS; lane i lands at lds_wave_base + 16 i.
// Inline asm rather than the compiler builtin: the compiler counts a builtin
// LDS DMA as an LDS operation of unknown order and then waits for every
// outstanding LDS read (lgkmcnt 0) before any MFMA that needs one of them,
// which serialises the fragment reads of the next k-step with the MFMAs of
// this one.  The hardware counts the DMA in vmcnt alone and the loops order
// it explicitly (a vmcnt wait before the barrier that publishes a stage).
// M0 takes the LDS address; one wait state separates its write from the DMA.
TTCD_DEV void g2l16(const void* src, void* lds_wave_base) {
  const uint32_t m = (uint32_t)(size_t)(lds_void_t*)lds_wave_base;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(src), "{m0}"(m) : "memory");
}
// barrier that leaves the in-flight stage fetches alone; every wave waits
// for the stage it needs with wait_vm before it
TTCD_DEV void barrier() { asm volatile("s_barrier" ::: "memory"); }
template <int N>
TTCD_DEV void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// rows of 64 bytes (4 chunks): chunk c of row r lives at c ^ ((r >> 2) & 3)
TTCD_DEV int swz(int row) { return (row >> 2) & 3; }
// the wave's LDS accesses so far are complete (and the compiler may not move
// memory accesses across): enough for lanes of one wave to exchange data
TTCD_DEV void lds_wave_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int NLD, class RowPtr>
TTCD_DEV void issue(char* dst, const RowPtr& row_ptr, long k0, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int p0 = (i * NW + wave) * 64;
    const int p = p0 + lane;
    const int row = p >> 2, cp = p & 3;
    const int c = cp ^ swz(row);
    g2l16(row_ptr(row) + k0 + 8 * c, dst + p0 * 16);
  }
}

// stages still in flight after the one waited for (0, 1 or 2)
TTCD_DEV void wait_pending(int pending) {
  if (pending >= 2)
    wait_vm<2 * LPW>();
  else if (pending == 1)
    wait_vm<LPW>();
  else
    wait_vm<0>();
}

// 3-stage ring (72 KB) fetched two stages ahead: two workgroups share a CU,
// so one's epilogue and stage waits overlap the other's MFMAs.
constexpr int NST = 3;
// CHUNKED: the B operand of output row block m0 is chosen per chunk of rows
// (the fast-weight apply: W_down0 for chunk 0, the state list after it)
template <typename OutT, int EPI, bool CHUNKED>
__global__ void __launch_bounds__(NTH, 2)
gemm_nt_big(GemmArgs g) {
  extern __shared__ __align__(16) char lds[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, r = lane & 31;
  const int z = blockIdx.z;
  constexpr bool swiglu = EPI == EPI_SWIGLU;
  const int ncols = swiglu ? BN / 2 : BN;                   // output columns per tile
  const int ntn = (g.N + ncols - 1) / ncols;
  const int ntm = (g.M + BM - 1) / BM;
  const uint32_t lid = xcd_remap(blockIdx.x, (uint32_t)(ntm * ntn));
  int tm, tn;
  grouped_tile(lid, ntm, ntn, 8, tm, tn);
  const long m0 = (long)tm * BM;
  const long n0 = (long)tn * ncols;

  const bf16_t* A = (const bf16_t*)g.A + z * g.sA;
  const bf16_t* Bm = (const bf16_t*)g.B + z * g.sB;
  const bf16_t* B2 = g.B2 ? (const bf16_t*)g.B2 + z * g.sB : nullptr;
  if constexpr (CHUNKED) {
    const long c = m0 / g.chunk;
    if (c > 0) Bm = (const bf16_t*)g.Bchunks + z * g.sBchunksBatch + (c - 1) * g.sBchunk;
  }
  const long mmax = g.M - 1, nmax = g.N - 1;
  const long lda = g.lda, ldb = g.ldb;
  // (captured by value: by reference, the two B pointers land in a stack
  // array whose scratch load would wait on every prefetch in flight)
  auto a_row = [=](int rr) { return A + min(m0 + rr, mmax) * lda; };
  const long b2_off = swiglu ? (long)(B2 - Bm) : 0;   // up rows relative to gate rows
  auto b_row = [=](int rr) {
    if (swiglu) {
      // LDS row blocks of 32 alternate gate / up for the same 32 columns
      const int blk = rr >> 5;
      const long col = min(n0 + 32 * (blk >> 1) + (rr & 31), nmax);
      return Bm + ((blk & 1) ? b2_off : 0) + col * ldb;
    }
    return Bm + min(n0 + rr, nmax) * ldb;
  };
  auto fetch = [=](int kt) {
    char* st = lds + (kt % NST) * STAGE;
    issue<ALD>(st, a_row, (long)kt * BK, wave, lane);
    issue<BLD>(st + AB, b_row, (long)kt * BK, wave, lane);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = zero16();

  const int nk = g.K / BK;
  const int npro = nk < NST - 1 ? nk : NST - 1;
  for (int kt = 0; kt < npro; ++kt) fetch(kt);
  wait_pending(npro - 1);
  barrier();
  // MFMA operand fragments of k-step ks (16 wide) of the stage at as
  struct Frag {
    bf16x8 a[4], b[2];
  };
  auto ldfrag = [&](const char* as, int ks, Frag& f) __attribute__((always_inline)) {
    const char* bs = as + AB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 128 * wm + 32 * i + r;
      f.a[i] = as_bf16x8(ld16(as + row * (BK * 2) + (((2 * ks + h) ^ swz(row)) << 4)));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = 64 * wn + 32 * j + r;
      f.b[j] = as_bf16x8(ld16(bs + row * (BK * 2) + (((2 * ks + h) ^ swz(row)) << 4)));
    }
  };
  auto mma = [&](const Frag& f) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(f.a[i], f.b[j], acc[i][j]);
  };
  // Software pipeline: the second k-step's fragments are read while the
  // first k-step's MFMAs run, the next stage's first fragments while the
  // second k-step's run.
  Frag f0, f1;
  ldfrag(lds, 0, f0);
  // drain the scalar loads of the set-up, so that inside the loop the LDS
  // counter holds fragment reads alone and the compiler can wait for the
  // older fragment set while the newer one is still in flight
  __builtin_amdgcn_s_waitcnt(0xC07F);    // lgkmcnt(0)
  for (int kt = 0; kt < nk; ++kt) {
    // the slot refilled here held stage kt-1; every wave finished reading it
    // before the barrier that ended the previous iteration
    if (kt + NST - 1 < nk) fetch(kt + NST - 1);
    const char* as = lds + (kt % NST) * STAGE;
    ldfrag(as, 1, f1);
    __builtin_amdgcn_sched_barrier(0);
    mma(f0);
    __builtin_amdgcn_sched_barrier(0);
    // stage kt+1 must have landed (later ones may still be in flight), and
    // this wave's reads of stage kt are complete before the barrier
    const int last = kt + NST - 1 < nk ? kt + NST - 1 : nk - 1;
    lds_wave_sync();
    wait_pending(last - (kt + 1));
    barrier();
    // (after the last stage this reads a slot nobody uses; it stays in bounds)
    ldfrag(lds + ((kt + 1) % NST) * STAGE, 0, f0);
    __builtin_amdgcn_sched_barrier(0);
    mma(f1);
    __builtin_amdgcn_sched_barrier(0);
  }
  // every wave's last MFMAs are done reading the ring before the epilogue
  // reuses it as slabs
  lds_wave_sync();
  barrier();

  // Epilogue through a wave-private LDS slab (the operand ring is idle after
  // the last barrier): one 32-row block row of the wave's tile at a time is
  // written as the MFMA layout leaves it and read back row-major, so each
  // lane stores 16 bytes of consecutive columns and loads the residual the
  // same way.  Tiles fully inside C skip the per-element bounds checks.
  OutT* C = (OutT*)g.C + z * g.sC;
  float* slab = reinterpret_cast<float*>(lds) + wave * (32 * EPS);
  constexpr int ocols = swiglu ? 32 : 64;             // output columns of the wave
  constexpr int per_row = ocols / 4;                  // 4-column pieces per row
  constexpr int npieces = 32 * per_row;               // per 32-row block
  const long nw0 = swiglu ? n0 + 32 * wn : n0 + 64 * wn;
  const bool full_tile = m0 + BM - 1 <= mmax && n0 + ncols - 1 <= nmax;
  const float* res = (const float*)g.res;
  const bf16_t* resb = (const bf16_t*)g.res;
  const bool res_bf16 = g.res_dt == BF16;
  const float* cscale = g.colscale ? g.colscale + z * g.sScale : nullptr;
  // The residual row of output row m needs a 64-bit remainder only when the
  // residual has fewer rows than C; the epilogue is compiled twice and the
  // wave takes the copy without it otherwise (every call in the layer passes
  // one residual row per output row).
  auto epilogue = [&](auto wrap_tag) __attribute__((always_inline)) {
    constexpr bool WRAP = decltype(wrap_tag)::value;
    auto res_row = [&](long m) __attribute__((always_inline)) {
      if constexpr (WRAP)
        return m % g.res_rows;
      else
        return m;
    };
    auto finish = [&](long m, long n, f32x4 val) __attribute__((always_inline)) {
      if constexpr (EPI == EPI_RESIDUAL) {
        const long rm = res_row(m) * g.ldr + n + z * g.sRes;
        if (res_bf16) {
          const uint2 u = *reinterpret_cast<const uint2*>(resb + rm);
          val[0] += __uint_as_float(u.x << 16);
          val[1] += __uint_as_float(u.x & 0xFFFF0000u);
          val[2] += __uint_as_float(u.y << 16);
          val[3] += __uint_as_float(u.y & 0xFFFF0000u);
        } else {
          const f32x4 f = *reinterpret_cast<const f32x4*>(res + rm);
          val += f;
        }
      } else if constexpr (EPI == EPI_STORE) {
        if (cscale) val *= *reinterpret_cast<const f32x4*>(cscale + n);
      }
      OutT* cp = C + m * g.ldc + n;
      if constexpr (sizeof(OutT) == 4) {
        *reinterpret_cast<f32x4*>(cp) = val;
      } else {
        *reinterpret_cast<uint2*>(cp) =
            uint2{pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
      }
    };
  #pragma unroll
    for (int i = 0; i < 4; ++i) {
  #pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 8 * (v >> 2) + 4 * h + (v & 3);
        if constexpr (swiglu) {
          slab[row * EPS + r] = silu(acc[i][0][v]) * acc[i][1][v];
        } else {
          slab[row * EPS + r] = acc[i][0][v];
          slab[row * EPS + 32 + r] = acc[i][1][v];
        }
      }
      lds_wave_sync();
      const long mb = m0 + 128 * wm + 32 * i;
      if (full_tile) {
  #pragma unroll
        for (int t = 0; t < npieces / 64; ++t) {
          const int idx = lane + 64 * t;
          const int rr = idx / per_row, c4 = 4 * (idx % per_row);
          finish(mb + rr, nw0 + c4, *reinterpret_cast<const f32x4*>(slab + rr * EPS + c4));
        }
      } else {
  #pragma unroll
        for (int t = 0; t < npieces / 64; ++t) {
          const int idx = lane + 64 * t;
          const int rr = idx / per_row, c4 = 4 * (idx % per_row);
          const long m = mb + rr, n = nw0 + c4;
          if (m > mmax || n > nmax) continue;
          f32x4 val = *reinterpret_cast<const f32x4*>(slab + rr * EPS + c4);
          if (n + 3 <= nmax) {
            finish(m, n, val);
            continue;
          }
          // ragged right edge: element by element
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (n + e > nmax) break;
            float x = val[e];
            if constexpr (EPI == EPI_RESIDUAL) {
              const long rm = res_row(m) * g.ldr + n + e + z * g.sRes;
              x += res_bf16 ? bf2f(resb[rm]) : res[rm];
            } else if constexpr (EPI == EPI_STORE) {
              if (cscale) x *= cscale[n + e];
            }
            stf(C + m * g.ldc + n + e, x);
          }
        }
      }
      lds_wave_sync();
    }
  };
  if (EPI == EPI_RESIDUAL && g.res_rows < g.M)
    epilogue(std::true_type{});
  else
    epilogue(std::false_type{});
}
}  // namespace big

// --------------------------------------------------------------------------
// Wide NT GEMM: 256 x 256 workgroup tile, 8 waves (two per SIMD) each
// owning a 128 x 64 block, BK = 32, a 4-stage global->LDS ring (128 KB, one
// workgroup per CU) fetched three stages ahead, so the direct-to-LDS loads
// of a stage have three stages of MFMA work to land behind.  The MFMA
// operand fragments of a stage's second k-step are read while the first
// k-step's MFMAs run, and the next stage's first fragments while the
// second k-step's run.  Per flop the tile moves 2/3 of the operand bytes of
// the 256 x 128 tile.
// --------------------------------------------------------------------------
namespace wide {
constexpr int BM = 256, BN = 256, BK = 32, NW = 8, NTH = 64 * NW, NST = 4;
constexpr int AB = BM * BK * 2, BB = BN * BK * 2;    // operand bytes per stage
constexpr int STAGE = AB + BB;                        // 32 KB
constexpr size_t LDS_BYTES = (size_t)NST * STAGE;     // 128 KB
constexpr int ALD = BM * BK / 8 / NTH;                // 16-byte loads per thread (A): 2
constexpr int BLD = BN * BK / 8 / NTH;                // (B): 2
constexpr int LPT = ALD + BLD;                        // loads per thread per stage
constexpr int EPS = 72;                               // epilogue slab row stride (floats)
static_assert(NW * 32 * EPS * 4 <= (int)LDS_BYTES, "epilogue slabs fit in the operand ring");

using big::barrier;

// 16 bytes per lane, global -> LDS; lane i lands at lds_wave_base + 16 i.
// Inline asm rather than the compiler builtin: the compiler counts a builtin
// LDS DMA as an LDS operation of unknown order and then waits for every
// outstanding LDS read (lgkmcnt 0) before any MFMA that needs one of them,
// which serialises the fragment reads of the next k-step with the MFMAs of
// this one.  The hardware counts the DMA in vmcnt alone and the loop orders
// it explicitly (wait_stages before the barrier that publishes a stage).
// M0 takes the LDS address; one wait state separates its write from the DMA.
TTCD_DEV void g2l16(const void* src, void* lds_wave_base) {
  const uint32_t m = (uint32_t)(size_t)(big::lds_void_t*)lds_wave_base;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(src), "{m0}"(m) : "memory");
}
using big::swz;
using big::lds_wave_sync;

template <int N>
TTCD_DEV void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// stages still in flight after the one waited for: 0, 1 or 2
TTCD_DEV void wait_stages(int pending) {
  if (pending >= 2)
    wait_vm<2 * LPT>();
  else if (pending == 1)
    wait_vm<LPT>();
  else
    wait_vm<0>();
}

template <typename OutT, int EPI, bool CHUNKED>
__global__ void __launch_bounds__(NTH, 1)
gemm_nt_wide(GemmArgs g) {
  extern __shared__ __align__(16) char lds[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  const int h = lane >> 5, r = lane & 31;
  // EPI_RESNORM is the residual epilogue plus the RMSNorm pieces
  constexpr int E = EPI == EPI_RESNORM ? EPI_RESIDUAL : EPI == EPI_SWIGLU_RS ? EPI_SWIGLU : EPI;
  constexpr bool NORM = EPI == EPI_RESNORM;
  constexpr bool RS = EPI == EPI_SWIGLU_RS;
  constexpr bool swiglu = E == EPI_SWIGLU;
  const int ncols = swiglu ? BN / 2 : BN;                   // output columns per tile
  const int ntn = (g.N + ncols - 1) / ncols;
  const int ntm = (g.M + BM - 1) / BM;
  // The remap runs over (batch, tile) in dispatch order (tile fastest), so
  // that each XCD takes whole batches of a batched call and the operands of
  // a batch are fetched into one L2 (the 63 chunk writes of the 64K
  // workload: 0.74 GB fetched instead of 1.83 GB).
  const uint32_t per = (uint32_t)(ntm * ntn);
  const uint32_t flat = xcd_remap(blockIdx.z * per + blockIdx.x, per * gridDim.z);
  const int z = (int)(flat / per);
  const uint32_t lid = flat % per;
  int tm, tn;
  grouped_tile(lid, ntm, ntn, 4, tm, tn);
  const long m0 = (long)tm * BM;
  const long n0 = (long)tn * ncols;

  const bf16_t* A = (const bf16_t*)g.A + z * g.sA;
  const bf16_t* Bm = (const bf16_t*)g.B + z * g.sB;
  const bf16_t* B2 = g.B2 ? (const bf16_t*)g.B2 + z * g.sB : nullptr;
  if constexpr (CHUNKED) {
    const long c = m0 / g.chunk;
    if (c > 0) Bm = (const bf16_t*)g.Bchunks + z * g.sBchunksBatch + (c - 1) * g.sBchunk;
  }
  const long mmax = g.M - 1, nmax = g.N - 1;
  const long lda = g.lda, ldb = g.ldb;
  auto a_row = [=](int rr) { return A + min(m0 + rr, mmax) * lda; };
  const long b2_off = swiglu ? (long)(B2 - Bm) : 0;
  auto b_row = [=](int rr) {
    if (swiglu) {
      // LDS row blocks of 32 alternate gate / up for the same 32 columns
      const int blk = rr >> 5;
      const long col = min(n0 + 32 * (blk >> 1) + (rr & 31), nmax);
      return Bm + ((blk & 1) ? b2_off : 0) + col * ldb;
    }
    return Bm + min(n0 + rr, nmax) * ldb;
  };
  // one 16-byte direct-to-LDS load of stage kt: idx < ALD are the A
  // tile's, the rest the B tile's; lane i of the wave lands at 16 i
  auto dma = [&](int kt, int idx) __attribute__((always_inline)) {
    char* st = lds + (kt % NST) * STAGE;
    const long k0 = (long)kt * BK;
    const bool is_a = idx < ALD;
    const int p0 = ((is_a ? idx : idx - ALD) * NW + wave) * 64;
    const int p = p0 + lane;
    const int row = p >> 2, c = (p & 3) ^ swz(row);
    if (is_a)
      g2l16(a_row(row) + k0 + 8 * c, st + p0 * 16);
    else
      g2l16(b_row(row) + k0 + 8 * c, st + AB + p0 * 16);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = zero16();

  // MFMA operand fragments of k-step ks (16 wide) of the stage at `as`
  struct Frag {
    bf16x8 a[4], b[2];
  };
  auto lfa = [&](const char* as, int ks, int i, Frag& f) __attribute__((always_inline)) {
    const int row = 128 * wm + 32 * i + r;
    f.a[i] = as_bf16x8(ld16(as + row * (BK * 2) + (((2 * ks + h) ^ swz(row)) << 4)));
  };
  auto lfb = [&](const char* as, int ks, int j, Frag& f) __attribute__((always_inline)) {
    const int row = 64 * wn + 32 * j + r;
    f.b[j] = as_bf16x8(ld16(as + AB + row * (BK * 2) + (((2 * ks + h) ^ swz(row)) << 4)));
  };

  const int nk = g.K / BK;
  const int npro = nk < NST - 1 ? nk : NST - 1;
  for (int kt = 0; kt < npro; ++kt)
#pragma unroll
    for (int idx = 0; idx < LPT; ++idx) dma(kt, idx);
  wait_stages(npro - 1);
  barrier();
  Frag f0, f1;
#pragma unroll
  for (int i = 0; i < 4; ++i) lfa(lds, 0, i, f0);
  lfb(lds, 0, 0, f0);
  lfb(lds, 0, 1, f0);
  // drain the scalar loads of the set-up before the loop, so that inside it
  // the LDS counter holds fragment reads alone and the compiler can wait for
  // the older fragment set while the newer one is still in flight
  __builtin_amdgcn_s_waitcnt(0xC07F);    // lgkmcnt(0)
  // Each wave issues its loads one or two at a time between its own MFMAs
  // (the scheduling barriers pin that order), so that they go out while
  // the matrix core works instead of in one burst after each barrier,
  // when every wave of the workgroup would stall on address issue at once.
#define SB __builtin_amdgcn_sched_barrier(0)
#define MM(F, I, J) acc[I][J] = mfma32(F.a[I], F.b[J], acc[I][J])
  static_assert(LPT == 4, "one load after every second MFMA of the first k-step");
  for (int kt = 0; kt < nk; ++kt) {
    // the slot refilled here held stage kt-1; every wave finished reading it
    // before the barrier that ended the previous iteration
    const bool pf = kt + NST - 1 < nk;
    const int kn = kt + NST - 1;
    const char* as = lds + (kt % NST) * STAGE;
    MM(f0, 0, 0); SB; if (pf) dma(kn, 0); SB;
    MM(f0, 0, 1); SB; lfa(as, 1, 0, f1); lfa(as, 1, 1, f1); SB;
    MM(f0, 1, 0); SB; if (pf) dma(kn, 1); SB;
    MM(f0, 1, 1); SB; lfa(as, 1, 2, f1); lfa(as, 1, 3, f1); SB;
    MM(f0, 2, 0); SB; if (pf) dma(kn, 2); SB;
    MM(f0, 2, 1); SB; lfb(as, 1, 0, f1); lfb(as, 1, 1, f1); SB;
    MM(f0, 3, 0); SB; if (pf) dma(kn, 3); SB;
    MM(f0, 3, 1); SB;
    // stage kt+1 must have landed (later ones may still be in flight), and
    // this wave's reads of stage kt are complete before the barrier
    const int last = kt + NST - 1 < nk ? kt + NST - 1 : nk - 1;
    lds_wave_sync();
    wait_stages(last - (kt + 1));
    barrier();
    // (after the last stage this reads a slot nobody uses; it stays in bounds)
    const char* an = lds + ((kt + 1) % NST) * STAGE;
    MM(f1, 0, 0); SB; lfa(an, 0, 0, f0); SB;
    MM(f1, 0, 1); SB; lfa(an, 0, 1, f0); SB;
    MM(f1, 1, 0); SB; lfa(an, 0, 2, f0); SB;
    MM(f1, 1, 1); SB; lfa(an, 0, 3, f0); SB;
    MM(f1, 2, 0); SB; lfb(an, 0, 0, f0); SB;
    MM(f1, 2, 1); SB; lfb(an, 0, 1, f0); SB;
    MM(f1, 3, 0); SB;
    MM(f1, 3, 1); SB;
  }
#undef MM
#undef SB
  // every wave's last MFMAs are done reading the ring before the epilogue
  // reuses it as slabs
  lds_wave_sync();
  barrier();

  // Epilogue through a wave-private LDS slab: one 32-row block row of the
  // wave's tile at a time, written as the MFMA layout leaves it and read back
  // row-major, so each lane stores 16 bytes of consecutive columns.
  OutT* C = (OutT*)g.C + z * g.sC;
  float* slab = reinterpret_cast<float*>(lds) + wave * (32 * EPS);
  constexpr int ocols = swiglu ? 32 : 64;
  constexpr int per_row = ocols / 4;
  constexpr int npieces = 32 * per_row;
  const long nw0 = swiglu ? n0 + 32 * wn : n0 + 64 * wn;
  const bool full_tile = m0 + BM - 1 <= mmax && n0 + ncols - 1 <= nmax;
  const int c4l_n = 4 * (lane % per_row);
  const float* res = (const float*)g.res;
  const bf16_t* resb = (const bf16_t*)g.res;
  const bool res_bf16 = g.res_dt == BF16;
  const float* cscale = g.colscale ? g.colscale + z * g.sScale : nullptr;
  const float* rsc = g.rowscale;   // read by the EPI_SWIGLU_RS copy only
  // RMSNorm pieces: a lane's 4 columns are fixed over the epilogue, so is
  // its gamma; the 16 lanes of a row piece hold its 64 columns
  f32x4 gam = {1.f, 1.f, 1.f, 1.f};
  if constexpr (NORM) {
    if (g.gamma) {
      const uint2 gu = *reinterpret_cast<const uint2*>((const bf16_t*)g.gamma + nw0 + c4l_n);
      gam = f32x4{__uint_as_float(gu.x << 16), __uint_as_float(gu.x & 0xFFFF0000u),
                  __uint_as_float(gu.y << 16), __uint_as_float(gu.y & 0xFFFF0000u)};
    }
  }
  auto finish = [&](long m, long n, f32x4 val) __attribute__((always_inline)) {
    if constexpr (E == EPI_RESIDUAL) {
      const long rm = (g.res_rows < g.M ? m % g.res_rows : m) * g.ldr + n + z * g.sRes;
      if (res_bf16) {
        const uint2 u = *reinterpret_cast<const uint2*>(resb + rm);
        val[0] += __uint_as_float(u.x << 16);
        val[1] += __uint_as_float(u.x & 0xFFFF0000u);
        val[2] += __uint_as_float(u.y << 16);
        val[3] += __uint_as_float(u.y & 0xFFFF0000u);
      } else {
        val += *reinterpret_cast<const f32x4*>(res + rm);
      }
    } else if constexpr (E == EPI_STORE) {
      if (cscale) val *= *reinterpret_cast<const f32x4*>(cscale + n);
    }
    OutT* cp = C + m * g.ldc + n;
    if constexpr (sizeof(OutT) == 4) {
      *reinterpret_cast<f32x4*>(cp) = val;
    } else {
      *reinterpret_cast<uint2*>(cp) = uint2{pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
    }
  };
  // In a full tile a lane's pieces all sit in the same 4 columns (64 is a
  // multiple of per_row): the column scale is read once, and the residual
  // of block row i + 1 is read before block row i is stored, so that the
  // reads are in flight together (a read issued after a store to C, which
  // may alias the residual, would wait for it).
  constexpr int NP = npieces / 64;
  static_assert(64 % per_row == 0, "a lane's pieces share their columns");
  const int c4l = 4 * (lane % per_row);
  f32x4 csv = {1.f, 1.f, 1.f, 1.f};
  if constexpr (E == EPI_STORE) {
    if (cscale && full_tile) csv = *reinterpret_cast<const f32x4*>(cscale + nw0 + c4l);
  }
  // the residual's type is fixed per call: two copies of the epilogue, so
  // that no branch sits between a residual read and its use
  auto run_epilogue = [&](auto RBc, auto FTc) __attribute__((always_inline)) {
    constexpr bool RB = decltype(RBc)::value;
    constexpr bool FT = decltype(FTc)::value;
    auto load_res = [&](int i, u32x4 (&rv)[NP]) __attribute__((always_inline)) {
      const long mb = m0 + 128 * wm + 32 * i;
#pragma unroll
      for (int t = 0; t < NP; ++t) {
        const long m = mb + (lane + 64 * t) / per_row;
        const long rm = (g.res_rows < g.M ? m % g.res_rows : m) * g.ldr + nw0 + c4l + z * g.sRes;
        if constexpr (RB) {
          const uint2 u = *reinterpret_cast<const uint2*>(resb + rm);
          rv[t] = u32x4{u.x, u.y, 0u, 0u};
        } else {
          rv[t] = *reinterpret_cast<const u32x4*>(res + rm);
        }
      }
    };
    u32x4 rva[NP], rvb[NP];
    if constexpr (E == EPI_RESIDUAL) {
      if constexpr (FT) load_res(0, rva);
    }
    // SwiGLU row scale: a lane's 16 rows of block row i are 4 runs of 4
    // (every tile is full); block row i + 1's are read before block row i
    // is stored, since a read issued after the stores would wait for them
    auto load_rs = [&](int i, f32x4 (&sv)[4]) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        sv[q] = *reinterpret_cast<const f32x4*>(rsc + m0 + 128 * wm + 32 * i + 8 * q + 4 * h);
    };
    f32x4 rsa[4], rsb[4];
    if constexpr (RS) load_rs(0, rsa);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 (&rcur)[NP] = (i & 1) ? rvb : rva;
      u32x4 (&rnext)[NP] = (i & 1) ? rva : rvb;
      if constexpr (E == EPI_RESIDUAL) {
        if (FT && i + 1 < 4) load_res(i + 1, rnext);
      }
      f32x4 (&scur)[4] = (i & 1) ? rsb : rsa;
      if constexpr (RS) {
        if (i + 1 < 4) load_rs(i + 1, (i & 1) ? rsa : rsb);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 8 * (v >> 2) + 4 * h + (v & 3);
        if constexpr (swiglu) {
          if constexpr (RS) {
            const float sc = scur[v >> 2][v & 3];
            slab[row * EPS + r] = silu(sc * acc[i][0][v]) * (sc * acc[i][1][v]);
          } else {
            slab[row * EPS + r] = silu(acc[i][0][v]) * acc[i][1][v];
          }
        } else {
          slab[row * EPS + r] = acc[i][0][v];
          slab[row * EPS + 32 + r] = acc[i][1][v];
        }
      }
      lds_wave_sync();
      const long mb = m0 + 128 * wm + 32 * i;
      if constexpr (FT) {
#pragma unroll
        for (int t = 0; t < NP; ++t) {
          const int rr = (lane + 64 * t) / per_row;
          f32x4 val = *reinterpret_cast<const f32x4*>(slab + rr * EPS + c4l);
          if constexpr (E == EPI_RESIDUAL) {
            if constexpr (RB) {
              val[0] += __uint_as_float(rcur[t][0] << 16);
              val[1] += __uint_as_float(rcur[t][0] & 0xFFFF0000u);
              val[2] += __uint_as_float(rcur[t][1] << 16);
              val[3] += __uint_as_float(rcur[t][1] & 0xFFFF0000u);
            } else {
              val[0] += __uint_as_float(rcur[t][0]);
              val[1] += __uint_as_float(rcur[t][1]);
              val[2] += __uint_as_float(rcur[t][2]);
              val[3] += __uint_as_float(rcur[t][3]);
            }
          } else if constexpr (E == EPI_STORE) {
            val *= csv;
          }
          if constexpr (NORM) {
            bf16_t* up = (bf16_t*)g.U + (mb + rr) * g.ldc + nw0 + c4l;
            *reinterpret_cast<uint2*>(up) = uint2{pack_bf16x2(val[0] * gam[0], val[1] * gam[1]),
                                                  pack_bf16x2(val[2] * gam[2], val[3] * gam[3])};
            float ss = val[0] * val[0] + val[1] * val[1] + val[2] * val[2] + val[3] * val[3];
#pragma unroll
            for (int o = 8; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
            if ((lane & 15) == 0) g.rowss[(nw0 >> 6) * (long)g.M + mb + rr] = ss;
          }
          OutT* cp = C + (mb + rr) * g.ldc + nw0 + c4l;
          if constexpr (sizeof(OutT) == 4) {
            *reinterpret_cast<f32x4*>(cp) = val;
          } else {
            *reinterpret_cast<uint2*>(cp) =
                uint2{pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
          }
        }
      } else {
#pragma unroll
        for (int t = 0; t < npieces / 64; ++t) {
          const int idx = lane + 64 * t;
          const int rr = idx / per_row, c4 = 4 * (idx % per_row);
          const long m = mb + rr, n = nw0 + c4;
          if (m > mmax || n > nmax) continue;
          f32x4 val = *reinterpret_cast<const f32x4*>(slab + rr * EPS + c4);
          if (n + 3 <= nmax) {
            finish(m, n, val);
            continue;
          }
          for (int e = 0; e < 4; ++e) {
            if (n + e > nmax) break;
            float x = val[e];
            if constexpr (E == EPI_RESIDUAL) {
              const long rm = (g.res_rows < g.M ? m % g.res_rows : m) * g.ldr + n + e + z * g.sRes;
              x += res_bf16 ? bf2f(resb[rm]) : res[rm];
            } else if constexpr (E == EPI_STORE) {
              if (cscale) x *= cscale[n + e];
            }
            stf(C + m * g.ldc + n + e, x);
          }
        }
      }
      lds_wave_sync();
    }
  };
  if (E == EPI_RESIDUAL && res_bf16) {
    if (full_tile)
      run_epilogue(std::true_type{}, std::true_type{});
    else
      run_epilogue(std::true_type{}, std::false_type{});
  } else {
    if (full_tile)
      run_epilogue(std::false_type{}, std::true_type{});
    else
      run_epilogue(std::false_type{}, std::false_type{});
  }
}
}  // namespace wide

// --------------------------------------------------------------------------
// Few-row NT GEMM (a decode step: one row per sequence), M <= 32.  One wave
// per 32-column tile and K slice: the MFMA operands come straight from
// global memory (every A and B row is read once per slice), so enough waves
// exist to stream the weight matrix at full bandwidth; the slices' fp32
// partial sums go to the workspace and a second kernel adds them and applies
// the epilogue.  For SwiGLU the gate columns are [0, N) and the up columns
// [N, 2N) of the partial sums.
// --------------------------------------------------------------------------
namespace skinny {
constexpr int TARGET_WAVES = 1024;

TTCD_DEV bf16x8 ld_frag(const bf16_t* row, long k, long kend) {
  return k < kend ? as_bf16x8(ld16(row + k)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
}

__global__ void __launch_bounds__(64)
gemm_skinny_part(GemmArgs g, int kslice, int ncols) {
  const int tn = blockIdx.x, ks = blockIdx.y;
  const int lane = threadIdx.x, r = lane & 31, h = lane >> 5;
  const bool swiglu = g.epi == EPI_SWIGLU;
  const int n = min(tn * 32 + r, ncols - 1);           // this lane's B row (output column)
  const bf16_t* br = (swiglu && n >= g.N) ? (const bf16_t*)g.B2 + (size_t)(n - g.N) * g.ldb
                                           : (const bf16_t*)g.B + (size_t)n * g.ldb;
  const bf16_t* ar = (const bf16_t*)g.A + (size_t)min(r, g.M - 1) * g.lda;
  const long k0 = (long)ks * kslice;
  const long k1 = min(k0 + (long)kslice, (long)g.K);
  f32x16 acc = zero16();
  for (long kk = k0; kk < k1; kk += 64) {
    bf16x8 af[4], bf[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const long k = kk + 16 * u + 8 * h;
      af[u] = ld_frag(ar, k, k1);
      bf[u] = ld_frag(br, k, k1);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc = mfma32(af[u], bf[u], acc);
  }
  // lane: column tn*32 + r, rows 8(v/4) + 4h + v%4
  const int col = tn * 32 + r;
  if (col >= ncols) return;
  float* part = g.ws + (size_t)ks * g.M * ncols;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int m = 8 * (v >> 2) + 4 * h + (v & 3);
    if (m < g.M) part[(size_t)m * ncols + col] = acc[v];
  }
}

template <typename OutT>
__global__ void __launch_bounds__(256)
gemm_skinny_reduce(GemmArgs g, int nks, int ncols) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)g.M * g.N) return;
  const int m = (int)(i / g.N), n = (int)(i % g.N);
  float a = 0.f, u = 0.f;
  for (int ks = 0; ks < nks; ++ks) {
    const float* part = g.ws + (size_t)ks * g.M * ncols + (size_t)m * ncols;
    a += part[n];
    if (g.epi == EPI_SWIGLU) u += part[g.N + n];
  }
  float val;
  if (g.epi == EPI_SWIGLU) {
    val = silu(a) * u;
  } else if (g.epi == EPI_RESIDUAL) {
    const long rm = (long)(m % g.res_rows) * g.ldr + n;
    val = a + (g.res_dt == BF16 ? bf2f(((const bf16_t*)g.res)[rm]) : ((const float*)g.res)[rm]);
  } else {
    val = g.colscale ? a * g.colscale[n] : a;
  }
  stf((OutT*)g.C + (size_t)m * g.ldc + n, val);
}

int ksplit_for(int N, int K, int epi) {
  const int ncols = epi == EPI_SWIGLU ? 2 * N : N;
  const int tiles = (ncols + 31) / 32;
  const int max_split = (K + 63) / 64;
  int ks = (TARGET_WAVES + tiles - 1) / tiles;
  return ks < 1 ? 1 : (ks > max_split ? max_split : ks);
}
}  // namespace skinny

bool skinny_ok(const GemmArgs& g) {
  return g.ws && g.M <= 32 && g.in_dt == BF16 && g.batch <= 1 && g.chunk == 0 &&
         g.K % 8 == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 &&
         gemm_skinny_ws_floats(g.M, g.N, g.K, g.epi) <= g.ws_floats;
}

bool big_ok(const GemmArgs& g) {
  if (g.in_dt != BF16) return false;
  if (g.K % big::BK || g.lda % 8 || g.ldb % 8) return false;
  // the epilogue moves 4 consecutive columns per access
  if (g.ldc % 4 || g.sC % 4) return false;
  if (g.epi == EPI_RESIDUAL && (g.ldr % 4 || g.sRes % 4)) return false;
  if (g.chunk > 0 && g.chunk % big::BM) return false;
  // enough tiles to fill the chip
  const long tiles = (long)((g.M + big::BM - 1) / big::BM) *
                     ((g.N + big::BN - 1) / (g.epi == EPI_SWIGLU ? big::BN / 2 : big::BN)) *
                     (g.batch > 0 ? g.batch : 1);
  return tiles >= 256;
}

bool wide_ok(const GemmArgs& g) {
  if (g.in_dt != BF16) return false;
  if (g.K % wide::BK || g.lda % 8 || g.ldb % 8) return false;
  if (g.ldc % 4 || g.sC % 4) return false;
  if ((g.epi == EPI_RESIDUAL || g.epi == EPI_RESNORM) && (g.ldr % 4 || g.sRes % 4)) return false;
  if (g.chunk > 0 && g.chunk % wide::BM) return false;
  // enough tiles to give every CU one
  const long tiles = (long)((g.M + wide::BM - 1) / wide::BM) *
                     ((g.N + wide::BN - 1) / (g.epi == EPI_SWIGLU ? wide::BN / 2 : wide::BN)) *
                     (g.batch > 0 ? g.batch : 1);
  return tiles >= 256;
}

bool mfma_ok(const GemmArgs& g) {
  if (g.in_dt != BF16) return false;
  if (g.K % 8 || g.lda % 8 || g.ldb % 8) return false;
  if (g.chunk > 0 && g.chunk % BM) return false;
  return true;
}

}  // namespace

size_t gemm_skinny_ws_floats(int M, int N, int K, int epi) {
  const int ncols = epi == EPI_SWIGLU ? 2 * N : N;
  return (size_t)skinny::ksplit_for(N, K, epi) * M * ncols;
}

namespace {
template <typename OutT, bool CHUNKED>
const void* big_kernel_epi(int epi) {
  switch (epi) {
    case EPI_STORE: return (const void*)big::gemm_nt_big<OutT, EPI_STORE, CHUNKED>;
    case EPI_RESIDUAL: return (const void*)big::gemm_nt_big<OutT, EPI_RESIDUAL, CHUNKED>;
    case EPI_SWIGLU: return CHUNKED ? nullptr : (const void*)big::gemm_nt_big<OutT, EPI_SWIGLU, false>;
    default: return nullptr;
  }
}
template <typename OutT, bool CHUNKED>
const void* wide_kernel_epi(int epi) {
  switch (epi) {
    case EPI_STORE: return (const void*)wide::gemm_nt_wide<OutT, EPI_STORE, CHUNKED>;
    case EPI_RESIDUAL: return (const void*)wide::gemm_nt_wide<OutT, EPI_RESIDUAL, CHUNKED>;
    case EPI_SWIGLU: return CHUNKED ? nullptr : (const void*)wide::gemm_nt_wide<OutT, EPI_SWIGLU, false>;
    case EPI_RESNORM:
      return CHUNKED || sizeof(OutT) != 4 ? nullptr
                                          : (const void*)wide::gemm_nt_wide<float, EPI_RESNORM, false>;
    default: return nullptr;
  }
}
const void* wide_kernel(bool out_bf16, int epi, bool chunked) {
  if (chunked)
    return out_bf16 ? wide_kernel_epi<bf16_t, true>(epi) : wide_kernel_epi<float, true>(epi);
  return out_bf16 ? wide_kernel_epi<bf16_t, false>(epi) : wide_kernel_epi<float, false>(epi);
}
const void* big_kernel(bool out_bf16, int epi, bool chunked) {
  if (chunked)
    return out_bf16 ? big_kernel_epi<bf16_t, true>(epi) : big_kernel_epi<float, true>(epi);
  return out_bf16 ? big_kernel_epi<bf16_t, false>(epi) : big_kernel_epi<float, false>(epi);
}
// the dynamic LDS limit of each kernel is raised once, on its first launch
// (a fixed table: launching allocates no host memory)
hipError_t lds_attr(const void* kern, size_t bytes) {
  static std::mutex mu;
  static const void* done[32];
  static int ndone = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < ndone; ++i)
    if (done[i] == kern) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)bytes);
  if (e == hipSuccess && ndone < 32) done[ndone++] = kern;
  return e;
}
}  // namespace

bool gemm_wide_full(const GemmArgs& g) {
  const int ncols = g.epi == EPI_SWIGLU ? wide::BN / 2 : wide::BN;
  return g.M > 0 && !skinny_ok(g) && wide_ok(g) && g.batch <= 1 && g.chunk == 0 &&
         g.M % wide::BM == 0 && g.N % ncols == 0;
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const int nb = g.batch > 0 ? g.batch : 1;
  // the RMSNorm pieces exist in the full-tile 256 x 256 epilogue only
  if (g.epi == EPI_RESNORM || g.rowscale) {
    if (!gemm_wide_full(g) || g.in_dt != BF16 || (g.epi == EPI_RESNORM && (!g.U || !g.rowss ||
                                                                           g.out_dt != F32)))
      return hipErrorInvalidValue;
  }
  if (skinny_ok(g)) {
    const int ncols = g.epi == EPI_SWIGLU ? 2 * g.N : g.N;
    const int nks = skinny::ksplit_for(g.N, g.K, g.epi);
    const int kslice = ((g.K + nks - 1) / nks + 63) / 64 * 64;
    const int nks_used = (g.K + kslice - 1) / kslice;
    hipLaunchKernelGGL(skinny::gemm_skinny_part, dim3((ncols + 31) / 32, nks_used), dim3(64), 0,
                       s, g, kslice, ncols);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned nblk = (unsigned)(((long)g.M * g.N + 255) / 256);
    if (g.out_dt == BF16)
      hipLaunchKernelGGL(skinny::gemm_skinny_reduce<bf16_t>, dim3(nblk), dim3(256), 0, s, g,
                         nks_used, ncols);
    else
      hipLaunchKernelGGL(skinny::gemm_skinny_reduce<float>, dim3(nblk), dim3(256), 0, s, g,
                         nks_used, ncols);
    return hipGetLastError();
  }
  if (wide_ok(g)) {
    const void* kern =
        g.rowscale ? (g.out_dt == BF16 && g.epi == EPI_SWIGLU
                          ? (const void*)wide::gemm_nt_wide<bf16_t, EPI_SWIGLU_RS, false>
                          : nullptr)
                   : wide_kernel(g.out_dt == BF16, g.epi, g.chunk > 0);
    if (!kern) return hipErrorInvalidValue;
    const hipError_t e = lds_attr(kern, wide::LDS_BYTES);
    if (e != hipSuccess) return e;
    const int ncols = g.epi == EPI_SWIGLU ? wide::BN / 2 : wide::BN;
    const unsigned tiles =
        (unsigned)(((g.M + wide::BM - 1) / wide::BM) * ((g.N + ncols - 1) / ncols));
    dim3 grid(tiles, 1, nb);
    void* args[] = {(void*)&g};
    return hipLaunchKernel(kern, grid, dim3(wide::NTH), args, wide::LDS_BYTES, s);
  }
  if (big_ok(g)) {
    const size_t lds = big::lds_bytes(big::NST);
    const void* kern = big_kernel(g.out_dt == BF16, g.epi, g.chunk > 0);
    if (!kern) return hipErrorInvalidValue;
    const hipError_t e = lds_attr(kern, lds);
    if (e != hipSuccess) return e;
    const int ncols = g.epi == EPI_SWIGLU ? big::BN / 2 : big::BN;
    const unsigned tiles = (unsigned)(((g.M + big::BM - 1) / big::BM) * ((g.N + ncols - 1) / ncols));
    dim3 grid(tiles, 1, nb);
    void* args[] = {(void*)&g};
    return hipLaunchKernel(kern, grid, dim3(big::NTH), args, lds, s);
  }
  if (mfma_ok(g)) {
    static bool attr = false;
    if (!attr) {
      (void)hipFuncSetAttribute((const void*)gemm_nt_mfma<float>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)GEMM_LDS);
      (void)hipFuncSetAttribute((const void*)gemm_nt_mfma<bf16_t>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)GEMM_LDS);
      attr = true;
    }
    const int ncols = g.epi == EPI_SWIGLU ? 64 : BN;
    dim3 grid((g.M + BM - 1) / BM, (g.N + ncols - 1) / ncols, nb);
    if (g.out_dt == BF16)
      hipLaunchKernelGGL(gemm_nt_mfma<bf16_t>, grid, dim3(NT), GEMM_LDS, s, g);
    else
      hipLaunchKernelGGL(gemm_nt_mfma<float>, grid, dim3(NT), GEMM_LDS, s, g);
    return hipGetLastError();
  }
  if (g.chunk > 0) {
    // one launch per chunk so that no row tile straddles two weights
    const int in_es = g.in_dt == BF16 ? 2 : 4, out_es = g.out_dt == BF16 ? 2 : 4;
    const int res_es = g.res_dt == BF16 ? 2 : 4;
    for (long c = 0; c * g.chunk < g.M; ++c) {
      GemmArgs h = g;
      const long r0 = c * g.chunk;
      h.chunk = 0;
      h.M = (int)std::min<long>(g.chunk, g.M - r0);
      h.A = (const char*)g.A + r0 * g.lda * in_es;
      h.C = (char*)g.C + r0 * g.ldc * out_es;
      if (g.res) {
        // residual rows follow the output rows of the same batch element
        h.res = (const char*)g.res + r0 * g.ldr * res_es;
        h.res_rows = g.res_rows - (int)r0;
      }
      if (c > 0) {
        h.B = (const char*)g.Bchunks + (c - 1) * g.sBchunk * in_es;
        h.sB = g.sBchunksBatch;
      }
      hipError_t e = launch_gemm(h, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  dim3 grid((g.M + SB - 1) / SB, (g.N + SB - 1) / SB, nb);
  if (g.in_dt == BF16) {
    if (g.out_dt == BF16)
      hipLaunchKernelGGL((gemm_nt_simple<bf16_t, bf16_t>), grid, dim3(256), 0, s, g);
    else
      hipLaunchKernelGGL((gemm_nt_simple<bf16_t, float>), grid, dim3(256), 0, s, g);
  } else {
    if (g.out_dt == BF16)
      hipLaunchKernelGGL((gemm_nt_simple<float, bf16_t>), grid, dim3(256), 0, s, g);
    else
      hipLaunchKernelGGL((gemm_nt_simple<float, float>), grid, dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

}  // namespace ttcd
