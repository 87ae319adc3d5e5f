// Dense contractions of the IP-TTCD layer on gfx950:
//   C = A B^T with A [M, K] and B [N, K] both K-contiguous ("NT"), bf16 in,
//   fp32 MFMA accumulate, with fused epilogues (residual add, SwiGLU,
//   per-column scale, chunk-indexed weights), and the fast-weight prefix
//   kernel that keeps a d x f tile of the weight in registers while it
//   walks the chunks in order (papernotes.org notes on "Learning What to
//   Remember", key design 2: causal prefix sum of the chunk updates;
//   key design 3: dW_i = beta_i R_i K_i^T).
#include <algorithm>

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

TTCD_DEV float silu(float a) { return a / (1.f + __expf(-a)); }

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

// Fast-weight prefix: one 128 x 128 tile of the d x f weight per workgroup.
template <typename StT>
__global__ void __launch_bounds__(NT, 1)
fw_states_mfma(StateArgs a) {
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
  const long n0 = (long)(lid % ncol_tiles) * BN;
  const bf16_t* A = (const bf16_t*)a.A + z * a.sA;
  const bf16_t* Bm = (const bf16_t*)a.B + z * a.sB;
  const bf16_t* W0 = (const bf16_t*)a.W0;

  Tile t;
#pragma unroll
  for (int bm = 0; bm < 2; ++bm)
#pragma unroll
    for (int bn = 0; bn < 2; ++bn)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const long m = m0 + 64 * wm + 32 * bm + 8 * (v >> 2) + 4 * h + (v & 3);
        const long n = n0 + 64 * wn + 32 * bn + r;
        t.acc[bm][bn][v] = (m < a.d && n < a.f) ? bf2f(W0[m * a.f + n]) : 0.f;
      }

  for (int i = 0; i < a.nwrites; ++i) {
    const long kb = (long)i * a.chunk;
    const long ke = min((long)(i + 1) * a.chunk, (long)a.T);
    mainloop(t, A, a.lda, m0, a.d, Bm, nullptr, a.ldb, n0, a.f, kb, ke, lds, 64 * wn,
             64 * wn + 32);
    StT* S = nullptr;
    if (i < a.nstates) S = (StT*)a.states + z * a.sStates + (long)i * a.d * a.f;
    float* Fo = (i == a.nwrites - 1 && a.final_out) ? a.final_out + z * a.sFinal : nullptr;
    if (!S && !Fo) continue;
#pragma unroll
    for (int bm = 0; bm < 2; ++bm)
#pragma unroll
      for (int bn = 0; bn < 2; ++bn)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const long m = m0 + 64 * wm + 32 * bm + 8 * (v >> 2) + 4 * h + (v & 3);
          const long n = n0 + 64 * wn + 32 * bn + r;
          if (m < a.d && n < a.f) {
            if (S) stf(S + m * a.f + n, t.acc[bm][bn][v]);
            if (Fo) Fo[m * a.f + n] = t.acc[bm][bn][v];
          }
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

template <typename InT, typename StT>
__global__ void __launch_bounds__(256) fw_states_simple(StateArgs a) {
  const int z = blockIdx.z;
  const long m0 = (long)blockIdx.x * SB, n0 = (long)blockIdx.y * SB;
  const InT* A = (const InT*)a.A + z * a.sA;
  const InT* Bm = (const InT*)a.B + z * a.sB;
  const InT* W0 = (const InT*)a.W0;
  const int tr = threadIdx.x / 16, tc = threadIdx.x % 16;
  float acc[4][4], dummy[4][4] = {};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long m = m0 + tr * 4 + i, n = n0 + tc * 4 + j;
      acc[i][j] = (m < a.d && n < a.f) ? ldf(W0 + m * a.f + n) : 0.f;
    }
  for (int c = 0; c < a.nwrites; ++c) {
    const long kb = (long)c * a.chunk, ke = min((long)(c + 1) * a.chunk, (long)a.T);
    simple_tile<InT>(acc, dummy, A, a.lda, m0, a.d, Bm, nullptr, a.ldb, n0, a.f, kb, ke);
    StT* S = c < a.nstates ? (StT*)a.states + z * a.sStates + (long)c * a.d * a.f : nullptr;
    float* Fo = (c == a.nwrites - 1 && a.final_out) ? a.final_out + z * a.sFinal : nullptr;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const long m = m0 + tr * 4 + i, n = n0 + tc * 4 + j;
        if (m >= a.d || n >= a.f) continue;
        if (S) stf(S + m * a.f + n, acc[i][j]);
        if (Fo) Fo[m * a.f + n] = acc[i][j];
      }
  }
}


// --------------------------------------------------------------------------
// Large-tile NT GEMM: 256 x 128 workgroup tile, 4 waves each owning a
// 128 x 64 block (8 MFMAs per 6 KB of LDS operand reads), BK = 32.  Operand
// tiles go straight from global memory into LDS (global_load_lds_dwordx4) in
// an XOR-swizzled layout that keeps the MFMA operand reads free of bank
// conflicts; a 3-stage ring is fetched two stages ahead, and two workgroups
// share a CU.  Requires K % 32 == 0 and 16-byte aligned rows.
// --------------------------------------------------------------------------
namespace big {
constexpr int BM = 256, BN = 128, BK = 32, NW = 4, NTH = 64 * NW, NST = 3;
constexpr int AB = BM * BK * 2, BB = BN * BK * 2;   // operand bytes per stage
constexpr int STAGE = AB + BB;
constexpr size_t LDS = (size_t)NST * STAGE;          // 72 KB
constexpr int ALD = BM * BK / 8 / (64 * NW);         // 16B loads per wave (A)
constexpr int BLD = BN * BK / 8 / (64 * NW);         // 16B loads per wave (B)
constexpr int LPW = ALD + BLD;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

TTCD_DEV void g2l16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)lds_wave_base, 16, 0, 0);
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

template <typename OutT>
__global__ void __launch_bounds__(NTH, 2)
gemm_nt_big(GemmArgs g) {
  extern __shared__ __align__(16) char lds[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, r = lane & 31;
  const int z = blockIdx.z;
  const bool swiglu = g.epi == EPI_SWIGLU;
  const int ncols = swiglu ? BN / 2 : BN;                   // output columns per tile
  const int ntn = (g.N + ncols - 1) / ncols;
  const int ntm = (g.M + BM - 1) / BM;
  const uint32_t lid = xcd_remap(blockIdx.x, (uint32_t)(ntm * ntn));
  const long m0 = (long)(lid / ntn) * BM;
  const long n0 = (long)(lid % ntn) * ncols;

  const bf16_t* A = (const bf16_t*)g.A + z * g.sA;
  const bf16_t* Bm = (const bf16_t*)g.B + z * g.sB;
  const bf16_t* B2 = g.B2 ? (const bf16_t*)g.B2 + z * g.sB : nullptr;
  if (g.chunk > 0) {
    const long c = m0 / g.chunk;
    if (c > 0) Bm = (const bf16_t*)g.Bchunks + z * g.sBchunksBatch + (c - 1) * g.sBchunk;
  }
  const long mmax = g.M - 1, nmax = g.N - 1;
  const long lda = g.lda, ldb = g.ldb;
  auto a_row = [&](int rr) { return A + min(m0 + rr, mmax) * lda; };
  auto b_row = [&](int rr) {
    if (swiglu) {
      // LDS row blocks of 32 alternate gate / up for the same 32 columns
      const int blk = rr >> 5;
      const long col = min(n0 + 32 * (blk >> 1) + (rr & 31), nmax);
      return ((blk & 1) ? B2 : Bm) + col * ldb;
    }
    return Bm + min(n0 + rr, nmax) * ldb;
  };
  auto fetch = [&](int kt) {
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
  fetch(0);
  if (nk > 1) {
    fetch(1);
    wait_vm<LPW>();
  } else {
    wait_vm<0>();
  }
  barrier();
  for (int kt = 0; kt < nk; ++kt) {
    const bool ahead = kt + 2 < nk;
    if (ahead) fetch(kt + 2);
    const char* as = lds + (kt % NST) * STAGE;
    const char* bs = as + AB;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 128 * wm + 32 * i + r;
        af[i] = as_bf16x8(ld16(as + row * (BK * 2) + (((2 * ks + h) ^ swz(row)) << 4)));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = 64 * wn + 32 * j + r;
        bfr[j] = as_bf16x8(ld16(bs + row * (BK * 2) + (((2 * ks + h) ^ swz(row)) << 4)));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
    // stage kt+1 must have landed; stage kt+2 may still be in flight
    if (ahead)
      wait_vm<LPW>();
    else
      wait_vm<0>();
    barrier();
  }

  OutT* C = (OutT*)g.C + z * g.sC;
  if (swiglu) {
    const long n = n0 + 32 * wn + r;
    if (n > nmax) return;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const long m = m0 + 128 * wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        if (m <= mmax) stf(C + m * g.ldc + n, silu(acc[i][0][v]) * acc[i][1][v]);
      }
    return;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const long n = n0 + 64 * wn + 32 * j + r;
    if (n > nmax) continue;
    float cs = 1.f;
    if (g.epi == EPI_STORE && g.colscale) cs = g.colscale[z * g.sScale + n];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const long m = m0 + 128 * wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        if (m > mmax) continue;
        float val = acc[i][j][v];
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
}  // namespace big

bool big_ok(const GemmArgs& g) {
  if (g.in_dt != BF16) return false;
  if (g.K % big::BK || g.lda % 8 || g.ldb % 8) return false;
  if (g.chunk > 0 && g.chunk % big::BM) return false;
  // enough tiles to fill the chip
  const long tiles = (long)((g.M + big::BM - 1) / big::BM) *
                     ((g.N + big::BN - 1) / (g.epi == EPI_SWIGLU ? big::BN / 2 : big::BN)) *
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

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const int nb = g.batch > 0 ? g.batch : 1;
  if (big_ok(g)) {
    static hipError_t a1 = hipFuncSetAttribute((const void*)big::gemm_nt_big<float>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)big::LDS);
    static hipError_t a2 = hipFuncSetAttribute((const void*)big::gemm_nt_big<bf16_t>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)big::LDS);
    if (a1 != hipSuccess) return a1;
    if (a2 != hipSuccess) return a2;
    const int ncols = g.epi == EPI_SWIGLU ? big::BN / 2 : big::BN;
    const unsigned tiles = (unsigned)(((g.M + big::BM - 1) / big::BM) * ((g.N + ncols - 1) / ncols));
    dim3 grid(tiles, 1, nb);
    if (g.out_dt == BF16)
      hipLaunchKernelGGL(big::gemm_nt_big<bf16_t>, grid, dim3(big::NTH), big::LDS, s, g);
    else
      hipLaunchKernelGGL(big::gemm_nt_big<float>, grid, dim3(big::NTH), big::LDS, s, g);
    return hipGetLastError();
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

hipError_t launch_fw_states(const StateArgs& a, hipStream_t s) {
  if (a.nwrites <= 0) return hipSuccess;
  const int nb = a.batch > 0 ? a.batch : 1;
  const bool mf = a.in_dt == BF16 && a.lda % 8 == 0 && a.ldb % 8 == 0 && a.chunk % 8 == 0;
  if (mf) {
    static bool attr = false;
    if (!attr) {
      (void)hipFuncSetAttribute((const void*)fw_states_mfma<float>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)GEMM_LDS);
      (void)hipFuncSetAttribute((const void*)fw_states_mfma<bf16_t>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)GEMM_LDS);
      attr = true;
    }
    dim3 grid((a.d + BM - 1) / BM, (a.f + BN - 1) / BN, nb);
    if (a.st_dt == BF16)
      hipLaunchKernelGGL(fw_states_mfma<bf16_t>, grid, dim3(NT), GEMM_LDS, s, a);
    else
      hipLaunchKernelGGL(fw_states_mfma<float>, grid, dim3(NT), GEMM_LDS, s, a);
    return hipGetLastError();
  }
  dim3 grid((a.d + SB - 1) / SB, (a.f + SB - 1) / SB, nb);
  if (a.in_dt == BF16) {
    if (a.st_dt == BF16)
      hipLaunchKernelGGL((fw_states_simple<bf16_t, bf16_t>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((fw_states_simple<bf16_t, float>), grid, dim3(256), 0, s, a);
  } else {
    if (a.st_dt == BF16)
      hipLaunchKernelGGL((fw_states_simple<float, bf16_t>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((fw_states_simple<float, float>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace ttcd
