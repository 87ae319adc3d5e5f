// Shared device helpers for the gfx950 kernels of the IP-TTCD layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 is carried as raw uint16_t bits in memory.
typedef uint16_t bf16_t;

#define TTCD_DEV __device__ __forceinline__

TTCD_DEV float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// round to nearest even (hardware conversion on gfx950)
TTCD_DEV bf16_t f2bf(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(bf16_t, h);
}

// two values in one packed conversion (v_cvt_pk_bf16_f32), lo in bits 0..15
TTCD_DEV uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){lo, hi}, bf16x2v));
}

template <typename T> struct elem;
template <> struct elem<float> {
  static TTCD_DEV float ld(const float* p) { return *p; }
  static TTCD_DEV void st(float* p, float v) { *p = v; }
};
template <> struct elem<bf16_t> {
  static TTCD_DEV float ld(const bf16_t* p) { return bf2f(*p); }
  static TTCD_DEV void st(bf16_t* p, float v) { *p = f2bf(v); }
};

template <typename T> TTCD_DEV float ldf(const T* p) { return elem<T>::ld(p); }
template <typename T> TTCD_DEV void stf(T* p, float v) { elem<T>::st(p, v); }

// 16-byte vector load/store through LDS or global memory.
TTCD_DEV u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
TTCD_DEV void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

TTCD_DEV bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// MFMA wrappers (CDNA4 dense bf16: 32x32x16 and 16x16x32, fp32 accumulate).
TTCD_DEV f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

TTCD_DEV f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

TTCD_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

TTCD_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
TTCD_DEV float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Logical tile id -> (tile row, tile column), gm tile rows at a time with the
// row index fastest: the few dozen workgroups an XCD runs at once then cover a
// gm x (that / gm) block of output tiles and share its A and B panels in L2,
// instead of one A panel and a sweep over every B panel.
TTCD_DEV void grouped_tile(uint32_t lid, int ntm, int ntn, int gm, int& tm, int& tn) {
  const int per_group = gm * ntn;
  const int first = (int)(lid / per_group) * gm;
  const int gsz = ntm - first < gm ? ntm - first : gm;
  const int in = (int)(lid % per_group);
  tm = first + in % gsz;
  tn = in / gsz;
}

// Map a linear workgroup id onto a logical tile id so that the tiles each
// XCD receives (hardware dispatches workgroup w to XCD w % 8) are
// contiguous in logical order: neighbouring tiles then share that XCD's L2.
TTCD_DEV uint32_t xcd_remap(uint32_t w, uint32_t total) {
  const uint32_t nx = 8;
  uint32_t q = total / nx, r = total % nx;
  uint32_t x = w % nx, k = w / nx;
  return x * q + (x < r ? x : r) + k;
}
