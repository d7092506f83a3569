// Device-side helpers shared by the HSTU kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define HSTU_DEV __device__ __forceinline__
// for lambdas inside kernels: an outlined lambda would move captured arrays to scratch
#define HSTU_INLINE_LAMBDA __attribute__((always_inline))

// -log2(e): the attention kernels evaluate exp(-s) as exp2(s * -log2(e)).
#define HSTU_NEG_LOG2E (-1.4426950408889634f)
#define HSTU_LN2 0.6931471805599453f

HSTU_DEV float bf2f(bf16 x) { return (float)x; }
HSTU_DEV bf16 f2bf(float x) { return (bf16)x; }  // round to nearest even (v_cvt_pk_bf16_f32)

HSTU_DEV uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (bf16)lo;
  v[1] = (bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Exact SiLU for epilogues: z / (1 + e^-z) with hardware exp2 and reciprocal.
HSTU_DEV float silu_f(float z) {
  float e = __builtin_amdgcn_exp2f(z * HSTU_NEG_LOG2E);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}
HSTU_DEV float sigmoid_f(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * HSTU_NEG_LOG2E));
}
HSTU_DEV float silu_grad_f(float z) {
  float s = sigmoid_f(z);
  return s * (1.0f + z * (1.0f - s));
}

// MFMA wrappers (bf16 in, fp32 accumulate).
//  32x32x16: A lane l holds row l%32, k = 8*(l/32)+e; B lane l holds column l%32,
//  the same k; C lane l register r holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
HSTU_DEV f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS tiles for MFMA operands: R rows (the M or N index) x C columns (the k
// index) of bf16, row stride C+8 elements.  The 16-byte column group of a
// row is XOR-swizzled by a function of the row so that transposed stores
// (one dword per lane, eight rows apart) spread over the banks while 16-byte
// row reads stay contiguous and aligned.
template <int C>
struct LdsTile {
  static constexpr int S_DW = C / 2 + 4;  // row stride in dwords
  static constexpr int BYTES_PER_ROW = S_DW * 4;
  HSTU_DEV static int swz(int row) {
    return (C >= 64 ? ((row >> 3) & 3) : ((row >> 3) & 1)) << 3;
  }
  // dword offset of (row, dword column dw)
  HSTU_DEV static int off(int row, int dw) { return row * S_DW + (dw ^ swz(row)); }
  static constexpr int bytes(int rows) { return rows * BYTES_PER_ROW; }
};

// Position of key kk inside a 16-key group of a transposed (k-major) tile so
// that the eight keys one MFMA lane group consumes are contiguous: bits 2
// and 3 of the key index are swapped.  The S^T accumulator of 32x32 MFMA
// leaves lane group g holding keys {4g..4g+3, 8+4g..8+4g+3} of each 16.
HSTU_DEV int kperm(int kk) {
  return (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

HSTU_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
HSTU_DEV int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}
HSTU_DEV int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

// Global 16-byte load / store helpers.
HSTU_DEV u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
HSTU_DEV void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
