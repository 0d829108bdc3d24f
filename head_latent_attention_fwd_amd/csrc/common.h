// Device-side helpers shared by the gfx950 kernels of the MLA library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bfloat16 storage (upper half of an fp32 word)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

#define MLA_DEV __device__ __forceinline__

MLA_DEV float bf2f(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even float -> bf16 (NaN stays NaN): gfx950's
// v_cvt_pk_bf16_f32, which the compiler emits for these conversions.
MLA_DEV bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// Two floats -> packed bf16 pair (lo in bits 0..15).
MLA_DEV uint32_t pack2bf(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2){lo, hi}, bf16x2));
}

MLA_DEV float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
MLA_DEV float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Generic element conversion used by the kernels templated on storage type.
template <typename T> MLA_DEV float to_f(T v);
template <> MLA_DEV float to_f<float>(float v) { return v; }
template <> MLA_DEV float to_f<bf16_t>(bf16_t v) { return bf2f(v); }
template <typename T> MLA_DEV T from_f(float v);
template <> MLA_DEV float from_f<float>(float v) { return v; }
template <> MLA_DEV bf16_t from_f<bf16_t>(float v) { return f2bf(v); }

MLA_DEV float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
MLA_DEV float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Logical block index -> block index remapped so that consecutive logical
// ids land on the same XCD.  The dispatcher hands workgroup b to XCD b % 8,
// so logical tile ranges [start_x, start_x + count_x) are assigned to XCD x.
MLA_DEV int xcd_remap(int b, int nblocks) {
  const int nx = 8;
  int x = b % nx, slot = b / nx;
  int base = nblocks / nx, rem = nblocks % nx;
  int start = x * base + (x < rem ? x : rem);
  return start + slot;
}

#define MLA_LDS __attribute__((address_space(3)))

// Position of sequence b in a decode step: the caller's per-sequence table
// (device int32, each entry clamped into [0, pmax] so that no value can
// address outside the cache) or, without a table, the uniform position.
MLA_DEV int seq_position(const int* __restrict__ pos, int b, int uniform, int pmax) {
  return pos ? min(max(pos[b], 0), pmax) : uniform;
}

// RoPE of 8 consecutive bf16 features (4 pairs (2i, 2i+1), pair index
// pair0 + i) at table row `pos`: (a, b) -> (a cos - b sin, a sin + b cos),
// computed in fp32 and rounded back to bf16.
MLA_DEV u32x4 rope8_bf16(u32x4 v, const float* __restrict__ rcos, const float* __restrict__ rsin,
                         long pos, int n_pairs, int pair0) {
  const floatx4 c = *(const floatx4*)(rcos + pos * n_pairs + pair0);
  const floatx4 s = *(const floatx4*)(rsin + pos * n_pairs + pair0);
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = lo_bf(v[i]), b = hi_bf(v[i]);
    o[i] = pack2bf(a * c[i] - b * s[i], a * s[i] + b * c[i]);
  }
  return o;
}
