// Device helpers shared by the gfx950 NVFP4 kernels.
//
// Number formats (NVFP4: E2M1 elements, one FP8 scale per 16 elements, one
// FP32 tensor scale — neurohive.io LongLive-2.0 summary, NVFP4 paragraph;
// tailorednewshub.com "LongLive-2.0: Infraestructura paralela NVFP4 para video
// largo", section "Entrenamiento NVFP4").  The FP8 flavour is OCP E4M3FN.
//
// Hardware conversions used here were checked on gfx950 against the format
// definitions before use:
//   * v_cvt_scalef32_pk_fp4_f32 with scale 1.0 equals round-to-nearest-even,
//     saturating E2M1 (sign kept for values that round to zero) on every
//     finite float32;
//   * v_cvt_scalef32_pk_f16_fp4 / _f32_fp4 decode E2M1 exactly when the scale
//     is 1.0 (the scale operand only contributes its exponent);
//   * v_cvt_f32_fp8 decodes all 256 E4M3FN bytes exactly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr float kGlobalMax = 2688.0f;  // E2M1 max 6 * E4M3 max 448
constexpr int kBlock = 16;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// E4M3FN byte of a non-negative finite float32, round-to-nearest-even,
// saturating at 448 (0x7E).  Pure integer logic on the float32 bit pattern for
// the normal range; the subnormal range (u < 2^-6) is u * 2^9 rounded to an
// integer (exact scaling, hardware round-to-nearest-even).
__device__ __forceinline__ uint32_t e4m3_rne_satfinite(float u) {
  const uint32_t b = __float_as_uint(u);
  if (b >= 0x43E00000u) return 0x7Eu;              // u >= 448
  if (b >= 0x3C800000u) {                          // 2^-6 <= u < 448
    const uint32_t e = (b >> 23) - 120u;           // E4M3 biased exponent, 1..15
    const uint32_t m = b & 0x7FFFFFu;
    uint32_t v = (e << 3) | (m >> 20);
    const uint32_t rem = m & 0xFFFFFu;
    v += (rem > 0x80000u) || (rem == 0x80000u && (v & 1u));
    return v;                                      // <= 0x7E because u < 448
  }
  return (uint32_t)__builtin_rintf(u * 512.0f);    // 0..8 (8 = 2^-6, code 0x08)
}

// float32 value of an E4M3FN byte (exact).
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8(byte, 0);
}

// bf16 bit pattern of a finite float32, round-to-nearest-even.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return b >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Max over the 64 lanes of a wavefront (every lane gets the result).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// A 16-byte load, non-temporal (last use of the data: streamed past the
// caches) or temporal (the data is read again soon, e.g. by the encode pass
// right after the amax pass: it can then come from the Infinity Cache).
template <bool NT, typename T>
__device__ __forceinline__ T load_hint(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// Load 16 consecutive elements (16-byte aligned) as float32.
template <int DT, bool NT = true>
__device__ __forceinline__ void load16(const void* __restrict__ base, int64_t elem_off, float (&v)[16]) {
  if constexpr (DT == 0) {
    const float4_t* p = reinterpret_cast<const float4_t*>(static_cast<const float*>(base) + elem_off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4_t q = load_hint<NT>(p + i);
      v[4 * i + 0] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
    }
    return;
  }
  const u32x4_t* p = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(base) + elem_off);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const u32x4_t q = load_hint<NT>(p + i);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j + 0] = __uint_as_float(w[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
}

// One element of a dense tensor as float32 (scalar load, any alignment).
template <int DT>
__device__ __forceinline__ float load1(const void* __restrict__ base, int64_t off) {
  if constexpr (DT == 0) return static_cast<const float*>(base)[off];
  else return bf16_to_f32(static_cast<const uint16_t*>(base)[off]);
}

// 16-point random Hadamard transform of one block, in place:
// v <- (1/4) H16 diag(d) v with d_j = -1 iff bit j of mask; fixed float32
// order (sign flip, butterflies of stride 1, 2, 4, 8, then * 0.25).
__device__ __forceinline__ void rht16(float (&v)[16], uint32_t mask) {
#pragma unroll
  for (int i = 0; i < 16; ++i)
    v[i] = __uint_as_float(__float_as_uint(v[i]) ^ (((mask >> i) & 1u) << 31));
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i & h) continue;
      const float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] *= 0.25f;
}

// Scale part of the recipe for one block: given the block amax `a` and the
// domain's tensor scale S, return the E4M3 byte and the element multiplier
// r = 1 / (f32(s_b) * S) (0 when that product is 0).  TARGET is the E2M1
// value the block maximum maps to: 6 in the core recipe, 4 for the second
// candidate of Four Over Six.
template <int TARGET = 6>
__device__ __forceinline__ uint32_t block_scale(float a, float S, float& r) {
  const float t = a / (float)TARGET;
  const float u = S > 0.0f ? t / S : 0.0f;
  const uint32_t sig = e4m3_rne_satfinite(u);
  const float d = e4m3_to_f32(sig) * S;
  r = d > 0.0f ? 1.0f / d : 0.0f;
  return sig;
}

// Encode 16 elements with multiplier r into 8 bytes of packed E2M1 codes
// (low nibble = even element).  The byte selector of the convert must be a
// compile-time constant, hence the explicit sequence.
__device__ __forceinline__ u32x2_t encode16(const float (&v)[16], float r) {
  uint32_t w0 = 0, w1 = 0;
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, v[0] * r, v[1] * r, 1.0f, 0);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, v[2] * r, v[3] * r, 1.0f, 1);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, v[4] * r, v[5] * r, 1.0f, 2);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, v[6] * r, v[7] * r, 1.0f, 3);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, v[8] * r, v[9] * r, 1.0f, 0);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, v[10] * r, v[11] * r, 1.0f, 1);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, v[12] * r, v[13] * r, 1.0f, 2);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, v[14] * r, v[15] * r, 1.0f, 3);
  return u32x2_t{w0, w1};
}

// Squared decode error of one encoded block (Four Over Six): with
// x'_i = f32(e2m1_i * s_b) * S the standard decode, E = sum (x_i - x'_i)^2,
// every operation a separately rounded float32 operation, summed from
// element 0 to 15 — the exact order the CPU reference uses, because the
// comparison of two such errors decides which bytes are stored.
__device__ __forceinline__ void decode8_f32(uint32_t w, float* o);
__device__ __forceinline__ float block_sq_error(const float (&v)[16], u32x2_t codes, uint32_t sig, float S) {
#pragma clang fp contract(off)
  float e2[16];
  decode8_f32(codes.x, e2);
  decode8_f32(codes.y, e2 + 8);
  const float sf = e4m3_to_f32(sig);
  float E = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float xd = (e2[i] * sf) * S;
    const float d = v[i] - xd;
    E = E + d * d;
  }
  return E;
}

// Decode 8 packed E2M1 codes (one dword, low nibble first) to float32.
__device__ __forceinline__ void decode8_f32(uint32_t w, float* o) {
  const float2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const float2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const float2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const float2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  o[0] = p0.x; o[1] = p0.y; o[2] = p1.x; o[3] = p1.y;
  o[4] = p2.x; o[5] = p2.y; o[6] = p3.x; o[7] = p3.y;
}

}  // namespace nvfp4
