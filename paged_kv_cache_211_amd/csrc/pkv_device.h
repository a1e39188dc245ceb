// Device-side helpers for gfx950 (CDNA4, wave64): element conversions and
// cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two bf16 from two fp32, packed low = a, high = b (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

// sum of the two bf16 products of a and b, plus c, in fp32 (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// Two E4M3FN codes (bytes 0,1, or 2,3 when HIGH) of w -> two fp32, exact
// (v_cvt_pk_f32_fp8).
template <bool HIGH>
__device__ __forceinline__ f32x2 fp8x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HIGH);
}

// fp32 -> OCP E4M3FN code: round to nearest, ties to even; |y| >= 448
// saturates to 448; NaN -> 0x7F.  Bit-level, independent of any hardware
// conversion mode.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;              // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;      // >= 448 (also inf)
  if (a >= 0x3c800000u) {                         // >= 2^-6: normal in E4M3
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);  // RNE at mantissa bit 20
    return sign | ((((r >> 23) - 120u) << 3) | ((r >> 20) & 7u));
  }
  // subnormal range: the code is round(|y| * 2^9) (k = 8 is the smallest normal)
  const float k = __builtin_rintf(__uint_as_float(a) * 512.0f);
  return sign | (uint32_t)k;
}

// ---- cross-lane helpers (wave64) -------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf,
                                                            0xf, false));
}
// DPP controls: quad_perm(1,0,3,2) = 0xB1, quad_perm(2,3,0,1) = 0x4E,
// row_ror:4 = 0x124, row_ror:8 = 0x128.

// Reductions within each row of 16 lanes (every lane gets the row result).
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x124>(v));
  v = fmaxf(v, dpp<0x128>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x124>(v);
  v += dpp<0x128>(v);
  return v;
}

__device__ __forceinline__ float xor_lanes(float v, int mask) { return __shfl_xor(v, mask, 64); }

// v[l] + v[l ^ 32] in every lane, without LDS: v_permlane32_swap exchanges the
// upper half of one register copy with the lower half of the other.
__device__ __forceinline__ float sum_xor32(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// v[l] + v[l ^ 16] (v_permlane16_swap exchanges odd rows with even rows).
__device__ __forceinline__ float sum_xor16(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// fp32 -> bf16 bits with the hardware conversion (round to nearest even).
__device__ __forceinline__ uint16_t cvt_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// ---- slot scatter of one 16-byte key unit and the matching value elements ----
// Token t's kv head h, key unit c (elements c*X .. c*X+X-1 of the row) goes to
// slot `slot` = block * BS + offset.  Pool layout: key [NB][H][D/X][BS][X],
// value [NB][H][D][BS] (X = 16 / element size of the cache).  CACHE selects
// the stored type; bf16 -> fp8 stores E4M3FN(fp32(x) * inv) (k_inv for keys,
// v_inv for values).  The caller has checked 0 <= slot < NB * BS.
template <int CACHE>
__device__ __forceinline__ void write_kv_unit(const void* __restrict__ key,
                                              const void* __restrict__ value,
                                              uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                                              int t, int h, int c, int slot, int H, int D, int BS,
                                              float k_inv, float v_inv) {
  constexpr int E = CACHE == PKV_F32 ? 4 : CACHE == PKV_BF16 ? 2 : 1;
  constexpr int X = 16 / E;
  const int b = slot / BS, o = slot % BS;
  const size_t row = ((size_t)t * H + h) * D + (size_t)c * X;   // first source element
  const size_t kdst = ((((size_t)b * H + h) * (D / X) + c) * BS + o) * 16;
  const size_t vdst0 = (((size_t)b * H + h) * D + (size_t)c * X) * BS + o;  // element index

  if constexpr (CACHE == PKV_F32) {
    const f32x4 k4 = *(const f32x4*)((const float*)key + row);
    const f32x4 v4 = *(const f32x4*)((const float*)value + row);
    *(f32x4*)(kc + kdst) = k4;
    float* vd = (float*)vc + vdst0;
    vd[0] = v4.x; vd[BS] = v4.y; vd[2 * BS] = v4.z; vd[3 * BS] = v4.w;
  } else if constexpr (CACHE == PKV_BF16) {
    const u32x4 k8 = *(const u32x4*)((const uint16_t*)key + row);
    const u32x4 v8 = *(const u32x4*)((const uint16_t*)value + row);
    *(u32x4*)(kc + kdst) = k8;
    uint16_t* vd = (uint16_t*)vc + vdst0;
    const uint32_t vw[4] = {v8.x, v8.y, v8.z, v8.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      vd[(2 * i) * BS] = (uint16_t)(vw[i] & 0xffffu);
      vd[(2 * i + 1) * BS] = (uint16_t)(vw[i] >> 16);
    }
  } else {  // bf16 -> fp8 E4M3FN, quantise on write
    const uint16_t* ks = (const uint16_t*)key + row;
    const uint16_t* vs = (const uint16_t*)value + row;
    const u32x4 ka = *(const u32x4*)ks, kb = *(const u32x4*)(ks + 8);
    const u32x4 va = *(const u32x4*)vs, vb = *(const u32x4*)(vs + 8);
    const uint32_t kw[8] = {ka.x, ka.y, ka.z, ka.w, kb.x, kb.y, kb.z, kb.w};
    const uint32_t vw[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
    uint32_t kout[4] = {0, 0, 0, 0};
    uint8_t* vd = vc + vdst0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t k0 = f32_to_e4m3(bf16_lo(kw[i]) * k_inv);
      const uint32_t k1 = f32_to_e4m3(bf16_hi(kw[i]) * k_inv);
      kout[i / 2] |= (k0 | (k1 << 8)) << (16 * (i % 2));
      vd[(2 * i) * BS] = (uint8_t)f32_to_e4m3(bf16_lo(vw[i]) * v_inv);
      vd[(2 * i + 1) * BS] = (uint8_t)f32_to_e4m3(bf16_hi(vw[i]) * v_inv);
    }
    *(u32x4*)(kc + kdst) = u32x4{kout[0], kout[1], kout[2], kout[3]};
  }
}

}  // namespace pkv
