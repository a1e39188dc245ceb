// PagedAttention decode: dispatch between the vector-ALU kernels (one
// source file per cache element type) and the matrix-core fp8 kernel, the
// split-K reduce kernel, and the decode step (store + decode).

#include <hip/hip_runtime.h>

#include <cmath>

#include "decode_common.h"

namespace pkv {
namespace valu {
// defined in decode_valu.h, instantiated in decode_{f32,bf16,fp8}.hip
template <int KV>
int launch_valu(const DecodeArgs& a, bool store, hipStream_t st);
template <int KV>
int valu_heads_per_wg(const DecodeArgs& a);
template <int KV>
int launch_valu_sk(const DecodeArgs& a, bool store, hipStream_t st);
template <int KV>
int valu_sk_workers(const DecodeArgs& a);
extern template int launch_valu<PKV_F32>(const DecodeArgs&, bool, hipStream_t);
extern template int launch_valu<PKV_BF16>(const DecodeArgs&, bool, hipStream_t);
extern template int launch_valu<PKV_FP8_E4M3>(const DecodeArgs&, bool, hipStream_t);
extern template int valu_heads_per_wg<PKV_F32>(const DecodeArgs&);
extern template int valu_heads_per_wg<PKV_BF16>(const DecodeArgs&);
extern template int valu_heads_per_wg<PKV_FP8_E4M3>(const DecodeArgs&);
extern template int launch_valu_sk<PKV_F32>(const DecodeArgs&, bool, hipStream_t);
extern template int launch_valu_sk<PKV_BF16>(const DecodeArgs&, bool, hipStream_t);
extern template int launch_valu_sk<PKV_FP8_E4M3>(const DecodeArgs&, bool, hipStream_t);
extern template int valu_sk_workers<PKV_F32>(const DecodeArgs&);
extern template int valu_sk_workers<PKV_BF16>(const DecodeArgs&);
extern template int valu_sk_workers<PKV_FP8_E4M3>(const DecodeArgs&);
}  // namespace valu

namespace {

using namespace dec;

// Combine n partials of one (sequence, query head) into output row `oi`:
// partial p is row row0 + p*stride of o (D floats each) and of (m, l) (2
// floats each); out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p with
// M = max_p m_p.  All 256 threads of the workgroup take part.
template <int D, bool F32OUT>
__device__ __forceinline__ void merge_partials(void* __restrict__ out, size_t oi,
                                               const float* __restrict__ ws_o,
                                               const float* __restrict__ ws_ml, size_t row0,
                                               size_t stride, int n) {
  constexpr int DQ = D / 4;      // float4 columns of a row
  constexpr int PL = 256 / DQ;   // partials handled in parallel
  __shared__ f32x4 o_red[PL][DQ];
  __shared__ float l_red[PL];
  __shared__ float mx_red[256];
  const int tid = threadIdx.x;

  float mx = -INFINITY;
  for (int p = tid; p < n; p += 256) mx = fmaxf(mx, ws_ml[(row0 + p * stride) * 2]);
  mx_red[tid] = mx;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (tid < k) mx_red[tid] = fmaxf(mx_red[tid], mx_red[tid + k]);
    __syncthreads();
  }
  const float M = mx_red[0];

  const int dq = tid % DQ, pl = tid / DQ;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  if (M != -INFINITY) {
    for (int p = pl; p < n; p += PL) {
      const size_t pi = row0 + p * stride;
      const float f = __builtin_amdgcn_exp2f(ws_ml[pi * 2] - M);
      l = fmaf(ws_ml[pi * 2 + 1], f, l);
      const f32x4 v = *(const f32x4*)(ws_o + pi * D + dq * 4);
      o.x = fmaf(v.x, f, o.x);
      o.y = fmaf(v.y, f, o.y);
      o.z = fmaf(v.z, f, o.z);
      o.w = fmaf(v.w, f, o.w);
    }
  }
  o_red[pl][dq] = o;
  if (dq == 0) l_red[pl] = l;
  __syncthreads();
  if (pl == 0) {
    f32x4 t = o_red[0][dq];
    float lt = l_red[0];
    for (int r = 1; r < PL; ++r) {
      const f32x4 u = o_red[r][dq];
      t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
      lt += l_red[r];
    }
    const float inv = lt > 0.f ? 1.f / lt : 0.f;   // a NaN partial stays NaN through t
    const size_t o4 = oi + dq * 4;
    const float r0 = t.x * inv, r1 = t.y * inv, r2 = t.z * inv, r3 = t.w * inv;
    if constexpr (F32OUT) {
      *(f32x4*)((float*)out + o4) = f32x4{r0, r1, r2, r3};
    } else {
      uint16_t* o16 = (uint16_t*)out + o4;
      const uint32_t lo = pack_bf16x2(r0, r1), hi = pack_bf16x2(r2, r3);
      *(uint2*)o16 = make_uint2(lo, hi);
    }
  }
}

// Split-K reduce: one workgroup per (sequence, query head) with > 1 partition.
template <int D, bool F32OUT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(void* __restrict__ out,
                                                            const float* __restrict__ ws,
                                                            const int32_t* __restrict__ part_off,
                                                            int Hq, int total_parts) {
  const int s = blockIdx.x, qh = blockIdx.y;
  const int p0 = part_off[s];
  const int n = part_off[s + 1] - p0;
  if (n <= 1) return;
  merge_partials<D, F32OUT>(out, ((size_t)s * Hq + qh) * D, ws, ws + (size_t)total_parts * Hq * D,
                            (size_t)p0 * Hq + qh, Hq, n);
}

// Stream-K reduce: one workgroup per (sequence, query head).  The item's
// tiles [start, start + n) of the T laid out end to end went to waves
// r(start) .. r(start + n - 1), r(x) = floor(((x + 1) R - 1) / T) being the
// wave whose slice [floor(r T / R), floor((r + 1) T / R)) holds tile x; with
// one wave the output is already written, with several their partials sit in
// consecutive slots r + hg*S + s.  A sequence without tiles gets zeros.
template <int D, bool F32OUT>
__global__ __launch_bounds__(256) void sk_reduce_kernel(void* __restrict__ out,
                                                        const float* __restrict__ ws,
                                                        const int32_t* __restrict__ tile_off,
                                                        int S, int Hq, int Hkv, int hpw, int R,
                                                        int CU) {
  const int s = blockIdx.x, qh = blockIdx.y;
  const int G = Hq / Hkv, groups = G / hpw;
  const int hkv = qh / G, g = (qh % G) / hpw, hh = qh % hpw;
  const int hg = hkv * groups + g;
  const int n = tile_off[s + 1] - tile_off[s];
  const size_t oi = ((size_t)s * Hq + qh) * D;
  if (n <= 0) {
    for (int i = threadIdx.x; i < D; i += 256) {
      if constexpr (F32OUT)
        ((float*)out)[oi + i] = 0.f;
      else
        ((uint16_t*)out)[oi + i] = 0;
    }
    return;
  }
  const int64_t T = (int64_t)CU * Hkv * groups;
  const int64_t start = (int64_t)hg * CU + tile_off[s], last = start + n - 1;
  if (start < 0 || last >= T) {   // offsets that are not running sums ending at CU
    for (int i = threadIdx.x; i < D; i += 256) {
      if constexpr (F32OUT)
        ((float*)out)[oi + i] = NAN;
      else
        ((uint16_t*)out)[oi + i] = 0x7fc0;
    }
    return;
  }
  const int r0 = (int)(((start + 1) * R - 1) / T), r1 = (int)(((last + 1) * R - 1) / T);
  if (r0 == r1) return;
  const size_t slots = (size_t)R + (size_t)Hkv * groups * S;
  const size_t slot0 = (size_t)r0 + (size_t)hg * S + s;
  merge_partials<D, F32OUT>(out, oi, ws, ws + slots * hpw * D, slot0 * hpw + hh, hpw, r1 - r0 + 1);
}

int launch_valu_any(const DecodeArgs& a, bool store, hipStream_t st) {
  switch (a.kv_dtype) {
    case PKV_F32: return valu::launch_valu<PKV_F32>(a, store, st);
    case PKV_BF16: return valu::launch_valu<PKV_BF16>(a, store, st);
    default: return valu::launch_valu<PKV_FP8_E4M3>(a, store, st);
  }
}

}  // namespace

bool decode_supported(pkv_dtype q, pkv_dtype kv, int D, int BS, int G) {
  const bool pair_ok = (q == PKV_F32 && kv == PKV_F32) || (q == PKV_BF16 && kv == PKV_BF16) ||
                       (q == PKV_BF16 && kv == PKV_FP8_E4M3);
  return pair_ok && (D == 64 || D == 128) && (BS == 16 || BS == 32) && G >= 1;
}

int launch_decode(const DecodeArgs& a, void* stream) {
  if (decode_mfma_eligible(a)) return launch_decode_mfma(a, stream);
  return launch_valu_any(a, false, (hipStream_t)stream);
}

bool decode_step_stores_in_kernel(const DecodeArgs& a) {
  const int G = a.Hq / a.Hkv;
  if (decode_mfma_eligible(a)) return G == 8;
  switch (a.kv_dtype) {
    case PKV_F32: return valu::valu_heads_per_wg<PKV_F32>(a) == G;
    case PKV_BF16: return valu::valu_heads_per_wg<PKV_BF16>(a) == G;
    default: return valu::valu_heads_per_wg<PKV_FP8_E4M3>(a) == G;
  }
}

int launch_decode_step(const DecodeArgs& a, void* stream) {
  if (!decode_step_stores_in_kernel(a)) return (int)hipErrorInvalidValue;
  if (decode_mfma_eligible(a)) return launch_decode_mfma(a, stream, true);
  return launch_valu_any(a, true, (hipStream_t)stream);
}

int decode_sk_workers(const DecodeArgs& a) {
  switch (a.kv_dtype) {
    case PKV_F32: return valu::valu_sk_workers<PKV_F32>(a);
    case PKV_BF16: return valu::valu_sk_workers<PKV_BF16>(a);
    default: return valu::valu_sk_workers<PKV_FP8_E4M3>(a);
  }
}

int decode_sk_heads_per_wave(const DecodeArgs& a) {
  switch (a.kv_dtype) {
    case PKV_F32: return valu::valu_heads_per_wg<PKV_F32>(a);
    case PKV_BF16: return valu::valu_heads_per_wg<PKV_BF16>(a);
    default: return valu::valu_heads_per_wg<PKV_FP8_E4M3>(a);
  }
}

// Waves actually used: at most one per tile, so that every wave's slice
// holds a tile and the pieces of an item sit in consecutive slots.
static DecodeArgs clamp_workers(const DecodeArgs& a) {
  DecodeArgs b = a;
  const int groups = a.Hq / a.Hkv / decode_sk_heads_per_wave(a);
  const int64_t T = (int64_t)a.sk_cu * a.Hkv * groups;
  if (T < b.sk_workers) b.sk_workers = T > 1 ? (int)T : 1;
  return b;
}

int launch_decode_sk(const DecodeArgs& a0, bool store, void* stream) {
  const DecodeArgs a = clamp_workers(a0);
  hipStream_t st = (hipStream_t)stream;
  switch (a.kv_dtype) {
    case PKV_F32: return valu::launch_valu_sk<PKV_F32>(a, store, st);
    case PKV_BF16: return valu::launch_valu_sk<PKV_BF16>(a, store, st);
    default: return valu::launch_valu_sk<PKV_FP8_E4M3>(a, store, st);
  }
}

int launch_sk_reduce(const DecodeArgs& a0, void* stream) {
  const DecodeArgs a = clamp_workers(a0);
  hipStream_t st = (hipStream_t)stream;
  const int hpw = decode_sk_heads_per_wave(a);
  dim3 grid(a.S, a.Hq), block(256);
  const bool f32 = a.q_dtype == PKV_F32;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, st, a.out, (const float*)a.ws, a.tile_off, a.S, a.Hq,
                       a.Hkv, hpw, a.sk_workers, a.sk_cu);
  };
  if (a.D == 64)
    f32 ? go(sk_reduce_kernel<64, true>) : go(sk_reduce_kernel<64, false>);
  else
    f32 ? go(sk_reduce_kernel<128, true>) : go(sk_reduce_kernel<128, false>);
  return (int)hipGetLastError();
}

int launch_splitk_reduce(void* out, const float* ws, const int32_t* part_off, int S, int Hq, int D,
                         int total_parts, pkv_dtype out_dtype, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  dim3 grid(S, Hq), block(256);
  const bool f32 = out_dtype == PKV_F32;
  if (D == 64) {
    if (f32)
      hipLaunchKernelGGL((splitk_reduce_kernel<64, true>), grid, block, 0, st, out, ws, part_off, Hq, total_parts);
    else
      hipLaunchKernelGGL((splitk_reduce_kernel<64, false>), grid, block, 0, st, out, ws, part_off, Hq, total_parts);
  } else {
    if (f32)
      hipLaunchKernelGGL((splitk_reduce_kernel<128, true>), grid, block, 0, st, out, ws, part_off, Hq, total_parts);
    else
      hipLaunchKernelGGL((splitk_reduce_kernel<128, false>), grid, block, 0, st, out, ws, part_off, Hq, total_parts);
  }
  return (int)hipGetLastError();
}

}  // namespace pkv
