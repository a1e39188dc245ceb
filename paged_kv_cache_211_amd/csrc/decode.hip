// PagedAttention decode: dispatch between the vector-ALU kernels (one
// source file per cache element type) and the matrix-core fp8 kernel, the
// split-K reduce kernel, and the decode step (store + decode).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <type_traits>

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

// Partial rows one thread of the reduce loads at once when a sequence has
// too many partials for four each (long contexts split into tens of
// partitions): one memory round trip instead of one per four rows.
constexpr int kReduceRowsInFlight = 32;

// Combine the n partials of HG query heads of one sequence: partial p of head
// hh is row row0 + p*pstride + hh of o (D floats each) and of (m, l) (2
// floats each); out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p with
// M = max_p m_p, written to out rows oi0 + hh*D.  The 256 threads first take
// (piece, head) pairs for the maxima and the weights (kept in LDS, a chunk
// of pieces at a time); then PL piece lanes each sum every PL-th piece over
// the NV = HG*D/4 float4 columns, four pieces' loads in flight, and LDS adds
// the lanes.  With at most 4*PL pieces (every sequence of up to a few
// partitions), or kReduceRowsInFlight*PL, all loads -- the (m, l) pairs and
// every partial row -- go out at once: the weights then come from registers
// and the partial rows are already in flight while the maxima are reduced,
// one memory round trip in all instead of three or more; up to twice
// kReduceRowsInFlight*PL pieces take two.
template <int D, bool F32OUT, int HG, bool WIDE = false>
__device__ __forceinline__ void merge_heads(void* __restrict__ out, size_t oi0,
                                            const float* __restrict__ ws_o,
                                            const float* __restrict__ ws_ml, size_t row0,
                                            size_t pstride, int n) {
  constexpr int NT = 256, PSTEP = NT / HG, PCH = 2048 / HG, NV = HG * D / 4, PL = NT / NV;
  static_assert(NV * PL == NT, "thread layout");
  __shared__ float red[NT];
  __shared__ float w_lds[PCH][HG];
  __shared__ float m_s[HG], l_s[HG];
  __shared__ f32x4 part[PL][NV];
  const int tid = threadIdx.x, hh_t = tid % HG, p_t = tid / HG;
  const int pl = tid / NV, e = tid % NV;
  const int hh_e = e * 4 / D, d4 = e * 4 % D;   // this thread's float4 column

  // combine the PL lanes' sums and the row sums, normalise, store
  auto finish = [&](f32x4 acc, float lsum) {
    part[pl][e] = acc;
    red[tid] = lsum;
    __syncthreads();
    for (int k = NT / 2; k >= HG; k >>= 1) {
      if (tid < k) red[tid] += red[tid + k];
      __syncthreads();
    }
    if (tid < HG) l_s[tid] = red[tid];
    __syncthreads();
    if (pl == 0) {
#pragma unroll
      for (int q = 1; q < PL; ++q) {
        const f32x4 u = part[q][e];
        acc.x += u.x; acc.y += u.y; acc.z += u.z; acc.w += u.w;
      }
      const float L = l_s[hh_e];
      const float inv = L > 0.f ? 1.f / L : 0.f;   // a NaN partial stays NaN through acc
      const float r0 = acc.x * inv, r1 = acc.y * inv, r2 = acc.z * inv, r3 = acc.w * inv;
      const size_t o4 = oi0 + (size_t)hh_e * D + d4;
      if constexpr (F32OUT) {
        *(f32x4*)((float*)out + o4) = f32x4{r0, r1, r2, r3};
      } else {
        uint16_t* o16 = (uint16_t*)out + o4;
        *(uint2*)o16 = make_uint2(pack_bf16x2(r0, r1), pack_bf16x2(r2, r3));
      }
    }
  };

  // all loads at once: UNR partial rows per piece lane (n <= UNR * PL)
  auto one_trip = [&](auto unr) {
    constexpr int UNR = decltype(unr)::value;
    float m_own = -INFINITY, l_own = 0.f;
    if (p_t < n) {
      const f32x2 ml = *(const f32x2*)(ws_ml + (row0 + (size_t)p_t * pstride + hh_t) * 2);
      m_own = ml.x;
      l_own = ml.y;
    }
    const float* op = ws_o + (row0 + hh_e) * D + d4;
    const size_t ps = pstride * D;
    f32x4 v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int p = pl + u * PL;
      v[u] = p < n ? *(const f32x4*)(op + (size_t)p * ps) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    red[tid] = m_own;
    __syncthreads();
    for (int k = NT / 2; k >= HG; k >>= 1) {
      if (tid < k) red[tid] = fmaxf(red[tid], red[tid + k]);
      __syncthreads();
    }
    const float M_t = red[hh_t];
    const float w_own = p_t < n && M_t != -INFINITY ? __builtin_amdgcn_exp2f(m_own - M_t) : 0.f;
    if (p_t < n) w_lds[p_t][hh_t] = w_own;
    __syncthreads();
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int p = pl + u * PL;
      if (p < n) {
        const float w = w_lds[p][hh_e];
        acc.x = fmaf(v[u].x, w, acc.x);
        acc.y = fmaf(v[u].y, w, acc.y);
        acc.z = fmaf(v[u].z, w, acc.z);
        acc.w = fmaf(v[u].w, w, acc.w);
      }
    }
    __syncthreads();   // every thread has read red / w_lds before finish reuses red
    finish(acc, p_t < n ? l_own * w_own : 0.f);
  };
  // up to twice that: the (m, l) pairs (two per thread) and the first half
  // of the partial rows go out at once, the second half as soon as the
  // first is summed -- two round trips
  auto two_trips = [&]() {
    constexpr int UNR = kReduceRowsInFlight;
    float m_own[2], l_own[2], w_own[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int p = p_t + k * PSTEP;
      m_own[k] = -INFINITY;
      l_own[k] = 0.f;
      if (p < n) {
        const f32x2 ml = *(const f32x2*)(ws_ml + (row0 + (size_t)p * pstride + hh_t) * 2);
        m_own[k] = ml.x;
        l_own[k] = ml.y;
      }
    }
    const float* op = ws_o + (row0 + hh_e) * D + d4;
    const size_t ps = pstride * D;
    f32x4 v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int p = pl + u * PL;
      v[u] = p < n ? *(const f32x4*)(op + (size_t)p * ps) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    red[tid] = fmaxf(m_own[0], m_own[1]);
    __syncthreads();
    for (int k = NT / 2; k >= HG; k >>= 1) {
      if (tid < k) red[tid] = fmaxf(red[tid], red[tid + k]);
      __syncthreads();
    }
    const float M_t = red[hh_t];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int p = p_t + k * PSTEP;
      w_own[k] = p < n && M_t != -INFINITY ? __builtin_amdgcn_exp2f(m_own[k] - M_t) : 0.f;
      if (p < n) w_lds[p][hh_t] = w_own[k];
    }
    __syncthreads();
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int pb = half * UNR * PL;
      if (half == 1) {
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int p = pb + pl + u * PL;
          v[u] = p < n ? *(const f32x4*)(op + (size_t)p * ps) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int p = pb + pl + u * PL;
        if (p < n) {
          const float w = w_lds[p][hh_e];
          acc.x = fmaf(v[u].x, w, acc.x);
          acc.y = fmaf(v[u].y, w, acc.y);
          acc.z = fmaf(v[u].z, w, acc.z);
          acc.w = fmaf(v[u].w, w, acc.w);
        }
      }
    }
    __syncthreads();   // every thread has read red / w_lds before finish reuses red
    finish(acc, l_own[0] * w_own[0] + l_own[1] * w_own[1]);
  };
  if (n <= 4 * PL && n <= PSTEP) {
    one_trip(std::integral_constant<int, 4>());
    return;
  }
  if constexpr (WIDE) {
    if (n <= kReduceRowsInFlight * PL && n <= PSTEP) {
      one_trip(std::integral_constant<int, kReduceRowsInFlight>());
      return;
    }
    if (n <= 2 * kReduceRowsInFlight * PL && n <= 2 * PSTEP) {
      two_trips();
      return;
    }
  }

  float mx = -INFINITY;
  for (int p = p_t; p < n; p += PSTEP) mx = fmaxf(mx, ws_ml[(row0 + p * pstride + hh_t) * 2]);
  red[tid] = mx;
  __syncthreads();
  for (int k = NT / 2; k >= HG; k >>= 1) {
    if (tid < k) red[tid] = fmaxf(red[tid], red[tid + k]);
    __syncthreads();
  }
  if (tid < HG) m_s[tid] = red[tid];
  __syncthreads();
  const float M_t = m_s[hh_t];

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
  for (int pc = 0; pc < n; pc += PCH) {
    const int np = min(PCH, n - pc);
    for (int p = p_t; p < np; p += PSTEP) {
      const float* ml = ws_ml + (row0 + (size_t)(pc + p) * pstride + hh_t) * 2;
      const float w = M_t == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[0] - M_t);
      w_lds[p][hh_t] = w;
      lsum = fmaf(ml[1], w, lsum);
    }
    __syncthreads();
    const float* op = ws_o + (row0 + (size_t)pc * pstride + hh_e) * D + d4;
    const size_t ps = pstride * D;
    int p = pl;
    for (; p + 3 * PL < np; p += 4 * PL) {
      f32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = *(const f32x4*)(op + (size_t)(p + u * PL) * ps);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float w = w_lds[p + u * PL][hh_e];
        acc.x = fmaf(v[u].x, w, acc.x);
        acc.y = fmaf(v[u].y, w, acc.y);
        acc.z = fmaf(v[u].z, w, acc.z);
        acc.w = fmaf(v[u].w, w, acc.w);
      }
    }
    for (; p < np; p += PL) {
      const f32x4 v = *(const f32x4*)(op + (size_t)p * ps);
      const float w = w_lds[p][hh_e];
      acc.x = fmaf(v.x, w, acc.x);
      acc.y = fmaf(v.y, w, acc.y);
      acc.z = fmaf(v.z, w, acc.z);
      acc.w = fmaf(v.w, w, acc.w);
    }
    __syncthreads();
  }
  finish(acc, lsum);
}

// Split-K reduce: one workgroup per (sequence, group of HG query heads);
// sequences with one partition are left alone, and a sequence the offsets
// give no partition (inconsistent offsets: no decode workgroup wrote it)
// gets NaN rows.  WIDE: sequences of up to kReduceRowsInFlight * PL partials
// also load everything at once (a larger register budget, so it is launched
// only where such sequences can occur).
// The grid is one-dimensional and sequence-major: the head groups of a
// sequence are neighbours, so a long sequence's merges are dispatched
// together (spread over the XCDs by the round-robin dispatch) instead of one
// head group per pass over all sequences, behind the workgroups of every
// unsplit sequence, which exit at once (skewed workload at split-K 512:
// reduce 18.0 -> 13.4 us).
template <int D, bool F32OUT, int HG, bool WIDE>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(void* __restrict__ out,
                                                            const float* __restrict__ ws,
                                                            const int32_t* __restrict__ part_off,
                                                            int Hq, int total_parts, int min_parts) {
  const int nhg = Hq / HG;
  const int s = (int)(blockIdx.x / (unsigned)nhg), qh0 = (int)(blockIdx.x % (unsigned)nhg) * HG;
  const int p0 = part_off[s];
  const int n = part_off[s + 1] - p0;
  if (n <= 0) {
    const size_t oi0 = ((size_t)s * Hq + qh0) * D;
    for (int i = threadIdx.x; i < HG * D; i += 256) {
      if constexpr (F32OUT)
        ((float*)out)[oi0 + i] = NAN;
      else
        ((uint16_t*)out)[oi0 + i] = 0x7fc0;
    }
    return;
  }
  if (n < min_parts) return;
  merge_heads<D, F32OUT, HG, WIDE>(out, ((size_t)s * Hq + qh0) * D, ws, ws + (size_t)total_parts * Hq * D,
                             (size_t)p0 * Hq + qh0, Hq, n);
}

// Stream-K reduce: one workgroup per (sequence, HG query heads of one head
// group hg of hpw).  The item's tiles [start, start + n) of the T laid out end to
// end went to waves r(start) .. r(start + n - 1), r(x) = floor(((x + 1) R -
// 1) / T) being the wave whose slice [floor(r T / R), floor((r + 1) T / R))
// holds tile x; with one wave the output is already written, with several
// their partials sit in consecutive slots r + hg*S + s.  A sequence without
// tiles gets zeros; offsets that are not running sums ending at CU, NaN.
template <int D, bool F32OUT, int HG>
__global__ __launch_bounds__(256) void sk_reduce_kernel(void* __restrict__ out,
                                                        const float* __restrict__ ws,
                                                        const int32_t* __restrict__ tile_off,
                                                        int S, int Hq, int Hkv, int hpw, int R,
                                                        int CU) {
  // sequence-major one-dimensional grid, as in splitk_reduce_kernel
  const int nhg = Hq / HG;
  const int s = (int)(blockIdx.x / (unsigned)nhg);
  const int qh0 = (int)(blockIdx.x % (unsigned)nhg) * HG;   // heads qh0 .. qh0 + HG - 1
  const int G = Hq / Hkv, groups = G / hpw;
  const int hkv = qh0 / G, hg = hkv * groups + (qh0 % G) / hpw, hh0 = qh0 % hpw;
  const int n = tile_off[s + 1] - tile_off[s];
  const size_t oi0 = ((size_t)s * Hq + qh0) * D;
  const int64_t T = (int64_t)CU * Hkv * groups;
  const int64_t start = (int64_t)hg * CU + tile_off[s], last = start + n - 1;
  if (n <= 0 || start < 0 || last >= T) {
    const bool zero = n == 0;
    for (int i = threadIdx.x; i < HG * D; i += 256) {
      if constexpr (F32OUT)
        ((float*)out)[oi0 + i] = zero ? 0.f : NAN;
      else
        ((uint16_t*)out)[oi0 + i] = zero ? 0 : 0x7fc0;
    }
    return;
  }
  const int r0 = (int)(((start + 1) * R - 1) / T), r1 = (int)(((last + 1) * R - 1) / T);
  if (r0 == r1) return;
  const size_t slots = (size_t)R + (size_t)Hkv * groups * S;
  const size_t slot0 = (size_t)r0 + (size_t)hg * S + s;
  merge_heads<D, F32OUT, HG>(out, oi0, ws, ws + slots * hpw * D, slot0 * hpw + hh0, hpw,
                             r1 - r0 + 1);
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
  if (decode_mfma_eligible(a)) return decode_mfma_sk_workers();
  switch (a.kv_dtype) {
    case PKV_F32: return valu::valu_sk_workers<PKV_F32>(a);
    case PKV_BF16: return valu::valu_sk_workers<PKV_BF16>(a);
    default: return valu::valu_sk_workers<PKV_FP8_E4M3>(a);
  }
}

int decode_sk_heads_per_wave(const DecodeArgs& a) {
  if (decode_mfma_eligible(a)) return 8;
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
  if (decode_mfma_eligible(a)) return launch_decode_mfma_sk(a, stream, store);
  hipStream_t st = (hipStream_t)stream;
  switch (a.kv_dtype) {
    case PKV_F32: return valu::launch_valu_sk<PKV_F32>(a, store, st);
    case PKV_BF16: return valu::launch_valu_sk<PKV_BF16>(a, store, st);
    default: return valu::launch_valu_sk<PKV_FP8_E4M3>(a, store, st);
  }
}

// Calls f(integral_constant<int, HG>) for HG in {1, 2, 4, 8}.
template <class F>
int with_hg(int hg, F&& f) {
  switch (hg) {
    case 8: return f(std::integral_constant<int, 8>());
    case 4: return f(std::integral_constant<int, 4>());
    case 2: return f(std::integral_constant<int, 2>());
    default: return f(std::integral_constant<int, 1>());
  }
}

int launch_sk_reduce(const DecodeArgs& a0, void* stream) {
  const DecodeArgs a = clamp_workers(a0);
  hipStream_t st = (hipStream_t)stream;
  const int hpw = decode_sk_heads_per_wave(a);
  const int hgs = std::min(hpw, 256 / a.D);   // heads per reduce workgroup
  const long long nwg = (long long)a.S * (a.Hq / hgs);
  if (nwg > INT_MAX) return (int)hipErrorInvalidConfiguration;
  dim3 grid((unsigned)nwg), block(256);
  const bool f32 = a.q_dtype == PKV_F32;
  return with_hg(hgs, [&](auto hg) {
    constexpr int HG = decltype(hg)::value;
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, block, 0, st, a.out, (const float*)a.ws, a.tile_off, a.S,
                         a.Hq, a.Hkv, hpw, a.sk_workers, a.sk_cu);
    };
    if (a.D == 64)
      f32 ? go(sk_reduce_kernel<64, true, HG>) : go(sk_reduce_kernel<64, false, HG>);
    else
      f32 ? go(sk_reduce_kernel<128, true, HG>) : go(sk_reduce_kernel<128, false, HG>);
    return (int)hipGetLastError();
  });
}

int launch_splitk_reduce(void* out, const float* ws, const int32_t* part_off, int S, int Hq, int D,
                         int total_parts, pkv_dtype out_dtype, void* stream, int min_parts,
                         int max_rows) {
  hipStream_t st = (hipStream_t)stream;
  const int cap = 256 / D;   // heads per workgroup: 64 float4 columns at most
  const int hgs = Hq % cap == 0 ? cap : Hq % 2 == 0 ? 2 : 1;
  const int pl = 256 / (hgs * D / 4);   // piece lanes of merge_heads
  const bool wide = max_rows > 4 * pl;
  const long long nwg = (long long)S * (Hq / hgs);
  if (nwg > INT_MAX) return (int)hipErrorInvalidConfiguration;
  dim3 grid((unsigned)nwg), block(256);
  const bool f32 = out_dtype == PKV_F32;
  return with_hg(hgs, [&](auto hg) {
    constexpr int HG = decltype(hg)::value;
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, block, 0, st, out, ws, part_off, Hq, total_parts, min_parts);
    };
    auto pick = [&](auto w) {
      constexpr bool W = decltype(w)::value;
      if (D == 64)
        f32 ? go(splitk_reduce_kernel<64, true, HG, W>) : go(splitk_reduce_kernel<64, false, HG, W>);
      else
        f32 ? go(splitk_reduce_kernel<128, true, HG, W>) : go(splitk_reduce_kernel<128, false, HG, W>);
    };
    wide ? pick(std::true_type()) : pick(std::false_type());
    return (int)hipGetLastError();
  });
}

}  // namespace pkv
