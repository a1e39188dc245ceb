// PagedAttention decode kernels for gfx950 (CDNA4, wave64).
//
// "PagedAttention Kernel：大模型推理优化的显存管理革新" §3.1 splits decode
// attention into QK^T per block, a softmax normalised locally, and PV
// accumulated block by block with fp32 accumulation (§6).  Here each
// workgroup owns (sequence, kv head, group of HPW query heads, split-K
// partition); its NW waves take the partition's blocks round-robin.  Per
// block (one "tile" = the block's rows for one kv head, BS*D*E contiguous
// bytes):
//   * the block id comes from the block table with a wave-uniform scalar load;
//   * the key tile and the value tile are read with 16-byte loads, every load
//     instruction covering 1 KiB of contiguous memory (§2.2: coalescing), and
//     the next tile's loads are issued before the current tile is consumed
//     (§2.2: prefetch of the next page);
//   * key layout [D/X][BS][X] puts one token in each lane with X dims per
//     load, so q.k is a per-lane dot product over NLOAD*X dims followed by a
//     reduction across the 64/BS lanes holding the same token;
//   * one-pass online softmax per tile (running max m, sum l, rescale of the
//     accumulator once per tile), in the log2 domain;
//   * probabilities go through LDS to the value layout [D][BS], where each
//     lane holds X consecutive tokens of one dim per load, so PV is a dot
//     product over token pairs.
// bf16 and fp8 tiles compute with packed bf16 pairs (v_dot2_f32_bf16,
// probabilities rounded to bf16, fp32 accumulation); fp32 tiles with fp32
// FMAs.  The waves of a workgroup merge their (m, l, acc) through LDS; a
// partition that is the whole sequence writes the output, otherwise the
// partial (m, l, unnormalised o) goes to the workspace for the split-K
// reduce kernel.

#include <hip/hip_runtime.h>

#include <cmath>

#include "decode_common.h"

namespace pkv {
namespace {

using namespace dec;

template <int KV, int D, int BS>
struct Geo {
  static constexpr int E = KV == PKV_F32 ? 4 : KV == PKV_BF16 ? 2 : 1;  // element bytes
  static constexpr int X = 16 / E;           // elements per 16-byte unit
  static constexpr int TILE = BS * D * E;    // bytes of one (block, kv head) tile
  static constexpr int NLOAD = TILE / 1024;  // 16-byte loads per lane per tile
  static constexpr int KL = 64 / BS;         // lanes holding the same token (keys)
  static constexpr int RU = BS * E / 16;     // 16-byte units per dim row (values)
  static constexpr int DPI = 64 / RU;        // dims covered by one value load
  static constexpr int PPC = X / 2;          // bf16 pairs per 16-byte unit
  static constexpr bool F32 = KV == PKV_F32;
  static_assert(TILE % 1024 == 0, "tile must be a multiple of 1 KiB");
  static_assert(64 % BS == 0, "block size must divide the wave");
  static_assert(RU >= 1 && 64 % RU == 0, "value row must divide the wave");
};

// A 16-byte unit of bf16 or fp8 elements -> PPC packed bf16 pairs (exact).
template <int KV>
__device__ __forceinline__ void unpack_pairs(const u32x4 r, uint32_t* p) {
  if constexpr (KV == PKV_BF16) {
    p[0] = r.x; p[1] = r.y; p[2] = r.z; p[3] = r.w;
  } else {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 lo = fp8x2_to_f32<false>(w[i]);
      const f32x2 hi = fp8x2_to_f32<true>(w[i]);
      // fp8 values have at most 4 significant bits: their fp32 top halves are exact bf16
      p[2 * i] = __builtin_amdgcn_perm(__float_as_uint(lo.y), __float_as_uint(lo.x), 0x07060302u);
      p[2 * i + 1] = __builtin_amdgcn_perm(__float_as_uint(hi.y), __float_as_uint(hi.x), 0x07060302u);
    }
  }
}

template <int BS>
__device__ __forceinline__ float tile_max(float v) {
  v = row16_max(v);
  if constexpr (BS == 32) v = max_xor16(v);
  return v;
}
template <int BS>
__device__ __forceinline__ float tile_sum(float v) {
  v = row16_sum(v);
  if constexpr (BS == 32) v = sum_xor16(v);
  return v;
}
// Sum over the 64/BS lanes that hold the same key token (lanes l, l^BS, ...).
template <int BS>
__device__ __forceinline__ float token_sum(float v) {
  if constexpr (BS == 16) v = sum_xor16(v);
  return sum_xor32(v);
}

template <int KV, int D, int BS, int HPW, int NW, int NBUF, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void decode_kernel(const DecodeArgs a) {
  using Gm = Geo<KV, D, BS>;
  constexpr int X = Gm::X, NLOAD = Gm::NLOAD, KL = Gm::KL, RU = Gm::RU, DPI = Gm::DPI;
  constexpr int PPC = Gm::PPC, TILE = Gm::TILE;
  constexpr bool F32 = Gm::F32;

  __shared__ float p_lds[NW][HPW][BS];
  __shared__ float o_lds[NW][HPW][D];
  __shared__ float m_lds[NW][HPW];
  __shared__ float l_lds[NW][HPW];
  __shared__ int bad_lds[NW];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const Work wk = locate<SPLIT, BS>(a, HPW, lane);
  const int s = wk.s, qh0 = wk.qh0, t1 = wk.t1;
  bool bad = wk.bad;
  const int32_t* __restrict__ tbl = a.tables + (size_t)s * a.max_blocks;
  const size_t head_off = (size_t)wk.hkv * TILE;
  const size_t blk_stride = (size_t)a.Hkv * TILE;

  // ---- query rows of the HPW heads ----
  // Either held in VGPRs (the dims of this lane's key chunks) or staged once
  // in LDS for all waves of the workgroup (PKV_DECODE_QLDS).
  constexpr int QE = F32 ? 4 : 2;              // query element bytes
  constexpr int QUL = 2 * X * QE / 32;         // 16-byte q units per key load (1 or 2)
  const int kchunk0 = lane / BS;               // key chunk of load l is l*KL + kchunk0
  const uint8_t* qsrc = (const uint8_t*)a.q + ((size_t)s * a.Hq + qh0) * D * QE;
#if PKV_DECODE_QLDS
  constexpr int QU = HPW * D * QE / 16;
  __shared__ u32x4 q_lds[QU];
  for (int u = threadIdx.x; u < QU; u += NW * 64) q_lds[u] = *(const u32x4*)(qsrc + 16 * u);
  __syncthreads();
  auto q_unit = [&](int hh, int l, int u) -> u32x4 {
    return q_lds[(hh * D + (l * KL + kchunk0) * X) * QE / 16 + u];
  };
#else
  u32x4 q_reg[HPW][NLOAD][QUL];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int l = 0; l < NLOAD; ++l)
#pragma unroll
      for (int u = 0; u < QUL; ++u)
        q_reg[hh][l][u] = *(const u32x4*)(qsrc + ((size_t)(hh * D + (l * KL + kchunk0) * X) * QE + 16 * u));
  auto q_unit = [&](int hh, int l, int u) -> u32x4 { return q_reg[hh][l][u]; };
#endif

  float m_run[HPW], l_run[HPW], acc[HPW][NLOAD];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    m_run[hh] = -INFINITY;
    l_run[hh] = 0.f;
#pragma unroll
    for (int j = 0; j < NLOAD; ++j) acc[hh][j] = 0.f;
  }

  const int tk = lane % BS;              // this lane's token in a key tile
  const int tv0 = (lane % RU) * X;       // first of this lane's X tokens in a value tile

  // One tile: QK^T for this lane's token, online softmax, PV.
  auto process = [&](int j, const u32x4* kr, const u32x4* vr) {
    // ---- QK^T for this lane's token, HPW heads ----
    float sc[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) sc[hh] = 0.f;
#pragma unroll
    for (int l = 0; l < NLOAD; ++l) {
      if constexpr (F32) {
        const f32x4 k4 = __builtin_bit_cast(f32x4, kr[l]);
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
          const f32x4 q4 = __builtin_bit_cast(f32x4, q_unit(hh, l, 0));
          sc[hh] = fmaf(q4.x, k4.x, sc[hh]);
          sc[hh] = fmaf(q4.y, k4.y, sc[hh]);
          sc[hh] = fmaf(q4.z, k4.z, sc[hh]);
          sc[hh] = fmaf(q4.w, k4.w, sc[hh]);
        }
      } else {
        uint32_t kp[PPC];
        unpack_pairs<KV>(kr[l], kp);
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
          for (int u = 0; u < PPC / 4; ++u) {
            const u32x4 q4 = q_unit(hh, l, u);
            sc[hh] = dot2_bf16(q4.x, kp[4 * u], sc[hh]);
            sc[hh] = dot2_bf16(q4.y, kp[4 * u + 1], sc[hh]);
            sc[hh] = dot2_bf16(q4.z, kp[4 * u + 2], sc[hh]);
            sc[hh] = dot2_bf16(q4.w, kp[4 * u + 3], sc[hh]);
          }
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) sc[hh] = token_sum<BS>(sc[hh]);

    // ---- online softmax over this tile ----
    const int tile_t0 = j * BS;
    const bool valid = tile_t0 + tk < t1;
    float cfac[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const float z = valid ? sc[hh] * a.qk_mult : -INFINITY;
      const float mnew = fmaxf(m_run[hh], tile_max<BS>(z));
      cfac[hh] = __builtin_amdgcn_exp2f(m_run[hh] - mnew);
      float p = __builtin_amdgcn_exp2f(z - mnew);
      m_run[hh] = mnew;
      uint16_t pb = 0;
      if constexpr (!F32) {
        pb = cvt_bf16(p);
        p = bf16_to_f32(pb);
      }
      l_run[hh] = l_run[hh] * cfac[hh] + p;
      if (lane < BS) {
        if constexpr (F32)
          p_lds[w][hh][lane] = p;
        else
          ((uint16_t*)&p_lds[w][hh][0])[lane] = pb;
      }
    }
    __builtin_amdgcn_wave_barrier();

    // ---- PV: acc[hh][dim] += sum over this lane's X tokens ----
    const int nvalid = t1 - tile_t0;  // tokens of this tile inside the partition
    const bool tail = nvalid < BS;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
      for (int l = 0; l < NLOAD; ++l) acc[hh][l] *= cfac[hh];
    }
    if constexpr (F32) {
      float pv[HPW][4];
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const f32x4 t = *(const f32x4*)&p_lds[w][hh][tv0];
        pv[hh][0] = t.x; pv[hh][1] = t.y; pv[hh][2] = t.z; pv[hh][3] = t.w;
      }
#pragma unroll
      for (int l = 0; l < NLOAD; ++l) {
        f32x4 v4 = __builtin_bit_cast(f32x4, vr[l]);
        if (tail) {
          v4.x = tv0 + 0 < nvalid ? v4.x : 0.f;
          v4.y = tv0 + 1 < nvalid ? v4.y : 0.f;
          v4.z = tv0 + 2 < nvalid ? v4.z : 0.f;
          v4.w = tv0 + 3 < nvalid ? v4.w : 0.f;
        }
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
          float t = acc[hh][l];
          t = fmaf(pv[hh][0], v4.x, t);
          t = fmaf(pv[hh][1], v4.y, t);
          t = fmaf(pv[hh][2], v4.z, t);
          t = fmaf(pv[hh][3], v4.w, t);
          acc[hh][l] = t;
        }
      }
    } else {
      uint32_t pp[HPW][PPC];
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const uint16_t* src = (const uint16_t*)&p_lds[w][hh][0] + tv0;
#pragma unroll
        for (int u = 0; u < PPC / 4; ++u) {
          const u32x4 t = *(const u32x4*)(src + 8 * u);
          pp[hh][4 * u] = t.x; pp[hh][4 * u + 1] = t.y;
          pp[hh][4 * u + 2] = t.z; pp[hh][4 * u + 3] = t.w;
        }
      }
#pragma unroll
      for (int l = 0; l < NLOAD; ++l) {
        uint32_t vp[PPC];
        unpack_pairs<KV>(vr[l], vp);
        if (tail) {
#pragma unroll
          for (int k = 0; k < PPC; ++k) {
            const int ta = tv0 + 2 * k;
            const uint32_t keep = (ta < nvalid ? 0x0000ffffu : 0u) | (ta + 1 < nvalid ? 0xffff0000u : 0u);
            vp[k] &= keep;
          }
        }
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
          float t = acc[hh][l];
#pragma unroll
          for (int k = 0; k < PPC; ++k) t = dot2_bf16(pp[hh][k], vp[k], t);
          acc[hh][l] = t;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  tile_loop<NBUF, NLOAD, NW>(tbl, wk.t0 / BS + w, wk.jend, a.nb,
                             (const uint8_t*)a.kc + head_off + lane * 16,
                             (const uint8_t*)a.vc + head_off + lane * 16, blk_stride, lane, bad,
                             process);

  // ---- per-wave totals ----
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const float lt = tile_sum<BS>(l_run[hh]);
#pragma unroll
    for (int l = 0; l < NLOAD; ++l) {
      float v = acc[hh][l];
#pragma unroll
      for (int msk = 1; msk < RU; msk <<= 1) v += xor_lanes(v, msk);
      if (lane % RU == 0) o_lds[w][hh][l * DPI + lane / RU] = v;
    }
    if (lane == 0) {
      m_lds[w][hh] = m_run[hh];
      l_lds[w][hh] = lt;
    }
  }
  if (lane == 0) bad_lds[w] = bad ? 1 : 0;
  __syncthreads();

  // ---- merge the waves, then write the output or the partial ----
  merge_store<HPW, D, NW, F32>(a, wk, !SPLIT || wk.nparts == 1, o_lds, m_lds, l_lds, bad_lds);
}

// Split-K reduce: one workgroup per (sequence, query head) with > 1 partition.
template <int D, bool F32OUT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(void* __restrict__ out,
                                                            const float* __restrict__ ws,
                                                            const int32_t* __restrict__ part_off,
                                                            int Hq, int total_parts) {
  constexpr int DQ = D / 4;      // float4 columns of a row
  constexpr int PL = 256 / DQ;   // partitions handled in parallel
  __shared__ f32x4 o_red[PL][DQ];
  __shared__ float l_red[PL];
  __shared__ float mx_red[256];

  const int s = blockIdx.x, qh = blockIdx.y;
  const int p0 = part_off[s];
  const int n = part_off[s + 1] - p0;
  if (n <= 1) return;
  const float* ws_o = ws;
  const float* ws_ml = ws + (size_t)total_parts * Hq * D;
  const int tid = threadIdx.x;

  float mx = -INFINITY;
  for (int p = tid; p < n; p += 256) mx = fmaxf(mx, ws_ml[((size_t)(p0 + p) * Hq + qh) * 2]);
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
      const size_t pi = (size_t)(p0 + p) * Hq + qh;
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
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const size_t oi = ((size_t)s * Hq + qh) * D + dq * 4;
    const float r0 = t.x * inv, r1 = t.y * inv, r2 = t.z * inv, r3 = t.w * inv;
    if constexpr (F32OUT) {
      *(f32x4*)((float*)out + oi) = f32x4{r0, r1, r2, r3};
    } else {
      uint16_t* o16 = (uint16_t*)out + oi;
      const uint32_t lo = pack_bf16x2(r0, r1), hi = pack_bf16x2(r2, r3);
      *(uint2*)o16 = make_uint2(lo, hi);
    }
  }
}


template <int KV, int D, int BS, int HPW>
int launch_t(const DecodeArgs& a, hipStream_t st) {
  const int groups = a.Hq / a.Hkv / HPW;
  dim3 block(kWaves * 64);
  if (a.partition > 0) {
    dim3 grid(a.total_parts, a.Hkv * groups);
    hipLaunchKernelGGL((decode_kernel<KV, D, BS, HPW, kWaves, kBufs, true>), grid, block, 0, st, a);
  } else {
    dim3 grid(a.S, a.Hkv * groups);
    hipLaunchKernelGGL((decode_kernel<KV, D, BS, HPW, kWaves, kBufs, false>), grid, block, 0, st, a);
  }
  return (int)hipGetLastError();
}

// Heads per workgroup: the largest power of two (at most 8) dividing G whose
// per-head registers fit the budget: the query dims of the lane's key chunks
// (64 VGPRs in all when q lives in VGPRs), else the accumulators and the
// probabilities of a value load (48 VGPRs in all).
template <int KV, int D, int BS>
constexpr int max_hpw() {
  using Gm = Geo<KV, D, BS>;
#if PKV_DECODE_QLDS
  constexpr int per_head = Gm::NLOAD + (Gm::F32 ? 4 : Gm::PPC), budget = 48;
#else
  constexpr int per_head = Gm::F32 ? Gm::NLOAD * 4 : Gm::NLOAD * Gm::PPC, budget = 64;
#endif
  return budget / per_head >= 8 ? 8 : budget / per_head >= 4 ? 4 : budget / per_head >= 2 ? 2 : 1;
}

template <int KV, int D, int BS>
int launch_kv(const DecodeArgs& a, hipStream_t st) {
  constexpr int MAXH = max_hpw<KV, D, BS>();
  const int G = a.Hq / a.Hkv;
  int h = 1;
  while (h * 2 <= MAXH && G % (h * 2) == 0) h *= 2;
  if constexpr (MAXH >= 8) if (h == 8) return launch_t<KV, D, BS, 8>(a, st);
  if constexpr (MAXH >= 4) if (h == 4) return launch_t<KV, D, BS, 4>(a, st);
  if constexpr (MAXH >= 2) if (h == 2) return launch_t<KV, D, BS, 2>(a, st);
  return launch_t<KV, D, BS, 1>(a, st);
}

template <int KV>
int launch_d(const DecodeArgs& a, hipStream_t st) {
  if (a.D == 64) return a.BS == 16 ? launch_kv<KV, 64, 16>(a, st) : launch_kv<KV, 64, 32>(a, st);
  return a.BS == 16 ? launch_kv<KV, 128, 16>(a, st) : launch_kv<KV, 128, 32>(a, st);
}

}  // namespace

bool decode_supported(pkv_dtype q, pkv_dtype kv, int D, int BS, int G) {
  const bool pair_ok = (q == PKV_F32 && kv == PKV_F32) || (q == PKV_BF16 && kv == PKV_BF16) ||
                       (q == PKV_BF16 && kv == PKV_FP8_E4M3);
  return pair_ok && (D == 64 || D == 128) && (BS == 16 || BS == 32) && G >= 1;
}

int launch_decode(const DecodeArgs& a, void* stream) {
  if (decode_mfma_eligible(a)) return launch_decode_mfma(a, stream);
  hipStream_t st = (hipStream_t)stream;
  switch (a.kv_dtype) {
    case PKV_F32: return launch_d<PKV_F32>(a, st);
    case PKV_BF16: return launch_d<PKV_BF16>(a, st);
    default: return launch_d<PKV_FP8_E4M3>(a, st);
  }
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
