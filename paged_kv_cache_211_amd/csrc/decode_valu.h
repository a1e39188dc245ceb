// PagedAttention decode kernels for gfx950 (CDNA4, wave64), vector-ALU path.
// Included by one source file per cache element type, each instantiating
// launch_valu<KV> and valu_heads_per_wg<KV> for its type.
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

#pragma once

#include <hip/hip_runtime.h>

#include <cmath>

#include "decode_common.h"

namespace pkv {
namespace valu {

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

// PW = false: the NW waves of a workgroup share one work item (taking its
// blocks round-robin) and merge through LDS.  PW = true: each wave owns a
// work item (flat item blockIdx.x * NW + wave) and writes its own output or
// partial; waves never synchronise.
//
// STORE (decode step): the workgroup that reads the last block of a
// sequence first stores the sequence's new token there.

template <int KV, int D, int BS, int HPW, int NW, int NBUF, bool SPLIT, bool PW, bool STORE = false>
__global__ __launch_bounds__(NW * 64) void decode_kernel(const DecodeArgs a) {
  static_assert(!(PW && STORE), "the decode step stores from shared-item workgroups");
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
  const int item = PW ? blockIdx.x * NW + w : blockIdx.x;
  if constexpr (PW) {
    if (item >= (SPLIT ? a.total_parts : a.S)) return;
  }
  const Work wk = locate<SPLIT, BS>(a, HPW, lane, item);
  if constexpr (STORE) store_new_token<KV, D, BS, NW * 64>(a, wk);
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

  tile_loop<NBUF, NLOAD, PW ? 1 : NW>(tbl, wk.t0 / BS + (PW ? 0 : w), wk.jend, a.nb,
                             (const uint8_t*)a.kc + head_off + lane * 16,
                             (const uint8_t*)a.vc + head_off + lane * 16, blk_stride, lane, bad,
                             process);

  if constexpr (PW) {
    // ---- this wave's item: write the output or the partial directly ----
    const bool final_out = !SPLIT || wk.nparts == 1;
    float* ws_o = a.ws;
    float* ws_ml = a.ws + (size_t)a.total_parts * a.Hq * D;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const float lt = tile_sum<BS>(l_run[hh]);
      const int qh = qh0 + hh;
      const float inv = lt > 0.f ? a.v_mult / lt : 0.f;
#pragma unroll
      for (int l = 0; l < NLOAD; ++l) {
        float v = acc[hh][l];
#pragma unroll
        for (int msk = 1; msk < RU; msk <<= 1) v += xor_lanes(v, msk);
        const int dim = l * DPI + lane / RU;
        if (lane % RU == 0) {
          if (final_out) {
            const float r = bad ? NAN : v * inv;
            const size_t oi = ((size_t)s * a.Hq + qh) * D + dim;
            if constexpr (F32)
              ((float*)a.out)[oi] = r;
            else
              ((uint16_t*)a.out)[oi] = f32_to_bf16(r);
          } else {
            ws_o[((size_t)item * a.Hq + qh) * D + dim] = bad ? NAN : v * a.v_mult;
          }
        }
      }
      if (!final_out && lane == 0) {
        const size_t pi = (size_t)item * a.Hq + qh;
        ws_ml[pi * 2] = m_run[hh];
        ws_ml[pi * 2 + 1] = bad ? NAN : lt;
      }
    }
    return;
  }

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

// store: whether the workgroups also store the new tokens (decode step; needs
// one workgroup per kv head, HPW == G).
template <int KV, int D, int BS, int HPW>
int launch_t(const DecodeArgs& a, bool store, hipStream_t st) {
  const int groups = a.Hq / a.Hkv / HPW;
  dim3 block(kWaves * 64);
  const int items = a.partition > 0 ? a.total_parts : a.S;
  if (store && (kPerWave || groups != 1)) return (int)hipErrorInvalidValue;
  dim3 grid(kPerWave ? (items + kWaves - 1) / kWaves : items, a.Hkv * groups);
  if (a.partition > 0) {
    if (store)
      hipLaunchKernelGGL((decode_kernel<KV, D, BS, HPW, kWaves, kBufs, true, false, true>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((decode_kernel<KV, D, BS, HPW, kWaves, kBufs, true, kPerWave>), grid, block, 0, st, a);
  } else {
    if (store)
      hipLaunchKernelGGL((decode_kernel<KV, D, BS, HPW, kWaves, kBufs, false, false, true>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((decode_kernel<KV, D, BS, HPW, kWaves, kBufs, false, kPerWave>), grid, block, 0, st, a);
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
int heads_per_wg(int G) {
  constexpr int MAXH = max_hpw<KV, D, BS>();
  int h = 1;
  while (h * 2 <= MAXH && G % (h * 2) == 0) h *= 2;
  return h;
}

template <int KV, int D, int BS>
int launch_kv(const DecodeArgs& a, bool store, hipStream_t st) {
  constexpr int MAXH = max_hpw<KV, D, BS>();
  const int h = heads_per_wg<KV, D, BS>(a.Hq / a.Hkv);
  if constexpr (MAXH >= 8) if (h == 8) return launch_t<KV, D, BS, 8>(a, store, st);
  if constexpr (MAXH >= 4) if (h == 4) return launch_t<KV, D, BS, 4>(a, store, st);
  if constexpr (MAXH >= 2) if (h == 2) return launch_t<KV, D, BS, 2>(a, store, st);
  return launch_t<KV, D, BS, 1>(a, store, st);
}

template <int KV>
int launch_valu(const DecodeArgs& a, bool store, hipStream_t st) {
  if (a.D == 64) return a.BS == 16 ? launch_kv<KV, 64, 16>(a, store, st) : launch_kv<KV, 64, 32>(a, store, st);
  return a.BS == 16 ? launch_kv<KV, 128, 16>(a, store, st) : launch_kv<KV, 128, 32>(a, store, st);
}

template <int KV>
int valu_heads_per_wg(const DecodeArgs& a) {
  const int G = a.Hq / a.Hkv;
  if (a.D == 64) return a.BS == 16 ? heads_per_wg<KV, 64, 16>(G) : heads_per_wg<KV, 64, 32>(G);
  return a.BS == 16 ? heads_per_wg<KV, 128, 16>(G) : heads_per_wg<KV, 128, 32>(G);
}

}  // namespace valu
}  // namespace pkv
