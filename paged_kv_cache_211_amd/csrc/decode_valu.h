// PagedAttention decode kernels for gfx950 (CDNA4, wave64), vector-ALU path.
// Included by one source file per cache element type, each instantiating
// launch_valu<KV>, launch_valu_sk<KV>, valu_heads_per_wg<KV> and
// valu_sk_workers<KV> for its type.
//
// "PagedAttention Kernel：大模型推理优化的显存管理革新" §3.1 splits decode
// attention into QK^T per block, a softmax normalised locally, and PV
// accumulated block by block with fp32 accumulation (§6).  Per block (one
// "tile" = the block's rows for one kv head, BS*D*E contiguous bytes):
//   * the block id comes from the block table (one vector load per 64 tiles,
//     read back lane by lane);
//   * the key tile and the value tile are read with 16-byte loads, every load
//     instruction covering 1 KiB of contiguous memory (§2.2: coalescing), and
//     the next tile's loads are issued before the current tile is consumed
//     (§2.2: prefetch of the next page);
//   * key layout [D/X][BS][X] puts one token in each lane with X dims per
//     load, so q.k is a per-lane dot product over NLOAD*X dims followed by a
//     reduction across the 64/BS lanes holding the same token;
//   * one-pass online softmax per tile in the log2 domain (running max m,
//     sum l; the accumulator is rescaled only when a tile's max exceeds the
//     reference by more than 2^8);
//   * probabilities go through LDS to the value layout [D][BS], where each
//     lane holds X consecutive tokens of one dim per load, so PV is a dot
//     product over token pairs.
// bf16 and fp8 tiles compute with packed bf16 pairs (v_dot2_f32_bf16,
// probabilities rounded to bf16, fp32 accumulation); fp32 tiles with fp32
// FMAs.
//
// Two schedules share that per-tile code (ValuHeads):
//   * decode_kernel -- one workgroup per (sequence, kv head, group of HPW
//     query heads, split-K partition); its NW waves take the partition's
//     blocks round-robin and merge their (m, l, acc) through LDS.  A
//     partition that is the whole sequence writes the output, otherwise the
//     partial (m, l, unnormalised o) goes to the workspace for the split-K
//     reduce (§3.2: uneven pages need the work split).
//   * decode_sk_kernel -- persistent "stream-K": the tiles of all (head
//     group, sequence) items are laid end to end and every wave takes an
//     equal contiguous slice, crossing item boundaries; an item cut between
//     waves leaves one partial per piece for the reduce.  Every wave streams
//     the same number of tiles whatever the length mix, and pays the start-up
//     of a work item (lookups, query load, first tiles) about once instead of
//     once per partition.

#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

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

// Softmax state and query of HPW heads held by one wave, and the per-tile
// step: QK^T for this lane's token, online softmax, PV.  QL = false: the
// query dims of the lane's key chunks live in VGPRs (HPW*NLOAD*QUL*4 of
// them); QL = true: the HPW query rows live in LDS (qs, QU 16-byte units,
// filled with fill_q) and are read per tile, which frees those VGPRs for a
// deeper ring of tiles in flight.
template <int KV, int D, int BS, int HPW, bool QL>
struct ValuHeads {
  using Gm = Geo<KV, D, BS>;
  static constexpr int X = Gm::X, NLOAD = Gm::NLOAD, KL = Gm::KL, RU = Gm::RU, DPI = Gm::DPI;
  static constexpr int PPC = Gm::PPC;
  static constexpr bool F32 = Gm::F32;
  static constexpr int QE = F32 ? 4 : 2;        // query element bytes
  static constexpr int QUL = 2 * X * QE / 32;   // 16-byte q units per key load (1 or 2)
  static constexpr int QU = HPW * D * QE / 16;  // 16-byte units of the HPW query rows

  u32x4 q[QL ? 1 : HPW][NLOAD][QUL];   // QL = false: this lane's query dims
  const u32x4* qs = nullptr;            // QL = true: the query rows in LDS
  float m_run[HPW], l_run[HPW], acc[HPW][NLOAD];

  // QL = false: load this lane's query dims into VGPRs.
  __device__ __forceinline__ void load_q(const DecodeArgs& a, int s, int qh0, int lane) {
    const int kchunk0 = lane / BS;   // key chunk of load l is l*KL + kchunk0
    const uint8_t* qsrc = (const uint8_t*)a.q + ((size_t)s * a.Hq + qh0) * D * QE;
#pragma unroll
    for (int hh = 0; hh < (QL ? 1 : HPW); ++hh)
#pragma unroll
      for (int l = 0; l < NLOAD; ++l)
#pragma unroll
        for (int u = 0; u < QUL; ++u)
          q[hh][l][u] = *(const u32x4*)(qsrc + ((size_t)(hh * D + (l * KL + kchunk0) * X) * QE + 16 * u));
  }

  // QL = true: copy the HPW query rows (contiguous in [S][Hq][D]) to dst in
  // LDS, threads tid, tid + nthreads, ...; the caller synchronises.
  __device__ __forceinline__ static void fill_q(const DecodeArgs& a, int s, int qh0, u32x4* dst,
                                                int tid, int nthreads) {
    const u32x4* src = (const u32x4*)((const uint8_t*)a.q + ((size_t)s * a.Hq + qh0) * D * QE);
    for (int u = tid; u < QU; u += nthreads) dst[u] = src[u];
  }

  __device__ __forceinline__ u32x4 qunit(int hh, int l, int u, int lane) const {
    if constexpr (QL)
      return qs[(hh * D + (l * KL + lane / BS) * X) * QE / 16 + u];
    else
      return q[hh][l][u];
  }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      m_run[hh] = -INFINITY;
      l_run[hh] = 0.f;
#pragma unroll
      for (int j = 0; j < NLOAD; ++j) acc[hh][j] = 0.f;
    }
  }

  // Tile j (tokens j*BS ..) of a range whose tokens end at t1; kr/vr: this
  // lane's key and value loads; prow: this wave's LDS rows [HPW][BS].
  __device__ __forceinline__ void tile(float qk_mult, int j, int t1, const u32x4* kr,
                                       const u32x4* vr, float (*prow)[BS], int lane) {
    const int tk = lane % BS;              // this lane's token in a key tile
    const int tv0 = (lane % RU) * X;       // first of this lane's X tokens in a value tile
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
          const f32x4 q4 = __builtin_bit_cast(f32x4, qunit(hh, l, 0, lane));
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
            const u32x4 q4 = qunit(hh, l, u, lane);
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
    // Probabilities are taken against a reference max m_run that moves only
    // when a tile's max exceeds it by more than 2^8 (then l and the
    // accumulator are rescaled: a rare, wave-uniform branch instead of a
    // correction factor and a rescale every tile).  p <= 2^8 keeps bf16 and
    // fp32 in range, and O / l does not depend on the reference.
    const int tile_t0 = j * BS;
    const bool valid = tile_t0 + tk < t1;
    float z[HPW], tmax[HPW];
    bool grow = false;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      z[hh] = valid ? sc[hh] * qk_mult : -INFINITY;
      tmax[hh] = tile_max<BS>(z[hh]);
      grow |= tmax[hh] > m_run[hh] + 8.0f;
    }
    if (__ballot(grow)) {
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const bool up = tmax[hh] > m_run[hh] + 8.0f;
        const float c = up ? __builtin_amdgcn_exp2f(m_run[hh] - tmax[hh]) : 1.0f;
        m_run[hh] = up ? tmax[hh] : m_run[hh];
        l_run[hh] *= c;
#pragma unroll
        for (int l = 0; l < NLOAD; ++l) acc[hh][l] *= c;
      }
    }
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      float p = __builtin_amdgcn_exp2f(z[hh] - m_run[hh]);
      uint16_t pb = 0;
      if constexpr (!F32) {
        pb = cvt_bf16(p);
        p = bf16_to_f32(pb);
      }
      l_run[hh] += p;
      if (lane < BS) {
        if constexpr (F32)
          prow[hh][lane] = p;
        else
          ((uint16_t*)&prow[hh][0])[lane] = pb;
      }
    }
    __builtin_amdgcn_wave_barrier();

    // ---- PV: acc[hh][dim] += sum over this lane's X tokens ----
    const int nvalid = t1 - tile_t0;  // tokens of this tile inside the partition
    const bool tail = nvalid < BS;
    if constexpr (F32) {
      float pv[HPW][4];
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const f32x4 t = *(const f32x4*)&prow[hh][tv0];
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
        const uint16_t* src = (const uint16_t*)&prow[hh][0] + tv0;
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
  }

  // Sum over the lanes holding this lane's dims of load l (lanes with
  // lane % RU == 0 get dim l*DPI + lane/RU).
  __device__ __forceinline__ float dim_sum(int hh, int l) const {
    float v = acc[hh][l];
#pragma unroll
    for (int msk = 1; msk < RU; msk <<= 1) v += xor_lanes(v, msk);
    return v;
  }
};

// Shared-item schedule.  STORE (decode step): the workgroup that reads the
// last block of a sequence first stores the sequence's new token there.
// The body takes its workgroup index so that another kernel can run it on a
// range of its own workgroups.
template <int KV, int D, int BS, int HPW, int NW, int NBUF, bool SPLIT, bool STORE>
__device__ __forceinline__ void decode_body(const DecodeArgs& a, int bid) {
  using St = ValuHeads<KV, D, BS, HPW, kQLds>;
  constexpr int NLOAD = St::NLOAD, RU = St::RU, DPI = St::DPI, TILE = Geo<KV, D, BS>::TILE;

  __shared__ float p_lds[NW][HPW][BS];
  __shared__ float o_lds[NW][HPW][D];
  __shared__ float m_lds[NW][HPW];
  __shared__ float l_lds[NW][HPW];
  __shared__ int bad_lds[NW];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // XCD-aware order: workgroup ids go round-robin to the 8 XCDs (each with
  // its own L2), so the head group is the id's low part: with 8 head groups
  // every XCD serves one kv head, and blocks that several sequences share
  // stay in that XCD's L2.
  const int nhg = a.Hkv * (a.Hq / a.Hkv / HPW);
  const Work wk = locate<SPLIT, BS>(a, HPW, lane, bid / nhg, bid % nhg);
  bool bad = wk.bad;
  const int32_t* __restrict__ tbl = a.tables + (size_t)wk.s * a.max_blocks;
  const size_t head_off = (size_t)wk.hkv * TILE;
  const size_t blk_stride = (size_t)a.Hkv * TILE;

  St st;
  if constexpr (kQLds) {
    __shared__ u32x4 q_lds[St::QU];
    St::fill_q(a, wk.s, wk.qh0, q_lds, threadIdx.x, NW * 64);
    __syncthreads();
    st.qs = q_lds;
  } else {
    st.load_q(a, wk.s, wk.qh0, lane);
  }
  st.reset();
  const int t1 = wk.t1;
  // STORE: the wave that reads the last block stores the new token into it
  // (waves take tiles t0/BS + w, + NW, ...), then waits for the store only
  // before loading that block.
  const int jlast = wk.jend - 1;
  const bool my_store = STORE && !wk.bad && wk.L > 0 && wk.t0 < wk.L && wk.t1 == wk.L &&
                        (jlast - wk.t0 / BS) % NW == w;
  tile_loop<NBUF, NLOAD, NW>(tbl, wk.t0 / BS + w, wk.jend, a.nb,
                             (const uint8_t*)a.kc + head_off + lane * 16,
                             (const uint8_t*)a.vc + head_off + lane * 16, blk_stride, lane, bad,
                             [&](int j, const u32x4* kr, const u32x4* vr) {
                               st.tile(a.qk_mult, j, t1, kr, vr, p_lds[w], lane);
                             },
                             my_store ? jlast : -1,
                             [&] {
                               if constexpr (STORE) {
                                 if (my_store) store_new_token<KV, D, BS>(a, wk.s, wk.hkv, wk.L, lane);
                               }
                             });

  // ---- per-wave totals ----
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const float lt = tile_sum<BS>(st.l_run[hh]);
#pragma unroll
    for (int l = 0; l < NLOAD; ++l) {
      const float v = st.dim_sum(hh, l);
      if (lane % RU == 0) o_lds[w][hh][l * DPI + lane / RU] = v;
    }
    if (lane == 0) {
      m_lds[w][hh] = st.m_run[hh];
      l_lds[w][hh] = lt;
    }
  }
  if (lane == 0) bad_lds[w] = bad ? 1 : 0;
  __syncthreads();

  // ---- merge the waves, then write the output or the partial ----
  merge_store<HPW, D, NW, St::F32>(a, wk, !SPLIT || wk.nparts == 1, o_lds, m_lds, l_lds, bad_lds);
}

template <int KV, int D, int BS, int HPW, int NW, int NBUF, bool SPLIT, bool STORE>
__global__ __launch_bounds__(NW * 64) void decode_kernel(const DecodeArgs a) {
  decode_body<KV, D, BS, HPW, NW, NBUF, SPLIT, STORE>(a, blockIdx.x);
}

// Stream-K schedule: wave gw of R = a.sk_workers takes tiles
// [floor(gw*T/R), floor((gw+1)*T/R)) of the T = CU * H_kv * groups tiles laid
// out as (head group hg, sequence s, tile j) at hg*CU + tile_off[s] + j, CU =
// tile_off[S].  The piece of item (hg, s) it covers is written as the output
// when it is the whole item, else as the partial in workspace slot
// gw + hg*S + s (rows [slot][HPW][D] of o, then [slot][HPW][2] of (m, l)).
// STORE: the wave holding an item's last tile first stores the sequence's
// new token (one head group per kv head, so it is the block's only reader).
template <int KV, int D, int BS, int HPW, int NW, int NBUF, bool STORE>
__global__ __launch_bounds__(NW * 64) void decode_sk_kernel(const DecodeArgs a) {
  using St = ValuHeads<KV, D, BS, HPW, kQLds>;
  constexpr int NLOAD = St::NLOAD, RU = St::RU, DPI = St::DPI, TILE = Geo<KV, D, BS>::TILE;

  __shared__ float p_lds[NW][HPW][BS];
  __shared__ u32x4 q_lds[kQLds ? NW : 1][kQLds ? St::QU : 1];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = blockIdx.x * NW + w;
  const int R = a.sk_workers;
  if (gw >= R) return;
  const int G = a.Hq / a.Hkv, groups = G / HPW;
  const int64_t CU = a.sk_cu;
  const int64_t T = CU * a.Hkv * groups;
  int64_t x = (int64_t)gw * T / R;
  const int64_t x1 = (int64_t)(gw + 1) * T / R;
  const size_t blk_stride = (size_t)a.Hkv * TILE;
  float* ws_o = a.ws;
  float* ws_ml = a.ws + (size_t)(R + (size_t)a.Hkv * groups * a.S) * HPW * D;

  St st;
  while (x < x1) {
    const int hg = (int)(x / CU);
    const int rem = (int)(x - (int64_t)hg * CU);
    const int s = min(__builtin_amdgcn_readfirstlane(find_seq(a.tile_off, a.S, rem, lane)), a.S - 1);
    const int off = a.tile_off[s];
    const int n_s = a.tile_off[s + 1] - off;
    const int j0 = rem - off;
    const int jn = (int)min((int64_t)n_s, (int64_t)j0 + (x1 - x));
    // offsets that are not running sums ending at sk_cu: stop rather than
    // loop without progress or index outside the table
    if (j0 < 0 || jn <= j0) break;
    x += jn - j0;

    int L = a.lens[s];
    bool bad = false;
    if (L < 0) { L = 0; bad = true; }
    if (L > a.max_blocks * BS) { L = a.max_blocks * BS; bad = true; }
    const int nt = (L + BS - 1) / BS;
    if (nt != n_s) bad = true;               // tile offsets disagree with the length
    const int jend = min(jn, nt), jfirst = min(j0, jend);
    const int hkv = hg / groups;
    const int qh0 = hkv * G + (hg % groups) * HPW;
    const int32_t* __restrict__ tbl = a.tables + (size_t)s * a.max_blocks;

    // STORE: the new token goes to the item's last tile, stored from the
    // start hook and waited for just before that tile is loaded.
    const bool my_store = STORE && !bad && L > 0 && jend == nt && jfirst < jend;

    if constexpr (kQLds) {
      __builtin_amdgcn_wave_barrier();   // the previous item's reads of q_lds come first
      St::fill_q(a, s, qh0, q_lds[w], lane, 64);
      __builtin_amdgcn_wave_barrier();
      st.qs = q_lds[w];
    } else {
      st.load_q(a, s, qh0, lane);
    }
    st.reset();
    const size_t head_off = (size_t)hkv * TILE;
    tile_loop<NBUF, NLOAD, 1>(tbl, jfirst, jend, a.nb, (const uint8_t*)a.kc + head_off + lane * 16,
                              (const uint8_t*)a.vc + head_off + lane * 16, blk_stride, lane, bad,
                              [&](int j, const u32x4* kr, const u32x4* vr) {
                                st.tile(a.qk_mult, j, L, kr, vr, p_lds[w], lane);
                              },
                              my_store ? nt - 1 : -1,
                              [&] {
                                if constexpr (STORE) {
                                  if (my_store) store_new_token<KV, D, BS>(a, s, hkv, L, lane);
                                }
                              });

    // ---- this piece: the output when it is the whole item, else a partial ----
    const bool whole = j0 == 0 && jn == n_s;
    const size_t slot = (size_t)gw + (size_t)hg * a.S + s;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const float lt = tile_sum<BS>(st.l_run[hh]);
      const float inv = lt > 0.f ? a.v_mult / lt : 0.f;
#pragma unroll
      for (int l = 0; l < NLOAD; ++l) {
        const float v = st.dim_sum(hh, l);
        const int dim = l * DPI + lane / RU;
        if (lane % RU == 0) {
          if (whole) {
            const float r = bad ? NAN : v * inv;
            const size_t oi = ((size_t)s * a.Hq + qh0 + hh) * D + dim;
            if constexpr (St::F32)
              ((float*)a.out)[oi] = r;
            else
              ((uint16_t*)a.out)[oi] = f32_to_bf16(r);
          } else {
            ws_o[(slot * HPW + hh) * D + dim] = bad ? NAN : v * a.v_mult;
          }
        }
      }
      if (!whole && lane == 0) {
        ws_ml[(slot * HPW + hh) * 2] = st.m_run[hh];
        ws_ml[(slot * HPW + hh) * 2 + 1] = bad ? NAN : lt;
      }
    }
  }
}

// Heads per workgroup: the largest power of two (at most 8) dividing G whose
// per-head registers fit the budget: the query dims of the lane's key chunks
// when q lives in VGPRs (64 VGPRs in all for tiles of up to 4 KiB, 32 for
// larger tiles, whose two buffers of key and value loads take 128 VGPRs or
// more: with two heads the kernel would exceed 256 VGPRs and spill into
// accumulation registers at one wave per SIMD), else the accumulators and
// the probabilities of a value load (48 VGPRs in all).
template <int KV, int D, int BS>
constexpr int max_hpw() {
  using Gm = Geo<KV, D, BS>;
  constexpr int per_head = kQLds ? Gm::NLOAD + (Gm::F32 ? 4 : Gm::PPC)
                                 : (Gm::F32 ? Gm::NLOAD * 4 : Gm::NLOAD * Gm::PPC);
  constexpr int budget = kQLds ? 48 : Gm::TILE <= 4096 ? 64 : 32;
  return budget / per_head >= 8 ? 8 : budget / per_head >= 4 ? 4 : budget / per_head >= 2 ? 2 : 1;
}

template <int KV, int D, int BS>
int heads_per_wg(int G) {
  constexpr int MAXH = max_hpw<KV, D, BS>();
  int h = 1;
  while (h * 2 <= MAXH && G % (h * 2) == 0) h *= 2;
  return h;
}

// Shared-item launch; store: the decode step's new-token store (needs one
// workgroup per kv head, HPW == G).
template <int KV, int D, int BS, int HPW>
int launch_t(const DecodeArgs& a, bool store, hipStream_t st) {
  const int groups = a.Hq / a.Hkv / HPW;
  if (store && groups != 1) return (int)hipErrorInvalidValue;
  dim3 block(kWaves * 64);
  dim3 grid((a.partition > 0 ? a.total_parts : a.S) * a.Hkv * groups);
  if (a.partition > 0) {
    if (store)
      hipLaunchKernelGGL((decode_kernel<KV, D, BS, HPW, kWaves, valu_bufs<HPW, Geo<KV, D, BS>::TILE>(), true, true>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((decode_kernel<KV, D, BS, HPW, kWaves, valu_bufs<HPW, Geo<KV, D, BS>::TILE>(), true, false>), grid, block, 0, st, a);
  } else {
    if (store)
      hipLaunchKernelGGL((decode_kernel<KV, D, BS, HPW, kWaves, valu_bufs<HPW, Geo<KV, D, BS>::TILE>(), false, true>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((decode_kernel<KV, D, BS, HPW, kWaves, valu_bufs<HPW, Geo<KV, D, BS>::TILE>(), false, false>), grid, block, 0, st, a);
  }
  return (int)hipGetLastError();
}

// Stream-K launch: a.sk_workers waves in workgroups of kSkWaves.
template <int KV, int D, int BS, int HPW>
int launch_sk_t(const DecodeArgs& a, bool store, hipStream_t st) {
  const int groups = a.Hq / a.Hkv / HPW;
  if (store && groups != 1) return (int)hipErrorInvalidValue;
  dim3 block(kSkWaves * 64), grid((a.sk_workers + kSkWaves - 1) / kSkWaves);
  if (store)
    hipLaunchKernelGGL((decode_sk_kernel<KV, D, BS, HPW, kSkWaves, sk_bufs<Geo<KV, D, BS>::TILE>(), true>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((decode_sk_kernel<KV, D, BS, HPW, kSkWaves, sk_bufs<Geo<KV, D, BS>::TILE>(), false>), grid, block, 0, st, a);
  return (int)hipGetLastError();
}

// Resident stream-K waves on this device: workgroups per CU at full
// occupancy times CUs times waves per workgroup.
template <int KV, int D, int BS, int HPW>
int sk_workers_t() {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(&decode_sk_kernel<KV, D, BS, HPW, kSkWaves, sk_bufs<Geo<KV, D, BS>::TILE>(), false>),
          kSkWaves * 64, 0) != hipSuccess)
    return -1;
  return max(1, per_cu) * cus * kSkWaves;
}

template <int KV, int D, int BS, class F>
int with_hpw(int G, F&& f) {
  constexpr int MAXH = max_hpw<KV, D, BS>();
  const int h = heads_per_wg<KV, D, BS>(G);
  if constexpr (MAXH >= 8) if (h == 8) return f(std::integral_constant<int, 8>());
  if constexpr (MAXH >= 4) if (h == 4) return f(std::integral_constant<int, 4>());
  if constexpr (MAXH >= 2) if (h == 2) return f(std::integral_constant<int, 2>());
  return f(std::integral_constant<int, 1>());
}

template <int KV, class F>
int with_shape(const DecodeArgs& a, F&& f) {
  const int G = a.Hq / a.Hkv;
  auto go = [&](auto d, auto bs) {
    return with_hpw<KV, decltype(d)::value, decltype(bs)::value>(
        G, [&](auto h) { return f(d, bs, h); });
  };
  if (a.D == 64)
    return a.BS == 16 ? go(std::integral_constant<int, 64>(), std::integral_constant<int, 16>())
                      : go(std::integral_constant<int, 64>(), std::integral_constant<int, 32>());
  return a.BS == 16 ? go(std::integral_constant<int, 128>(), std::integral_constant<int, 16>())
                    : go(std::integral_constant<int, 128>(), std::integral_constant<int, 32>());
}

template <int KV>
int launch_valu(const DecodeArgs& a, bool store, hipStream_t st) {
  return with_shape<KV>(a, [&](auto d, auto bs, auto h) {
    return launch_t<KV, decltype(d)::value, decltype(bs)::value, decltype(h)::value>(a, store, st);
  });
}

template <int KV>
int launch_valu_sk(const DecodeArgs& a, bool store, hipStream_t st) {
  return with_shape<KV>(a, [&](auto d, auto bs, auto h) {
    return launch_sk_t<KV, decltype(d)::value, decltype(bs)::value, decltype(h)::value>(a, store, st);
  });
}

template <int KV>
int valu_heads_per_wg(const DecodeArgs& a) {
  return with_shape<KV>(a, [&](auto, auto, auto h) { return (int)decltype(h)::value; });
}

template <int KV>
int valu_sk_workers(const DecodeArgs& a) {
  return with_shape<KV>(a, [&](auto d, auto bs, auto h) {
    return sk_workers_t<KV, decltype(d)::value, decltype(bs)::value, decltype(h)::value>();
  });
}

}  // namespace valu
}  // namespace pkv
