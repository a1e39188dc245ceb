// Pieces shared by the decode kernels: locating a workgroup's (sequence,
// partition, head group), the chunked block-table walk with its prefetch
// ring of tiles, and the merge of the waves' softmax states.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>

#include "pkv_device.h"
#include "pkv_internal.h"

// Launch shape (fixed at build time; -D overrides exist for tuning sweeps).
#ifndef PKV_DECODE_WAVES
#define PKV_DECODE_WAVES 4
#endif
#ifndef PKV_DECODE_NT
#define PKV_DECODE_NT 1
#endif
#ifndef PKV_DECODE_DEPTH
#define PKV_DECODE_DEPTH 1
#endif
#ifndef PKV_SK_WAVES
#define PKV_SK_WAVES 4
#endif
#ifndef PKV_DECODE_QLDS
#define PKV_DECODE_QLDS 0
#endif
#ifndef PKV_MFMA_DEPTH
#define PKV_MFMA_DEPTH 0
#endif

namespace pkv {
namespace dec {

constexpr int kWaves = PKV_DECODE_WAVES;
constexpr int kSkWaves = PKV_SK_WAVES;            // waves per workgroup, stream-K kernels
constexpr bool kQLds = PKV_DECODE_QLDS;           // vector-ALU kernels: query rows in LDS

constexpr int kBufs = PKV_DECODE_DEPTH + 1;      // tiles in registers per wave (VALU kernel)
#ifndef PKV_DECODE_DEPTH_1H
#define PKV_DECODE_DEPTH_1H 2
#endif
// Tiles in registers per wave of the split-K vector-ALU kernel holding HPW
// query heads over tiles of TILE bytes: one more when a wave holds a single
// head, whose query takes few registers, and a tile is at most 4 KiB (32
// VGPRs for its key and value loads).  One kv head per query head: 3 tiles
// in flight measured 2.5% faster; 4 heads per wave: slower, at 244 VGPRs.
// A 16 KiB tile (fp32, head_dim 128, block 32) takes 128 VGPRs for its key
// and value loads, so such tiles go one at a time (no register ring; the
// other waves of the compute unit keep loads in flight).
template <int HPW, int TILE>
constexpr int valu_bufs() {
  return TILE > 8192 ? 1 : HPW == 1 && TILE <= 4096 ? PKV_DECODE_DEPTH_1H + 1 : kBufs;
}
// Same for the stream-K vector-ALU kernel.
template <int TILE>
constexpr int sk_bufs() { return TILE > 8192 ? 1 : kBufs; }
constexpr int kMfmaBufs = PKV_MFMA_DEPTH + 1;    // same, matrix-core kernel

// Number of i in [1, S] with part_off[i] <= idx, i.e. the sequence owning
// flat partition idx (part_off is non-decreasing, part_off[0] = 0).
__device__ __forceinline__ int find_seq(const int32_t* __restrict__ part_off, int S, int idx,
                                        int lane) {
  int s = 0;
  for (int base = 1; base <= S; base += 64) {
    const int i = base + lane;
    const bool le = i <= S && part_off[i] <= idx;
    s += __popcll(__ballot(le));
  }
  return s;
}

// Longest-first dispatch of split-K partitions.  Launch slots are filled
// in workgroup-id order, so the slot -> partition map decides which work is
// left for the end of the grid.  Every partition but a sequence's last has P
// tokens; the last ones vary from 1 to P tokens.  Slots x < F = total_parts -
// S take the F non-last partitions in sequence order; slot F + r takes the
// last partition with the r-th most tiles (ties: lower sequence first), so
// the grid ends on its shortest pieces ("PagedAttention Kernel：大模型推理优化
// 的显存管理革新" §3.2: pages of uneven length leave units idle unless the
// work is balanced).  The rank is found with a binary search over tile
// counts, one ballot per 64 sequences and step, on counts held in registers;
// with more than 64 * kOrderChunks sequences, or offsets that do not add up
// or give a sequence no partition, slots map to partitions in sequence
// order.  Returns the sequence and its partition; the workspace row stays
// part_off[s] + part.
constexpr int kOrderChunks = 8;

// part_off / lens: the partition offsets and lengths to read (the
// arguments' device arrays, or a copy of them in LDS).
template <int BS>
__device__ __forceinline__ void split_slot(const DecodeArgs& a, int x, int lane, int& s,
                                           int& part, const int32_t* __restrict__ part_off,
                                           const int32_t* __restrict__ lens) {
  const int S = a.S;
  const int F = a.total_parts - S;
  auto in_order = [&] {
    // clamped: offsets that end below total_parts leave slots past the last
    // sequence's partitions, which then cover no tokens (their partial rows
    // are never read)
    s = min(__builtin_amdgcn_readfirstlane(find_seq(part_off, S, x, lane)), S - 1);
    part = x - part_off[s];
  };
  if (S > 64 * kOrderChunks || F < 0 || part_off[S] != a.total_parts) {
    in_order();
    return;
  }
  if (x < F) {
    // sequence s owns non-last slots [part_off[s] - s, part_off[s+1] - s - 1)
    int c = 0;
    bool empty = false;   // a sequence without partitions
    for (int base = 1; base <= S; base += 64) {
      const int i = base + lane;
      const int hi = i <= S ? part_off[i] : 0, lo = i <= S ? part_off[i - 1] : 0;
      c += __popcll(__ballot(i <= S && hi - i <= x));
      empty |= __ballot(i <= S && hi - lo < 1) != 0;
    }
    if (empty) {
      in_order();
      return;
    }
    s = __builtin_amdgcn_readfirstlane(c);
    part = x - (part_off[s] - s);
    return;
  }
  const int r = x - F;                      // rank among the last partitions, < S
  const int kmax = a.partition / BS;        // tiles of a full partition
  int key[kOrderChunks];
  bool empty = false;
#pragma unroll
  for (int ch = 0; ch < kOrderChunks; ++ch) {
    const int i = ch * 64 + lane;
    key[ch] = -1;                           // no sequence: never counted
    int n = 1;
    if (ch * 64 < S && i < S) {
      int L = lens[i];
      L = L < 0 ? 0 : min(L, a.max_blocks * BS);
      n = part_off[i + 1] - part_off[i];
      const int t = L - (n - 1) * a.partition;
      key[ch] = min(max((t + BS - 1) / BS, 0), kmax);
    }
    if (ch * 64 < S) empty |= __ballot(n < 1) != 0;
  }
  if (empty) {
    in_order();
    return;
  }
  auto count_gt = [&](int c) {
    int n = 0;
#pragma unroll
    for (int ch = 0; ch < kOrderChunks; ++ch)
      if (ch * 64 < S) n += __popcll(__ballot(key[ch] > c));
    return n;
  };
  // smallest c with count_gt(c) <= r: the tile count of the rank-r piece
  int lo = 0, hi = kmax;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (count_gt(mid) <= r) hi = mid; else lo = mid + 1;
  }
  int idx = r - count_gt(lo);               // position among the pieces with lo tiles
  int found = S - 1;
#pragma unroll
  for (int ch = 0; ch < kOrderChunks; ++ch) {
    if (ch * 64 < S) {
      const uint64_t m = __ballot(key[ch] == lo);
      const int n = __popcll(m);
      if (idx >= 0 && idx < n) {
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        const uint64_t sel = __ballot(key[ch] == lo && below == idx);
        found = ch * 64 + (int)__builtin_ctzll(sel);
      }
      idx -= n;
    }
  }
  s = __builtin_amdgcn_readfirstlane(found);
  part = part_off[s + 1] - part_off[s] - 1;
}

// One 16-byte load of streamed key/value data.
__device__ __forceinline__ u32x4 load16(const uint8_t* p) {
#if PKV_DECODE_NT
  return __builtin_nontemporal_load((const u32x4*)p);
#else
  return *(const u32x4*)p;
#endif
}

// Split-K partitions of a sequence of L tokens: ceil(L / P), at least one.
__device__ __forceinline__ int split_parts(int L, int P) {
  return L > 0 ? (int)(((int64_t)L + P - 1) / P) : 1;
}

// What one workgroup works on.
struct Work {
  int s;       // sequence
  int nparts;  // partitions of that sequence
  int t0, t1;  // token range [t0, t1) of this partition
  int jend;    // one past the last block of the range
  int L;       // context length (clamped to the table)
  int p0;      // first flat partition of the sequence (SPLIT)
  int hkv;     // kv head
  int qh0;     // first query head of the group
  int item;    // flat work index (partial row of the workspace)
  bool bad;    // length out of range: the output becomes NaN
};

// `item` is the flat work index: the split-K partition (SPLIT) or the
// sequence (one pass); `hg` the head group (kv head * groups + group).
template <bool SPLIT, int BS>
__device__ __forceinline__ Work locate(const DecodeArgs& a, int hpw, int lane, int item, int hg) {
  Work wk;
  const int G = a.Hq / a.Hkv;
  const int groups = G / hpw;
  wk.hkv = hg / groups;
  wk.qh0 = wk.hkv * G + (hg % groups) * hpw;
  wk.item = item;
  int part;
  int tstart = 0, nsuf = 0;
  if constexpr (SPLIT) {
    if (a.t_start) {
      wk.s = min(__builtin_amdgcn_readfirstlane(find_seq(a.part_off, a.S, item, lane)), a.S - 1);
      part = item - a.part_off[wk.s];
    } else {
      split_slot<BS>(a, item, lane, wk.s, part, a.part_off, a.lens);
    }
    wk.p0 = a.part_off[wk.s];
    wk.item = wk.p0 + part;
    wk.nparts = a.part_off[wk.s + 1] - wk.p0;
    if (a.t_start) {   // shared-prefix suffix pass: always a partial row
      tstart = a.t_start[wk.s];
      wk.item = a.row_off[wk.s] + part;
      nsuf = wk.nparts;
      wk.nparts = 2;
    }
  } else {
    wk.s = item;
    wk.p0 = item;
    part = 0;
    wk.nparts = 1;
  }
  int L = a.lens[wk.s];
  wk.bad = false;
  if (L < 0) { L = 0; wk.bad = true; }
  if (L > a.max_blocks * BS) { L = a.max_blocks * BS; wk.bad = true; }
  // split-K offsets must describe this length: ceil(L / P) partitions (one
  // for L = 0); stale offsets would drop tokens or leave rows unwritten
  if (SPLIT && !a.t_start && wk.nparts != split_parts(L, a.partition)) wk.bad = true;
  // suffix pass: ceil((L - tstart) / P) partitions of the sequence's own
  // tokens (a sequence without own tokens may hold one empty partition)
  if (SPLIT && a.t_start) {
    const int own = L - tstart;
    const int want = own > 0 ? (int)(((int64_t)own + a.partition - 1) / a.partition) : 0;
    if (own < 0 || (nsuf != want && !(want == 0 && nsuf == 1))) wk.bad = true;
  }
  wk.L = L;
  wk.t0 = SPLIT ? tstart + part * a.partition : 0;
  wk.t1 = SPLIT ? min(L, wk.t0 + a.partition) : L;
  wk.jend = (wk.t1 + BS - 1) / BS;
  return wk;
}

// Walk this wave's tiles jfirst, jfirst + NW, ... < jend.  Table entries
// come 64 tiles at a time from one vector load (lane i holds the entry of
// the chunk's i-th tile, read back with v_readlane) issued while no tile load
// is in flight, so no tile load waits on a lookup.  Within a chunk a ring of
// NBUF register buffers keeps the next tiles in flight while one is consumed
// ("PagedAttention Kernel：大模型推理优化的显存管理革新" §2.2: prefetch the
// next page while computing the current one).  The steady-state loop issues
// its prefetches unconditionally, so the compiler's wait counts leave exactly
// the younger tiles outstanding.  kbase/vbase point at this lane's 16 bytes
// of load 0 of block 0 (head and lane offsets included); load l of a tile is
// l KiB further.  A block id outside [0, nb) sets `bad` and reads block 0.
// start() runs once, after the first chunk's table load is issued and before
// any tile load (so memory operations it issues share the table load's wait
// and precede every tile load); j_sync >= 0: every earlier memory operation
// of the wave (a store into that tile, say) completes before tile j_sync is
// loaded.
struct NoStart {
  __device__ __forceinline__ void operator()() const {}
};

template <int NBUF, int NLOAD, int NW, class Proc, class Start = NoStart>
__device__ __forceinline__ void tile_loop(const int32_t* __restrict__ tbl, int jfirst, int jend,
                                          int nb, const uint8_t* kbase, const uint8_t* vbase,
                                          size_t blk_stride, int lane, bool& bad, Proc&& process,
                                          int j_sync = -1, Start&& start = Start()) {
  u32x4 kbuf[NBUF][NLOAD], vbuf[NBUF][NLOAD];
  int tbl_v = 0, chunk0 = 0;
  auto load_tile = [&](int jj, u32x4* kd, u32x4* vd) {
    if (jj == j_sync) __builtin_amdgcn_s_waitcnt(0);
    int b = __builtin_amdgcn_readlane(tbl_v, (jj - chunk0) / NW);
    if ((unsigned)b >= (unsigned)nb) { bad = true; b = 0; }
    const uint8_t* kt = kbase + (size_t)b * blk_stride;
    const uint8_t* vt = vbase + (size_t)b * blk_stride;
#pragma unroll
    for (int l = 0; l < NLOAD; ++l) kd[l] = load16(kt + l * 1024);
#pragma unroll
    for (int l = 0; l < NLOAD; ++l) vd[l] = load16(vt + l * 1024);
  };
  for (chunk0 = jfirst; chunk0 < jend; chunk0 += 64 * NW) {
    const int n = min(64, (jend - chunk0 + NW - 1) / NW);  // tiles of this wave in the chunk
    tbl_v = lane < n ? tbl[chunk0 + lane * NW] : 0;
    if (chunk0 == jfirst) start();
    auto tile = [&](int k) { return chunk0 + k * NW; };
    int k = 0;
    if (n >= NBUF) {
#pragma unroll
      for (int b = 0; b < NBUF; ++b) load_tile(tile(b), kbuf[b], vbuf[b]);
      for (; k + 2 * NBUF <= n; k += NBUF) {
#pragma unroll
        for (int b = 0; b < NBUF; ++b) {
          process(tile(k + b), kbuf[b], vbuf[b]);
          load_tile(tile(k + NBUF + b), kbuf[b], vbuf[b]);
        }
      }
    } else {
#pragma unroll
      for (int b = 0; b < NBUF; ++b)
        if (b < n) load_tile(tile(b), kbuf[b], vbuf[b]);
    }
    // buffers hold tiles k .. k+NBUF-1 (those < n); at most 2*NBUF-1 remain
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      if (k + b < n) {
        process(tile(k + b), kbuf[b], vbuf[b]);
        if (k + NBUF + b < n) load_tile(tile(k + NBUF + b), kbuf[b], vbuf[b]);
      }
    }
#pragma unroll
    for (int b = 0; b < NBUF; ++b)
      if (k + NBUF + b < n) process(tile(k + NBUF + b), kbuf[b], vbuf[b]);
  }
}

// Merge the NW waves' (m, l, o) of HPW heads: M = max m_w, L = sum l_w 2^(m_w - M),
// O = sum o_w 2^(m_w - M).  A sequence covered by one partition gets its
// output O / L (times the value scale); otherwise the partial (M, L, O) goes
// to the workspace for the split-K reduce.
template <int HPW, int D, int NW, bool F32OUT>
__device__ __forceinline__ void merge_store(const DecodeArgs& a, const Work& wk, bool final_out,
                                            const float (&o_lds)[NW][HPW][D],
                                            const float (&m_lds)[NW][HPW],
                                            const float (&l_lds)[NW][HPW],
                                            const int (&bad_lds)[NW]) {
  int any_bad = 0;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) any_bad |= bad_lds[ww];
  float* ws_o = a.ws;
  float* ws_ml = a.ws + (size_t)(a.ws_rows ? a.ws_rows : a.total_parts) * a.Hq * D;
  for (int i = threadIdx.x; i < HPW * D; i += NW * 64) {
    const int hh = i / D, dim = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, m_lds[ww][hh]);
    float Ls = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float f = __builtin_amdgcn_exp2f(m_lds[ww][hh] - M);
        Ls = fmaf(l_lds[ww][hh], f, Ls);
        O = fmaf(o_lds[ww][hh][dim], f, O);
      }
    }
    const int qh = wk.qh0 + hh;
    if (final_out) {
      float r = Ls > 0.f ? O * a.v_mult / Ls : 0.f;
      if (any_bad) r = NAN;
      const size_t oi = ((size_t)wk.s * a.Hq + qh) * D + dim;
      if constexpr (F32OUT)
        ((float*)a.out)[oi] = r;
      else
        ((uint16_t*)a.out)[oi] = f32_to_bf16(r);
    } else {
      const size_t pi = (size_t)wk.item * a.Hq + qh;
      ws_o[pi * D + dim] = any_bad ? NAN : O * a.v_mult;
      if (dim == 0) {
        ws_ml[pi * 2] = M;
        ws_ml[pi * 2 + 1] = any_bad ? NAN : Ls;
      }
    }
  }
}

// Decode step: stores sequence s's new token (position L - 1; kv head hkv)
// into the slot its table gives, from the lanes of the one wave that will
// read that block; returns the block's tile index (the wave's j_sync) or -1
// when there is nothing to store.  Called from tile_loop's start hook, so
// the new row's loads share the table load's wait and the stores precede
// every tile load of the wave.
template <int KV, int D, int BS>
__device__ __forceinline__ void store_new_token(const DecodeArgs& a, int s, int hkv, int L,
                                                int lane) {
  constexpr int X = 16 / (KV == PKV_F32 ? 4 : KV == PKV_BF16 ? 2 : 1);
  const int pos = L - 1;
  const int blk = a.tables[(size_t)s * a.max_blocks + pos / BS];
  if ((unsigned)blk >= (unsigned)a.nb) return;
  for (int c = lane; c < D / X; c += 64)
    write_kv_unit<KV>(a.new_k, a.new_v, (uint8_t*)a.kc, (uint8_t*)a.vc, s, hkv, c,
                      blk * BS + pos % BS, a.Hkv, D, BS, a.k_inv, a.v_inv);
}

}  // namespace dec
}  // namespace pkv
