// Chunked prefill over the paged cache: the last C tokens of a sequence are
// a chunk of new query rows, and chunk row i (position p = L - C + i)
// attends the sequence's tokens 0 .. p, all read through the block table
// ("Day 6/90 of Inference Engineering": the table makes the scattered blocks
// read as one contiguous cache; "PagedAttention Kernel：大模型推理优化的显存
// 管理革新" §3.1: QK^T per block, softmax, PV block by block on matrix
// units; fp32 accumulation per §6).
//
// One wave carries 32 query rows, (position, query head) pairs of one kv head
// in position-major order, and walks the blocks its rows can see two at a
// time (32 tokens).  Both products run transposed on
// v_mfma_f32_32x32x16_bf16 so that every lane owns one query row:
//   S^T[32 tokens x 32 rows] = K[tokens x 128] . Q^T[128 x rows]   (8 k-steps)
//   O^T[128 dims x 32 rows] += V^T[dims x 16 tokens] . P^T[16 tokens x rows]
//                                                   (per block, 4 dim slices)
// The row's running max and sum then live in the lane (no cross-lane
// reductions per tile) and the rescale of O is a per-lane multiply.
//
// Lane layouts of the 32x32x16 bf16 MFMA (lane l, col = l % 32, g = l / 32):
//   A[i][k]: lane holds row i = col, k = 8g .. 8g+7
//   B[k][j]: lane holds column j = col, k = 8g .. 8g+7
//   C[i][j]: register r holds row 8(r/4) + 4g + r%4, column col
// S^T: A row i of a block pair is the key of token sigma(i) (bits 2 and 3 of
// the in-block index swapped), loaded as its 16-byte key unit for dims
// 16sl + 8g .. +7; then C register 8b + i of lane (col, g) holds token
// 16b + 8g + i of block b of the pair, which is exactly the B-operand slot
// (k = 8g + i) that P^T needs for block b, and V^T's A operand (dim row col,
// k = tokens 8g .. 8g+7) is one 16-byte load of the value row.

#include <hip/hip_runtime.h>

#include <cmath>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 128, kBS = 16;
constexpr int kTile = kBS * kD * 2;   // bytes of a bf16 (block, kv head) tile
constexpr int kRows = 32;             // query rows per wave
constexpr int kNW = 4;                // waves per workgroup

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Read-only int32 arrays (lengths, row offsets, block tables) through the
// constant address space: they do not change during the launch, so
// wave-uniform reads become scalar loads and everything derived from them
// (the wave's block range, the table address) stays in scalar registers.
typedef const int32_t __attribute__((address_space(4))) * cint_ptr;
__device__ __forceinline__ cint_ptr as_const(const int32_t* p) { return (cint_ptr)p; }

// LDS ring: kStages block pairs per workgroup, each [K block 0][K block 1]
// [V block 0][V block 1] of kTile bytes.  Keys keep the pool's layout; the
// 16-byte units of a value tile are swizzled so that the transposed reads
// (lanes 0..15 reading dim rows 0..15 at one half) hit distinct banks: dim
// row d's half h sits in unit 2d + (h ^ ((d >> 3) & 1)).
constexpr int kStages = 3;
constexpr int kPairBytes = 4 * kTile;

__device__ __forceinline__ int vunit(int d, int h) { return 2 * d + (h ^ ((d >> 3) & 1)); }

// Workgroup wg (after the XCD remap) covers query block qb of (s, hkv):
// rows [qb * kNW * 32, (qb + 1) * kNW * 32) of the C * G rows of that kv head.
// Its waves share one copy of each block pair in LDS: every wave loads a
// quarter of the pair straight into LDS (16-byte direct loads), a barrier per
// pair publishes it, and each wave reads its matrix-core operands from LDS.
__global__ __launch_bounds__(kNW * 64) __attribute__((amdgpu_waves_per_eu(3)))
void prefill_kernel(const PrefillArgs a) {
  __shared__ __align__(16) uint8_t ring[kStages][kPairBytes];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, g = lane >> 5;

  // Workgroup ids go round robin over the 8 XCDs.  XCD x takes the
  // (sequence, kv head) units x, x + 8, x + 16, ... with all query blocks of
  // a unit in a row, so the blocks a unit's query blocks all read stay in
  // that XCD's L2; units run kv head first, so with 8 kv heads every XCD
  // serves one head of every sequence and gets the same amount of work
  // whatever the length mix (a contiguous eighth of the units per XCD left
  // one XCD with 1.28x the mean work on the 16-sequence prefill workload).
  // Within an XCD the units run longest first: with at most 64 sequences,
  // unit slot v takes kv head v % H_kv of the sequence with the (v / H_kv)-th
  // most visible (row, token) pairs, C (2L - C + 1) / 2 (ties: lower index),
  // so each XCD ends on its cheapest units.
  const int nunits = a.total_wg / a.qblocks;
  const int k = blockIdx.x / 8;
  const int vslot = (int)(blockIdx.x % 8) + 8 * (k / a.qblocks);
  const int qb = k % a.qblocks;
  if (vslot >= nunits) return;   // whole workgroup
  const int hkv = vslot % a.Hkv;
  int s = vslot / a.Hkv;
  if (a.S <= 64) {
    float key = -1.f;
    if (lane < a.S) {
      const float Li = (float)a.lens[lane];
      const float Ci = (float)(a.q_start[lane + 1] - a.q_start[lane]);
      key = fmaxf(Ci * (2.f * Li - Ci + 1.f), 0.f);
    }
    int rank = 0;
    for (int j = 0; j < a.S; ++j) {
      const float kj = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(key), j));
      rank += (kj > key || (kj == key && j < lane)) ? 1 : 0;
    }
    const uint64_t hit = __ballot(lane < a.S && rank == s);
    s = __builtin_amdgcn_readfirstlane(hit ? (int)__builtin_ctzll(hit) : s);
  }
  const int G = a.Hq / a.Hkv;
  const int r0q = as_const(a.q_start)[s];
  const int C = as_const(a.q_start)[s + 1] - r0q;
  const int L = as_const(a.lens)[s];
  const int nrows = C * G;
  const int wg_row0 = qb * kNW * kRows;
  if (wg_row0 >= nrows) return;   // whole workgroup: no rows here
  // a chunk longer than its context or a context beyond the table: NaN rows
  bool bad = C > L || L > a.max_blocks * kBS || C < 0;
  const int row0 = wg_row0 + w * kRows;
  const bool active = row0 < nrows;   // a wave past the chunk still loads and syncs

  // ---- this lane's query row ----
  const int row = row0 + col;
  const bool row_ok = row < nrows;
  const int pl = row_ok ? row / G : C - 1;       // chunk position (padding rows: the last)
  const int qh = hkv * G + (row_ok ? row % G : 0);
  const int p = L - C + pl;                       // tokens 0 .. p are visible to this row
  // first row's position of this wave and last row's of the workgroup;
  // uniform (the divisions expand on the vector ALUs, so their results are
  // moved back to scalar registers)
  const int p_min = __builtin_amdgcn_readfirstlane(L - C + min(row0, nrows - 1) / G);
  const int wg_last = min(nrows - 1, wg_row0 + kNW * kRows - 1);
  const int wg_p_max = __builtin_amdgcn_readfirstlane(L - C + wg_last / G);
  const int nblk = bad ? 0 : (wg_p_max + kBS) / kBS;   // blocks holding tokens 0 .. wg_p_max
  const int npairs = (nblk + 1) / 2;

  // Scores are used as exp2(s * qk - m) with qk = |scale| * log2(e) > 0: a
  // negative scale flips the sign bits of q (exact in bf16), and a zero scale
  // becomes a tiny positive one (every score ~0, as it should be) so that a
  // hidden token's -inf stays -inf.
  const float qk = fmaxf(fabsf(a.qk_mult), 1e-30f);
  const uint32_t qflip = a.qk_mult < 0.f ? 0x80008000u : 0u;
  u32x4 qv[8];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + ((size_t)(r0q + pl) * a.Hq + qh) * kD;
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      qv[sl] = row_ok && !bad ? *(const u32x4*)(qrow + 16 * sl + 8 * g) : u32x4{0, 0, 0, 0};
      qv[sl] ^= qflip;
    }
  }

  // scalar table reads stay off the vector load counter
  const cint_ptr tbl = as_const(a.tables + (size_t)s * a.max_blocks);
  const size_t head_off = (size_t)hkv * kTile;
  const size_t blk_stride = (size_t)a.Hkv * kTile;

  // ---- staging: this wave's quarter of pair jp into ring stage st ----
  // key units: identity; value units: lane slot q = 64w + lane holds dim
  // row q / 2, half (q & 1) ^ bit 3 of that row
  const int kq = w * 64 + lane;
  const int vd = kq >> 1, vh = (kq & 1) ^ ((vd >> 3) & 1);
  auto stage_pair = [&](int jp, int st) {   // jp, st wave-uniform, jp < npairs
    const int j0 = 2 * jp;
    int id0 = tbl[j0];
    int id1 = tbl[min(j0 + 1, nblk - 1)];
    if ((unsigned)id0 >= (unsigned)a.nb || (unsigned)id1 >= (unsigned)a.nb) {
      bad = true;
      id0 = id1 = 0;
    }
    if (j0 + 1 >= nblk) id1 = id0;   // past the last block: a copy of the first, hidden
    const size_t b[2] = {(size_t)id0 * blk_stride + head_off, (size_t)id1 * blk_stride + head_off};
    uint8_t* dst = ring[st] + w * 1024;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)((const uint8_t*)a.kc + b[t] + kq * 16),
          (void __attribute__((address_space(3)))*)(dst + t * kTile), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)((const uint8_t*)a.vc + b[t] +
                                                           (2 * vd + vh) * 16),
          (void __attribute__((address_space(3)))*)(dst + (2 + t) * kTile), 16, 0, 0);
    }
  };

  // Value tokens past the workgroup's last position (wg_p_max) exist only in
  // its last pair; their probabilities are 0 for every row, but the bytes
  // may lie past the context (anything, NaN included) or repeat the pair's
  // first block.  Once that pair is in LDS, the workgroup zeroes them there
  // (2 blocks x 128 dim rows x 2 halves = 512 units of 8 tokens), so the
  // product loop needs no per-pair masking.  Tokens up to wg_p_max are
  // context tokens, finite like every stored value.
  auto zero_value_tail = [&](int st, int jp) {   // workgroup-uniform jp
    const int zero_from = wg_p_max + 1 - 32 * jp;   // first pair token to zero
    if (zero_from >= 32) return;
    for (int u = threadIdx.x; u < 512; u += kNW * 64) {
      const int b = u >> 8, d = (u >> 1) & 127, h = u & 1;
      const int keep = min(max(zero_from - (16 * b + 8 * h), 0), 8);   // tokens kept, 0..8
      if (keep == 8) continue;
      u32x4* unit = (u32x4*)(ring[st] + (2 + b) * kTile + vunit(d, h) * 16);
      u32x4 v = *unit;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k2 = keep - 2 * e;   // tokens kept in this dword
        v[e] &= k2 >= 2 ? 0xffffffffu : k2 == 1 ? 0x0000ffffu : 0u;
      }
      *unit = v;
    }
  };

  // ---- operands from LDS ----
  // key row of A for this lane: token sigma(col) of block col / 16
  const int kt = col & 15;
  const int ktok = (kt & 3) | ((kt & 4) << 1) | ((kt & 8) >> 1);
  const int koff = (col >> 4) * kTile + (g * kBS + ktok) * 16;
  auto qk_scores = [&](int st) {   // S^T = K Q^T over the 8 dim slices
    const uint8_t* kp = ring[st] + koff;
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      const u32x4 k = *(const u32x4*)(kp + sl * 2 * kBS * 16);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(k), as_bf16x8(qv[sl]), sc, 0, 0, 0);
    }
    return sc;
  };

  // m_run: the row's reference max in log2 units (qk * score); l_run: this
  // lane's part of the row sum (the other half of the row's tokens sits in
  // lane ^ 32)
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[m][r] = 0.f;
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);

  // Pipeline: pairs up to jp + kAhead stream into LDS while pair jp + 1's
  // QK^T runs on the matrix cores and pair jp's softmax and PV on the
  // vector ALUs and matrix cores.  One barrier per pair: before it, every
  // wave waits until its own quarter of pair jp + 1 has landed (later pairs'
  // loads may stay in flight: loads complete in order, 4 per pair), so after
  // it pair jp + 1 is in LDS and every wave is done with pair jp - 1's
  // stage, which pair jp + kAhead then overwrites.
  constexpr int kAhead = kStages - 1;
  static_assert(kAhead >= 2 && 4 * (kAhead - 2) <= 15, "stage count");
  // s_waitcnt: vector loads <= 4 (kAhead - 2), LDS and scalar loads done
  constexpr int kTopWait = 4 * (kAhead - 2) | (7 << 4);
  f32x16 sc = {};
  if (npairs > 0) {
#pragma unroll
    for (int i = 0; i < kAhead; ++i)
      if (i < npairs) stage_pair(i, i);
    __builtin_amdgcn_s_waitcnt(0);   // all loads, query rows included
    __syncthreads();
    if (npairs == 1) zero_value_tail(0, 0);   // published by the loop's first barrier
    if (active) sc = qk_scores(0);
  }
  for (int jp = 0; jp < npairs; ++jp) {
    const int t0 = 32 * jp;   // first token of the pair
    const int st = jp % kStages;
    __builtin_amdgcn_s_waitcnt(kTopWait);   // this wave's quarter of pair jp + 1
    __syncthreads();
    if (jp + kAhead < npairs) stage_pair(jp + kAhead, (jp + kAhead) % kStages);
    // pair jp + 1 is in LDS (its keys are read below, its values next
    // iteration, after the next barrier)
    if (jp + 2 == npairs) zero_value_tail((jp + 1) % kStages, jp + 1);
    if (!active) continue;

    // ---- tokens after the row's position are hidden (diagonal pairs only) ----
    // register 8b + i holds token t0 + 16b + 8g + i
    if (t0 + 31 > p_min) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = t0 + 16 * (r >> 3) + 8 * g + (r & 7);
        sc[r] = tok <= p ? sc[r] : -INFINITY;
      }
    }
    // A reference max that moves only when a score exceeds it by 2^8 (rare,
    // wave-uniform rescale): every p stays <= 2^8, and O / l does not depend
    // on the reference.
    float tm = fmaxf(__builtin_fmaxf(sc[0], sc[1]), sc[2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) tm = fmaxf(fmaxf(tm, sc[r]), sc[r + 1]);
    tm = fmaxf(tm, sc[15]) * qk;
    if (__ballot(tm > m_run + 8.0f)) {
      tm = fmaxf(tm, __shfl_xor(tm, 32));   // the row's other 16 tokens
      const bool up = tm > m_run + 8.0f;
      const float c = up ? __builtin_amdgcn_exp2f(m_run - tm) : 1.0f;
      m_run = up ? tm : m_run;
      l_run *= c;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][r] *= c;
    }
    // P^T as the B operand: bf16 of exp2(qk s - m), eight tokens per block;
    // the row sum adds the same bf16 values.  In the same block, the next
    // pair's scores (its stage is in LDS: the barrier above covers pair
    // jp + 1; after the last pair the stage holds stale bytes whose scores
    // are never used): each link of that dependent chain of 8 matrix-core
    // products is followed by a share of the exponentials, so the vector ALU
    // works while the matrix core does instead of after it.
    u32x4 pb[2];
    // this block and the products below feed the matrix core: the wave asks
    // for issue priority over the other waves of its SIMD until it is done
    __builtin_amdgcn_s_setprio(1);
    f32x16 sn;
    {
      const uint8_t* kp = ring[(jp + 1) % kStages] + koff;
#pragma unroll
      for (int r = 0; r < 16; ++r) sn[r] = 0.f;
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) {
        const u32x4 k = *(const u32x4*)(kp + sl * 2 * kBS * 16);
        sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(k), as_bf16x8(qv[sl]), sn, 0, 0, 0);
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        uint32_t w4[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const f32x2 e = {__builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * b + 2 * k], qk, -m_run)),
                           __builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * b + 2 * k + 1], qk, -m_run))};
          const bf16x2 pk = __builtin_convertvector(e, bf16x2);
          l_run = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, l_run, false);
          w4[k] = __builtin_bit_cast(uint32_t, pk);
        }
        pb[b] = u32x4{w4[0], w4[1], w4[2], w4[3]};
      }
      // schedule: two key reads ahead, each product followed by 5 vector
      // ops and the next key read
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        if (i < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }

    // ---- O^T += V^T P^T, block by block, value rows from LDS ----
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const uint8_t* vt = ring[st] + (2 + b) * kTile;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const u32x4 vr = *(const u32x4*)(vt + vunit(32 * m + col, g) * 16);
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vr), as_bf16x8(pb[b]), acc[m],
                                                         0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    sc = sn;
  }

  // ---- out = O / l, rows of this lane: dims 32m + 8q + 4g + (0..3) ----
  if (!active || !row_ok) return;
  const float lt = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / lt;
  uint16_t* orow = (uint16_t*)a.out + ((size_t)(r0q + pl) * a.Hq + qh) * kD;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = bad ? NAN : acc[m][4 * q + e] * inv;
      *(uint2*)(orow + 32 * m + 8 * q + 4 * g) =
          make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
  }
}

}  // namespace

bool prefill_supported(pkv_dtype q, pkv_dtype kv, int D, int BS) {
  return q == PKV_BF16 && kv == PKV_BF16 && D == kD && BS == kBS;
}

int prefill_query_blocks(int max_query_len, int G) {
  const long long rows = (long long)max_query_len * G;
  return (int)((rows + kNW * kRows - 1) / (kNW * kRows));
}

int launch_prefill(const PrefillArgs& a, void* stream) {
  if (a.total_wg <= 0) return 0;
  const int nunits = a.total_wg / a.qblocks;
  const int per = (nunits + 7) / 8 * a.qblocks;   // workgroups per XCD
  dim3 grid(8 * per), block(kNW * 64);
  hipLaunchKernelGGL(prefill_kernel, grid, block, 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // namespace pkv
