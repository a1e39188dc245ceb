// Shared-prefix decode: the blocks that a group of sequences shares at the
// start of their tables are read once for the whole group.
//
// "Day 6/90 of Inference Engineering" (PagedAttention notes): prompts that
// begin alike share their prefix blocks by reference and continue in blocks
// of their own.  Decode still attends over every token of every sequence, so
// a plain decode reads each shared block once per sequence.  Here the
// shared blocks of a group are instead read by waves that each carry 32
// query rows -- (member sequence, query head) pairs of one kv head -- so a
// block is read once per 32 rows: QK^T is Q[32 x 128] K^T[128 x 32 tokens]
// and PV is P[32 x 32] V[32 x 128] on v_mfma_f32_32x32x16_bf16, two 16-token
// bf16 blocks per step ("PagedAttention Kernel：大模型推理优化的显存管理革新"
// §3.1: QK^T per block, softmax, PV; fp32 accumulation per §6).  Each wave
// leaves one partial (m, l, unnormalised o) per row for its 8 blocks; the
// sequences' own tokens (from the end of the prefix) are decoded by one wave
// per (sequence, kv head, split-K partition) with the vector-ALU per-tile
// code, and the split-K reduce combines both.
//
// Lane layouts of the 32x32x16 bf16 MFMA (lane l, col = l % 32, g = l / 32):
//   A[i][k]: lane holds row i = col, k = 8g .. 8g+7
//   B[k][j]: lane holds column j = col, k = 8g .. 8g+7
//   C[i][j]: register r holds row 8(r/4) + 4g + r%4, column col
// QK^T slice sl (dims 16sl .. 16sl+15): A = Q rows, k slot 8g + i <-> dim
//   16sl + 8g + i; B = K^T, column col = token col of the block pair, whose
//   16-byte key unit (chunk 2sl + g, token col % 16 of block col / 16) holds
//   exactly those 8 dims.
// PV for block b of the pair: A = P rows, k slot 8g + i <-> token 8g + i of
//   block b; B = V, column col = dim 32m + col, whose value row holds tokens
//   8g .. 8g+7 in 16 contiguous bytes.

#include <hip/hip_runtime.h>

#include "decode_common.h"
#include "decode_valu.h"

namespace pkv {
namespace {

using namespace dec;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPD = 128, kPBS = 16;        // head dim, block size
constexpr int kPTile = kPBS * kPD * 2;     // bytes of a bf16 (block, kv head) tile
constexpr int kRows = 32;                  // query rows per wave

// Work item (one wave): group g, kv head hkv, row block rb, prefix piece pp
// (blocks 8pp .. 8pp+7 of the group's prefix); flat index
// pre_off[g] + ((hkv * npre + pp) * RB + rb), so the row blocks of one piece
// are neighbours (one workgroup reads each block for up to 128 rows).
template <int NW>
__device__ __forceinline__ void prefix_body(const DecodeArgs& a, const PrefixArgs& p, int bid) {
  constexpr int D = kPD, BS = kPBS, TILE = kPTile;
  __shared__ __align__(16) uint16_t p_lds[NW][kRows][2 * BS];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, g = lane >> 5;
  const int item = bid * NW + w;
  if (item >= p.total_items) return;

  // ---- locate: group, then (kv head, piece, row block) ----
  const int grp = __builtin_amdgcn_readfirstlane(find_seq(p.pre_off, p.n_groups, item, lane));
  const int s0 = p.group_off[grp], members = p.group_off[grp + 1] - s0;
  const int G = a.Hq / a.Hkv;
  int pblocks = p.group_blocks[grp];
  // decode step: a member whose new token (position L - 1) lies in the
  // group's shared blocks would be stored into blocks this pass reads
  const long long shared_tokens = (long long)pblocks * BS;
  bool bad = false;
  if (pblocks > a.max_blocks) { pblocks = a.max_blocks; bad = true; }   // beyond the table
  const int npre = (pblocks + kPrefixPieceBlocks - 1) / kPrefixPieceBlocks;
  const int RB = (members * G + kRows - 1) / kRows;
  int local = item - p.pre_off[grp];
  const int rb = local % RB;
  local /= RB;
  const int pp = local % npre;
  const int hkv = local / npre;
  const int jfirst = pp * kPrefixPieceBlocks;
  const int jend = min(pblocks, jfirst + kPrefixPieceBlocks);
  // the group's prefix blocks, from its first member's table
  const int32_t* __restrict__ tbl = a.tables + (size_t)s0 * a.max_blocks;

  // ---- this lane's query row (A operand of QK^T) ----
  const int row = rb * kRows + col;
  const bool row_ok = row < members * G;
  const int rs = s0 + (row_ok ? row / G : 0);           // member sequence
  const int rqh = hkv * G + (row_ok ? row % G : 0);      // its query head
  bf16x8 qa[8];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + ((size_t)rs * a.Hq + rqh) * D;
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      const u32x4 v = row_ok ? *(const u32x4*)(qrow + 16 * sl + 8 * g) : u32x4{0, 0, 0, 0};
      qa[sl] = __builtin_bit_cast(bf16x8, v);
    }
  }

  float m_run[16], l_run[16];
  f32x16 acc[4];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
  }
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[m][r] = 0.f;

  const size_t head_off = (size_t)hkv * TILE;
  const size_t blk_stride = (size_t)a.Hkv * TILE;
  // the piece's block ids, all loaded up front
  int blk[kPrefixPieceBlocks];
#pragma unroll
  for (int i = 0; i < kPrefixPieceBlocks; ++i) blk[i] = jfirst + i < jend ? tbl[jfirst + i] : 0;
  auto block_base = [&](int i) -> size_t {   // i: block of the piece
    int b = blk[i];
    if ((unsigned)b >= (unsigned)a.nb) { bad = true; b = 0; }
    return (size_t)b * blk_stride + head_off;
  };
  // partial-row base of each member sequence this wave's rows touch: lane l
  // holds member mfirst + l's first prefix row (its suffix rows come first)
  const int mfirst = rb * kRows / G;
  int prow_l = 0;
  {
    const int m = mfirst + lane;
    if (m < members && lane <= kRows) {
      const int s = s0 + m;
      prow_l = p.row_off[s] + (p.suf_off[s + 1] - p.suf_off[s]);
    }
  }

#pragma unroll
  for (int i = 0; i < kPrefixPieceBlocks; i += 2) {
    const int j = jfirst + i;
    if (j >= jend) break;
    const bool two = j + 1 < jend;
    const size_t base0 = block_base(i);
    const size_t base1 = two ? block_base(i + 1) : base0;
    const size_t kb = (col < 16 ? base0 : base1);
    // ---- loads: 8 key units (one per dim slice), 4 value rows per block ----
    // Plain (cached) loads: every row block of the group re-reads these
    // blocks, so they should stay in the L2; the non-temporal policy of the
    // streamed suffix tiles would mark them for early eviction.
    u32x4 kr[8], vr[2][4];
    // key unit (chunk 2sl + g, token col % 16) at ((2sl + g) * BS + token) * 16
    const uint8_t* kp = (const uint8_t*)a.kc + kb + (size_t)(g * BS + (col & 15)) * 16;
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) kr[sl] = *(const u32x4*)(kp + (size_t)sl * 2 * BS * 16);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const uint8_t* vp = (const uint8_t*)a.vc + (b == 0 ? base0 : base1) + col * (BS * 2) + g * 16;
#pragma unroll
      for (int m = 0; m < 4; ++m) vr[b][m] = *(const u32x4*)(vp + (size_t)m * 32 * BS * 2);
    }

    // ---- scores S[row][token] for the 32 tokens of the pair ----
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
    for (int sl = 0; sl < 8; ++sl)
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[sl], __builtin_bit_cast(bf16x8, kr[sl]), sc, 0, 0, 0);

    // ---- online softmax per row (register r: row 8(r/4) + 4g + r%4) ----
    // A reference max that moves only when a tile's max exceeds it by 2^8
    // (rare, wave-uniform rescale): p <= 2^8 stays in range, and O / l does
    // not depend on the reference.
    const bool valid = two || col < 16;
    float z[16];
    bool grow = false;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      z[r] = valid ? sc[r] * a.qk_mult : -INFINITY;
      const float tmax = max_xor16(row16_max(z[r]));
      grow |= tmax > m_run[r] + 8.0f;
      sc[r] = tmax;   // reuse: the pair's row max
    }
    if (__ballot(grow)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool up = sc[r] > m_run[r] + 8.0f;
        const float c = up ? __builtin_amdgcn_exp2f(m_run[r] - sc[r]) : 1.0f;
        m_run[r] = up ? sc[r] : m_run[r];
        l_run[r] *= c;
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[m][r] *= c;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint16_t pb = cvt_bf16(__builtin_amdgcn_exp2f(z[r] - m_run[r]));
      l_run[r] += bf16_to_f32(pb);
      p_lds[w][8 * (r / 4) + 4 * g + (r % 4)][col] = pb;
    }
    __builtin_amdgcn_wave_barrier();

    // ---- O[row][dim] += P V, block by block (16 tokens = one k step) ----
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if (b == 1 && !two) break;
      const bf16x8 pa = __builtin_bit_cast(bf16x8, *(const u32x4*)&p_lds[w][col][16 * b + 8 * g]);
#pragma unroll
      for (int m = 0; m < 4; ++m)
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, __builtin_bit_cast(bf16x8, vr[b][m]),
                                                         acc[m], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- partials: row (member, head) -> its sequence's prefix row pp ----
  float* ws_o = a.ws;
  float* ws_ml = a.ws + (size_t)p.total_rows * a.Hq * D;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rr = rb * kRows + 8 * (r / 4) + 4 * g + (r % 4);
    const float lt = sum_xor16(row16_sum(l_run[r]));
    const int base = __shfl(prow_l, rr / G - mfirst);
    if (rr < members * G) {
      const bool nan_row = bad || (p.step && a.lens[s0 + rr / G] <= shared_tokens);
      const int qh = hkv * G + rr % G;
      const size_t pi = (size_t)(base + pp) * a.Hq + qh;
      float* o = ws_o + pi * D + col;
#pragma unroll
      for (int m = 0; m < 4; ++m) o[32 * m] = nan_row ? NAN : acc[m][r];
      if (col == 0) {
        ws_ml[pi * 2] = m_run[r];
        ws_ml[pi * 2 + 1] = nan_row ? NAN : lt;
      }
    }
  }
}

template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_prefix_kernel(const DecodeArgs a, PrefixArgs p) {
  prefix_body<NW>(a, p, blockIdx.x);
}

// The suffix pass with one wave per item: item x of the split-K schedule over
// the sequences' own tokens (head group x % nhg, launch slot x / nhg, as in
// decode_body), walked by this wave alone, its partial written to the row
// the shared-prefix plan gives (row_off[s] + part).  The suffixes are short
// (tens of blocks), so a wave that takes all of an item's tiles pays the
// item's start (query, table, first tiles) once instead of four times and
// needs no merge through LDS.  STORE (decode step, one wave per (sequence,
// kv head, partition)): the wave whose partition ends at the context's end
// reads the block of the new token, so it stores the token first, as the
// split-K decode step does (from tile_loop's start hook, waiting for the
// store only before loading that block).
template <int HPW, bool STORE>
__device__ __forceinline__ void suffix_wave(const DecodeArgs& b, int x, int lane,
                                            float (*p_w)[kPBS], u32x4* q_w) {
  using St = valu::ValuHeads<PKV_BF16, kPD, kPBS, HPW, kQLds>;
  constexpr int NLOAD = St::NLOAD, RU = St::RU, DPI = St::DPI, TILE = kPTile, D = kPD;
  const int nhg = b.Hkv * (b.Hq / b.Hkv / HPW);
  if (x >= b.total_parts * nhg) return;
  const Work wk = locate<true, kPBS>(b, HPW, lane, x / nhg, x % nhg);
  bool bad = wk.bad;
  const int32_t* __restrict__ tbl = b.tables + (size_t)wk.s * b.max_blocks;
  const size_t head_off = (size_t)wk.hkv * TILE;
  St st;
  if constexpr (kQLds) {
    St::fill_q(b, wk.s, wk.qh0, q_w, lane, 64);
    __builtin_amdgcn_wave_barrier();
    st.qs = q_w;
  } else {
    st.load_q(b, wk.s, wk.qh0, lane);
  }
  st.reset();
  const int t1 = wk.t1;
  const bool my_store = STORE && !wk.bad && wk.L > 0 && wk.t0 < wk.L && wk.t1 == wk.L;
  tile_loop<kBufs, NLOAD, 1>(tbl, wk.t0 / kPBS, wk.jend, b.nb,
                             (const uint8_t*)b.kc + head_off + lane * 16,
                             (const uint8_t*)b.vc + head_off + lane * 16, (size_t)b.Hkv * TILE,
                             lane, bad, [&](int j, const u32x4* kr, const u32x4* vr) {
                               st.tile(b.qk_mult, j, t1, kr, vr, p_w, lane);
                             },
                             my_store ? wk.jend - 1 : -1, [&] {
                               if constexpr (STORE) {
                                 if (my_store)
                                   store_new_token<PKV_BF16, kPD, kPBS>(b, wk.s, wk.hkv, wk.L, lane);
                               }
                             });
  float* ws_o = b.ws;
  float* ws_ml = b.ws + (size_t)b.ws_rows * b.Hq * D;
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const float lt = valu::tile_sum<kPBS>(st.l_run[hh]);
    const size_t pi = (size_t)wk.item * b.Hq + wk.qh0 + hh;
#pragma unroll
    for (int l = 0; l < NLOAD; ++l) {
      const float v = st.dim_sum(hh, l);
      if (lane % RU == 0) ws_o[pi * D + l * DPI + lane / RU] = bad ? NAN : v * b.v_mult;
    }
    if (lane == 0) {
      ws_ml[pi * 2] = st.m_run[hh];
      ws_ml[pi * 2 + 1] = bad ? NAN : lt;
    }
  }
}

// Both passes in one launch: workgroups [0, npre) run the prefix pass (args
// a), the rest the suffix pass over each sequence's own tokens (args b), one
// wave per item.
// Both are bound by memory latency, not bandwidth, so side by side on the
// same compute units they hide each other's waits; npre is a multiple of 8,
// so the regrouping of the prefix items by XCD below is a permutation of
// [0, npre) and the split-K workgroups keep their XCD order.  STORE: the
// decode step's store in the suffix waves.
template <int HPW, bool STORE>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_prefix_fused_kernel(const DecodeArgs a, const DecodeArgs b, PrefixArgs p, int npre) {
  if ((int)blockIdx.x < npre) {
    // Workgroup ids go round robin over the 8 XCDs: XCD x runs the
    // contiguous eighth x of the prefix items, so the workgroups that read
    // one piece (consecutive items) share that XCD's L2.
    const int bx = (int)blockIdx.x;
    prefix_body<kWaves>(a, p, (bx % 8) * (npre / 8) + bx / 8);
  } else {
    __shared__ float p_lds[kWaves][HPW][kPBS];
    __shared__ u32x4 q_lds[kQLds ? kWaves : 1][kQLds ? HPW * kPD * 2 / 16 : 1];
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // the suffix waves' streams end the launch (the longest suffixes run
    // last), so their instructions go first when a prefix wave on the same
    // SIMD is ready too
    __builtin_amdgcn_s_setprio(1);
    suffix_wave<HPW, STORE>(b, ((int)blockIdx.x - npre) * kWaves + w, threadIdx.x & 63, p_lds[w],
                     q_lds[kQLds ? w : 0]);
  }
}

}  // namespace

int launch_decode_prefix_fused(const DecodeArgs& a, const DecodeArgs& b, const PrefixArgs& p,
                               void* stream, bool store) {
  const int npre = ((p.total_items + kWaves - 1) / kWaves + 7) / 8 * 8;
  return valu::with_hpw<PKV_BF16, kPD, kPBS>(a.Hq / a.Hkv, [&](auto h) {
    constexpr int HPW = decltype(h)::value;
    const int groups = b.Hq / b.Hkv / HPW;
    const long long items = (long long)b.total_parts * b.Hkv * groups;   // one wave each
    if (store && groups != 1) return (int)hipErrorInvalidValue;
    dim3 block(kWaves * 64), grid(npre + (unsigned)((items + kWaves - 1) / kWaves));
    if (store)
      hipLaunchKernelGGL((decode_prefix_fused_kernel<HPW, true>), grid, block, 0,
                         (hipStream_t)stream, a, b, p, npre);
    else
      hipLaunchKernelGGL((decode_prefix_fused_kernel<HPW, false>), grid, block, 0,
                         (hipStream_t)stream, a, b, p, npre);
    return (int)hipGetLastError();
  });
}

bool decode_prefix_supported(const DecodeArgs& a) {
  return a.q_dtype == PKV_BF16 && a.kv_dtype == PKV_BF16 && a.D == kPD && a.BS == kPBS;
}

bool decode_prefix_step_in_kernel(const DecodeArgs& a) {
  const int G = a.Hq / a.Hkv;
  return decode_prefix_supported(a) && valu::heads_per_wg<PKV_BF16, kPD, kPBS>(G) == G;
}

int launch_decode_prefix(const DecodeArgs& a, const PrefixArgs& p, void* stream) {
  if (p.total_items <= 0) return 0;
  dim3 block(kWaves * 64), grid((p.total_items + kWaves - 1) / kWaves);
  hipLaunchKernelGGL((decode_prefix_kernel<kWaves>), grid, block, 0, (hipStream_t)stream, a, p);
  return (int)hipGetLastError();
}

}  // namespace pkv
