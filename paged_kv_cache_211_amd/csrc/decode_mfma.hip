// PagedAttention decode with matrix cores, for fp8 (E4M3FN) key/value tiles
// of 32 tokens x 128 dims and 8 query heads per kv head.
//
// With 8 query heads sharing one kv head, QK^T of a block is the dense
// product Q[8 x 128] K^T[128 x 32] and PV is P[8 x 32] V[32 x 128]; on VALU
// the 8 heads' query vectors do not fit a lane's registers, so the tile would
// be read once per head pair.  Here both products run on
// v_mfma_f32_32x32x16_bf16 (fp8 codes convert exactly to bf16), with the 8
// heads in the A operand's rows, so every tile is read from HBM once
// ("PagedAttention Kernel：大模型推理优化的显存管理革新" §3.1: QK^T per block,
// softmax, PV accumulated block by block; fp32 accumulation per §6).
//
// Lane layouts of the 32x32x16 bf16 MFMA (lane l, col = l % 32, g = l / 32):
//   A[i][k]: lane holds row i = col, k = 8g .. 8g+7
//   B[k][j]: lane holds column j = col, k = 8g .. 8g+7
//   C[i][j]: register r holds row 8(r/4) + 4g + r%4, column col
// QK^T: A = Q (rows = heads), B = K^T (columns = the 32 tokens).  The plain
//   16-byte key load already matches: lane l holds token col's 16 dims of
//   key chunk 2*load + g; its low and high 8 bytes feed two MFMAs.
// PV: A = P (rows = heads, k = tokens), B = V (columns = 32 dims).  Each
//   1 KiB value load is permuted across lanes (still one contiguous KiB) so
//   lane l holds dim 32*load + col, tokens 16g .. 16g+15.
// The k index pairs with the same dims (QK) or tokens (PV) in A and B, so the
// assignment of dims/tokens to k slots is free and chosen to match the loads.
// Score and output rows r = 0..3 of lane l are head 4g + r; rows 8..31 are
// padding (zero query rows).
// Work: one wave per (sequence, split-K partition, kv head), or per piece of
// a stream-K slice; the wave keeps its own softmax state and writes its
// output or partial directly, so no workgroup-wide merge or barrier is needed.

#include <hip/hip_runtime.h>

#include "decode_common.h"

namespace pkv {
namespace {

using namespace dec;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Eight E4M3FN codes (two words, byte order) -> eight bf16, exact.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

constexpr int kD = 128, kBS = 32, kHPW = 8;
constexpr int kTile = kBS * kD;         // bytes of an fp8 (block, kv head) tile
constexpr int kNLoad = kTile / 1024;    // 4 loads of 16 bytes per lane

// One wave's work on tiles [jfirst, jend) of sequence s (tokens end at t1)
// for the 8 query heads qh0 .. qh0+7 of kv head hkv: QK^T and PV on matrix
// cores, online softmax, then the output rows (final_out) or the partial
// rows prow0 + h (h = 0..7) of ws_o / ws_ml.  prow: this wave's LDS rows.
__device__ __forceinline__ void mfma_item(const DecodeArgs& a, int s, int hkv, int qh0, int jfirst,
                                          int jend, int t1, bool bad, bool final_out, size_t prow0,
                                          float* ws_o, float* ws_ml, uint16_t (*prow)[kBS],
                                          int lane, bool store_new = false, int L = 0) {
  constexpr int D = kD, BS = kBS, HPW = kHPW, TILE = kTile, NLOAD = kNLoad;
  constexpr int NBUF = kMfmaBufs;
  const int col = lane & 31, g = lane >> 5;
  const int32_t* __restrict__ tbl = a.tables + (size_t)s * a.max_blocks;
  const size_t head_off = (size_t)hkv * TILE;
  const size_t blk_stride = (size_t)a.Hkv * TILE;

  // Q as the A operand of QK^T: row = head col (rows >= 8 are zero), k slots
  // 8g .. 8g+7 <-> dims 16*(2*l + g) + 8*h + (0..7) for key load l, half h.
  bf16x8 qa[NLOAD][2];
  {
    const bool valid = col < HPW;
    const uint16_t* qrow = (const uint16_t*)a.q + ((size_t)s * a.Hq + qh0 + (valid ? col : 0)) * D;
#pragma unroll
    for (int l = 0; l < NLOAD; ++l)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 v = valid ? *(const u32x4*)(qrow + 16 * (2 * l + g) + 8 * h) : u32x4{0, 0, 0, 0};
        qa[l][h] = __builtin_bit_cast(bf16x8, v);
      }
  }

  float m_run[4], l_run[4];
  f32x16 acc[NLOAD];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
  }
#pragma unroll
  for (int m = 0; m < NLOAD; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[m][r] = 0.f;

  auto process = [&](int j, const u32x4* kr, const u32x4* vr) {
    // ---- scores S[head][token] = Q K^T for the 32 tokens of the tile ----
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
    for (int l = 0; l < NLOAD; ++l) {
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[l][0], fp8x8_to_bf16(kr[l].x, kr[l].y), sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[l][1], fp8x8_to_bf16(kr[l].z, kr[l].w), sc, 0, 0, 0);
    }
    // ---- online softmax, rows r = 0..3 (head 4g + r), column = token col ----
    // Probabilities are taken against a reference max m_run that moves only
    // when a tile's max exceeds it by more than 2^8 (then l and the
    // accumulator are rescaled, a rare, wave-uniform branch).  p <= 2^8 stays
    // exact in range for bf16 and fp32, and the result O / l does not depend
    // on the reference.
    const int tile_t0 = j * BS;
    const bool valid = tile_t0 + col < t1;
    float z[4], tmax[4];
    bool grow = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      z[r] = valid ? sc[r] * a.qk_mult : -INFINITY;
      tmax[r] = max_xor16(row16_max(z[r]));
      grow |= tmax[r] > m_run[r] + 8.0f;
    }
    if (__ballot(grow)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool up = tmax[r] > m_run[r] + 8.0f;
        const float c = up ? __builtin_amdgcn_exp2f(m_run[r] - tmax[r]) : 1.0f;
        m_run[r] = up ? tmax[r] : m_run[r];
        l_run[r] *= c;
#pragma unroll
        for (int m = 0; m < NLOAD; ++m) acc[m][r] *= c;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint16_t pb = cvt_bf16(__builtin_amdgcn_exp2f(z[r] - m_run[r]));
      l_run[r] += bf16_to_f32(pb);
      prow[4 * g + r][col] = pb;
    }
    __builtin_amdgcn_wave_barrier();
    // P as the A operand of PV: row = head col, k slots 8g .. 8g+7 <->
    // tokens 16g + 8*half + (0..7).
    bf16x8 pa[2];
    {
      u32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
      if (col < HPW) {
        const u32x4* src = (const u32x4*)&prow[col][16 * g];
        lo = src[0];
        hi = src[1];
      }
      pa[0] = __builtin_bit_cast(bf16x8, lo);
      pa[1] = __builtin_bit_cast(bf16x8, hi);
    }
    // ---- O[head][dim] += P V; value load m holds dims 32m + col ----
    // Value codes of tokens past the end of the range become 0 (+0.0) by a
    // byte mask on the fp8 words (the same tokens in every dim group), so
    // uninitialised slots never reach the accumulator (0 * NaN).
    const int nvalid = t1 - tile_t0;
    uint32_t vmask[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int keep = min(max(nvalid - (16 * g + 8 * h), 0), 8);  // bytes kept of these 8 tokens
      const uint64_t m64 = keep >= 8 ? ~0ull : ((1ull << (8 * keep)) - 1ull);
      vmask[h][0] = (uint32_t)m64;
      vmask[h][1] = (uint32_t)(m64 >> 32);
    }
#pragma unroll
    for (int m = 0; m < NLOAD; ++m) {
      acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          pa[0], fp8x8_to_bf16(vr[m].x & vmask[0][0], vr[m].y & vmask[0][1]), acc[m], 0, 0, 0);
      acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          pa[1], fp8x8_to_bf16(vr[m].z & vmask[1][0], vr[m].w & vmask[1][1]), acc[m], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  };

  tile_loop<NBUF, NLOAD, 1>(tbl, jfirst, jend, a.nb, (const uint8_t*)a.kc + head_off + lane * 16,
                            (const uint8_t*)a.vc + head_off + col * 32 + g * 16, blk_stride,
                            lane, bad, process, store_new ? jend - 1 : -1, [&] {
                              if (store_new) store_new_token<PKV_FP8_E4M3, D, BS>(a, s, hkv, L, lane);
                            });

  // ---- epilogue: rows r = 0..3 are head 4g + r; lane holds dims 32m + col ----
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float lt = sum_xor16(row16_sum(l_run[r]));
    const int hh = 4 * g + r;
    if (final_out) {
      const float inv = lt > 0.f ? a.v_mult / lt : 0.f;
      uint16_t* o = (uint16_t*)a.out + ((size_t)s * a.Hq + qh0 + hh) * D + col;
#pragma unroll
      for (int m = 0; m < NLOAD; ++m) o[32 * m] = f32_to_bf16(bad ? NAN : acc[m][r] * inv);
    } else {
      const size_t pi = prow0 + hh;
      float* o = ws_o + pi * D + col;
#pragma unroll
      for (int m = 0; m < NLOAD; ++m) o[32 * m] = bad ? NAN : acc[m][r] * a.v_mult;
      if (col == 0) {
        ws_ml[pi * 2] = m_run[r];
        ws_ml[pi * 2 + 1] = bad ? NAN : lt;
      }
    }
  }
}

// Split-K schedule: each wave owns one work item, (sequence, partition) for
// the kv head of blockIdx.y, flat item blockIdx.x * NW + wave; it writes its
// own output (one-partition sequence) or partial.  STORE (decode step, one
// group of 8 query heads per kv head): the wave that reads a sequence's last
// block first stores the sequence's new token; it is that block's only reader.
template <int NW, bool SPLIT, bool STORE = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_mfma_fp8_kernel(const DecodeArgs a) {
  constexpr int BS = kBS, HPW = kHPW, D = kD;
  __shared__ uint16_t p_lds[NW][HPW][BS];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // XCD-aware order (workgroup ids go round-robin to the 8 XCDs): the head
  // group is the id's low part, so with 8 head groups every XCD serves one
  // kv head.
  const int G = a.Hq / a.Hkv;
  const int nhg = a.Hkv * (G / HPW);
  const int hg = blockIdx.x % nhg;
  const int item = (blockIdx.x / nhg) * NW + w;
  const int n_items = SPLIT ? a.total_parts : a.S;
  if (item >= n_items) return;

  // ---- locate the work item ----
  const int hkv = hg / (G / HPW);
  const int qh0 = hkv * G + (hg % (G / HPW)) * HPW;
  int s, part, nparts, row;
  if constexpr (SPLIT) {
    split_slot<BS>(a, item, lane, s, part);
    const int p0 = a.part_off[s];
    row = p0 + part;
    nparts = a.part_off[s + 1] - p0;
  } else {
    s = item;
    part = 0;
    nparts = 1;
    row = item;
  }
  int L = a.lens[s];
  bool bad = false;
  if (L < 0) { L = 0; bad = true; }
  if (L > a.max_blocks * BS) { L = a.max_blocks * BS; bad = true; }
  if (SPLIT && nparts != split_parts(L, a.partition)) bad = true;   // stale offsets
  const int t0 = SPLIT ? part * a.partition : 0;
  const int t1 = SPLIT ? min(L, t0 + a.partition) : L;
  const int jend = (t1 + BS - 1) / BS;
  mfma_item(a, s, hkv, qh0, t0 / BS, jend, t1, bad, !SPLIT || nparts == 1,
            (size_t)row * a.Hq + qh0, a.ws, a.ws + (size_t)a.total_parts * a.Hq * D, p_lds[w],
            lane, STORE && !bad && L > 0 && t0 < L && t1 == L, L);
}

// Stream-K schedule (see the vector-ALU stream-K kernel): wave gw of
// R = a.sk_workers takes tiles [floor(gw*T/R), floor((gw+1)*T/R)) of the
// T = CU * H_kv * groups tiles laid out as (head group hg, sequence s, tile)
// and writes each piece as the output (whole item) or as the partial rows
// [slot][8] of slot gw + hg*S + s.
template <int NW, bool STORE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_mfma_sk_kernel(const DecodeArgs a) {
  constexpr int BS = kBS, HPW = kHPW, D = kD;
  __shared__ uint16_t p_lds[NW][HPW][BS];

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
  const size_t slots = (size_t)R + (size_t)a.Hkv * groups * a.S;
  float* ws_ml = a.ws + slots * HPW * D;

  while (x < x1) {
    const int hg = (int)(x / CU);
    const int rem = (int)(x - (int64_t)hg * CU);
    const int s = min(__builtin_amdgcn_readfirstlane(find_seq(a.tile_off, a.S, rem, lane)), a.S - 1);
    const int off = a.tile_off[s];
    const int n_s = a.tile_off[s + 1] - off;
    const int j0 = rem - off;
    const int jn = (int)min((int64_t)n_s, (int64_t)j0 + (x1 - x));
    if (j0 < 0 || jn <= j0) break;   // offsets are not running sums ending at sk_cu
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
    const size_t slot = (size_t)gw + (size_t)hg * a.S + s;
    mfma_item(a, s, hkv, qh0, jfirst, jend, L, bad, j0 == 0 && jn == n_s, slot * HPW, a.ws, ws_ml,
              p_lds[w], lane, STORE && !bad && L > 0 && jend == nt && jfirst < jend, L);
  }
}

}  // namespace

// PKV_DECODE_MFMA=0 (a measurement build only) leaves every shape to the
// vector-ALU kernels, for comparing the two on the same fp8 shape.
#ifndef PKV_DECODE_MFMA
#define PKV_DECODE_MFMA 1
#endif

bool decode_mfma_eligible(const DecodeArgs& a) {
  return PKV_DECODE_MFMA && a.kv_dtype == PKV_FP8_E4M3 && a.q_dtype == PKV_BF16 && a.D == 128 &&
         a.BS == 32 && (a.Hq / a.Hkv) % 8 == 0;
}

int launch_decode_mfma(const DecodeArgs& a, void* stream, bool store) {
  hipStream_t st = (hipStream_t)stream;
  const int groups = a.Hq / a.Hkv / 8;
  if (store && groups != 1) return (int)hipErrorInvalidValue;
  dim3 block(kWaves * 64);
  const int items = a.partition > 0 ? a.total_parts : a.S;
  dim3 grid((items + kWaves - 1) / kWaves * a.Hkv * groups);
  if (a.partition > 0) {
    if (store)
      hipLaunchKernelGGL((decode_mfma_fp8_kernel<kWaves, true, true>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((decode_mfma_fp8_kernel<kWaves, true>), grid, block, 0, st, a);
  } else {
    if (store)
      hipLaunchKernelGGL((decode_mfma_fp8_kernel<kWaves, false, true>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((decode_mfma_fp8_kernel<kWaves, false>), grid, block, 0, st, a);
  }
  return (int)hipGetLastError();
}

int launch_decode_mfma_sk(const DecodeArgs& a, void* stream, bool store) {
  hipStream_t st = (hipStream_t)stream;
  if (store && a.Hq / a.Hkv != 8) return (int)hipErrorInvalidValue;
  dim3 block(kSkWaves * 64), grid((a.sk_workers + kSkWaves - 1) / kSkWaves);
  if (store)
    hipLaunchKernelGGL((decode_mfma_sk_kernel<kSkWaves, true>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((decode_mfma_sk_kernel<kSkWaves, false>), grid, block, 0, st, a);
  return (int)hipGetLastError();
}

int decode_mfma_sk_workers() {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(&decode_mfma_sk_kernel<kSkWaves, false>),
          kSkWaves * 64, 0) != hipSuccess)
    return -1;
  return (per_cu > 1 ? per_cu : 1) * cus * kSkWaves;
}

}  // namespace pkv
