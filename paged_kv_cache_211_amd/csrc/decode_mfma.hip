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

template <int NW, int NBUF, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void decode_mfma_fp8_kernel(const DecodeArgs a) {
  constexpr int D = 128, BS = 32, HPW = 8;
  constexpr int TILE = BS * D;          // bytes of an fp8 (block, kv head) tile
  constexpr int NLOAD = TILE / 1024;    // 4 loads of 16 bytes per lane

  __shared__ uint16_t p_lds[NW][HPW][BS];
  __shared__ float o_lds[NW][HPW][D];
  __shared__ float m_lds[NW][HPW];
  __shared__ float l_lds[NW][HPW];
  __shared__ int bad_lds[NW];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, g = lane >> 5;
  const Work wk = locate<SPLIT, BS>(a, HPW, lane);
  const int t1 = wk.t1;
  bool bad = wk.bad;
  const int32_t* __restrict__ tbl = a.tables + (size_t)wk.s * a.max_blocks;
  const size_t head_off = (size_t)wk.hkv * TILE;
  const size_t blk_stride = (size_t)a.Hkv * TILE;

  // Q as the A operand of QK^T: row = head col (rows >= 8 are zero), k slots
  // 8g .. 8g+7 <-> dims 16*(2*l + g) + 8*h + (0..7) for key load l, half h.
  bf16x8 qa[NLOAD][2];
  {
    const bool valid = col < HPW;
    const uint16_t* qrow = (const uint16_t*)a.q + ((size_t)wk.s * a.Hq + wk.qh0 + (valid ? col : 0)) * D;
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
    const int tile_t0 = j * BS;
    const bool valid = tile_t0 + col < t1;
    float cfac[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float z = valid ? sc[r] * a.qk_mult : -INFINITY;
      const float mnew = fmaxf(m_run[r], max_xor16(row16_max(z)));
      cfac[r] = __builtin_amdgcn_exp2f(m_run[r] - mnew);
      const uint16_t pb = cvt_bf16(__builtin_amdgcn_exp2f(z - mnew));
      m_run[r] = mnew;
      l_run[r] = l_run[r] * cfac[r] + bf16_to_f32(pb);
      p_lds[w][4 * g + r][col] = pb;
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int m = 0; m < NLOAD; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[m][r] *= cfac[r];
    // P as the A operand of PV: row = head col, k slots 8g .. 8g+7 <->
    // tokens 16g + 8*half + (0..7).
    bf16x8 pa[2];
    {
      u32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
      if (col < HPW) {
        const u32x4* src = (const u32x4*)&p_lds[w][col][16 * g];
        lo = src[0];
        hi = src[1];
      }
      pa[0] = __builtin_bit_cast(bf16x8, lo);
      pa[1] = __builtin_bit_cast(bf16x8, hi);
    }
    // ---- O[head][dim] += P V; value load m holds dims 32m + col ----
    const int nvalid = t1 - tile_t0;
    const bool tail = nvalid < BS;
#pragma unroll
    for (int m = 0; m < NLOAD; ++m) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 vb = fp8x8_to_bf16(h ? vr[m].z : vr[m].x, h ? vr[m].w : vr[m].y);
        if (tail) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (16 * g + 8 * h + e >= nvalid) vb[e] = (__bf16)0.f;
        }
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[h], vb, acc[m], 0, 0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  tile_loop<NBUF, NLOAD, NW>(tbl, wk.t0 / BS + w, wk.jend, a.nb,
                             (const uint8_t*)a.kc + head_off + lane * 16,
                             (const uint8_t*)a.vc + head_off + col * 32 + g * 16, blk_stride,
                             lane, bad, process);

  // ---- per-wave totals: l over the 32 tokens of each half, o from the MFMA rows ----
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float lt = sum_xor16(row16_sum(l_run[r]));
#pragma unroll
    for (int m = 0; m < NLOAD; ++m) o_lds[w][4 * g + r][32 * m + col] = acc[m][r];
    if (col == 0) {
      m_lds[w][4 * g + r] = m_run[r];
      l_lds[w][4 * g + r] = lt;
    }
  }
  if (lane == 0) bad_lds[w] = bad ? 1 : 0;
  __syncthreads();
  merge_store<HPW, D, NW, false>(a, wk, !SPLIT || wk.nparts == 1, o_lds, m_lds, l_lds, bad_lds);
}

}  // namespace

bool decode_mfma_eligible(const DecodeArgs& a) {
  return a.kv_dtype == PKV_FP8_E4M3 && a.q_dtype == PKV_BF16 && a.D == 128 && a.BS == 32 &&
         (a.Hq / a.Hkv) % 8 == 0;
}

int launch_decode_mfma(const DecodeArgs& a, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int groups = a.Hq / a.Hkv / 8;
  dim3 block(kWaves * 64);
  if (a.partition > 0) {
    hipLaunchKernelGGL((decode_mfma_fp8_kernel<kWaves, kBufs, true>), dim3(a.total_parts, a.Hkv * groups),
                       block, 0, st, a);
  } else {
    hipLaunchKernelGGL((decode_mfma_fp8_kernel<kWaves, kBufs, false>), dim3(a.S, a.Hkv * groups),
                       block, 0, st, a);
  }
  return (int)hipGetLastError();
}

}  // namespace pkv
