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
//
// Three schedules share that per-tile code (MfmaHeads):
//   * decode_mfma_fp8_kernel (split-K and one pass, the default): one wave
//     per item, dispatched by the hardware, whose workgroup dispatcher hands
//     the next workgroup to whichever CU slot frees first.
//   * decode_mfma_queue_kernel (paged_attention_decode_queue): persistent
//     waves, each taking (sequence, partition, kv head) items one after
//     another -- the first by its wave index, the rest from a work counter
//     -- and fetching the next item's table entries and query while the
//     current item's tiles stream, and its first tile as soon as the
//     current item's last tile is in registers ("PagedAttention Kernel…"
//     §3.2: an atomic work counter in a persistent loop balances uneven
//     work; §2.2: prefetch of the next page).  Items go in the longest-first
//     order of split_slot.  Measured slower than the default: a claim's
//     answer is a vector-memory return, and the wave's in-order memory
//     counter makes the next tile wait for it.
//   * decode_mfma_sk_kernel: stream-K slices.
// Every wave keeps its own softmax state and writes its output or partial
// directly, so no workgroup-wide merge or barrier is needed.

#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>

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
constexpr int kQBytes = kHPW * kD * 2;  // the 8 query rows of an item (bf16)
// split-K partitions shorter than this many tokens keep two tiles in flight
// per wave (the skewed fp8 workload at 512-token partitions: step 303 -> 299
// us; at 1536 one tile measures 1% faster)
constexpr int kDeepBelow = 1024;

// The 8 query heads of one kv head held by one wave: the query as MFMA A
// operands, the online-softmax state of rows r = 0..3 (head 4g + r) and the
// output accumulators (lane holds dims 32m + col of those rows).
struct MfmaHeads {
  bf16x8 qa[kNLoad][2];
  float m_run[4], l_run[4];
  f32x16 acc[kNLoad];

  // Q as the A operand of QK^T: row = head col (rows >= 8 are zero), k slots
  // 8g .. 8g+7 <-> dims 16*(2*l + g) + 8*h + (0..7) for key load l, half h.
  // `rows` points at the 8 query rows (8 x 128 bf16, global or LDS memory).
  __device__ __forceinline__ void set_q(const uint16_t* rows, int col, int g) {
    const bool valid = col < kHPW;
    const uint16_t* qrow = rows + (valid ? col : 0) * kD;
#pragma unroll
    for (int l = 0; l < kNLoad; ++l)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 v = valid ? *(const u32x4*)(qrow + 16 * (2 * l + g) + 8 * h) : u32x4{0, 0, 0, 0};
        qa[l][h] = __builtin_bit_cast(bf16x8, v);
      }
  }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      m_run[r] = -INFINITY;
      l_run[r] = 0.f;
    }
#pragma unroll
    for (int m = 0; m < kNLoad; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][r] = 0.f;
  }

  // Tile j (tokens j*32 ..) of a range whose tokens end at t1.
  __device__ __forceinline__ void tile(float qk_mult, int j, int t1, const u32x4* kr,
                                       const u32x4* vr, uint16_t (*prow)[kBS], int col, int g) {
    // ---- scores S[head][token] = Q K^T for the 32 tokens of the tile ----
    f32x16 sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
    for (int l = 0; l < kNLoad; ++l) {
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[l][0], fp8x8_to_bf16(kr[l].x, kr[l].y), sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[l][1], fp8x8_to_bf16(kr[l].z, kr[l].w), sc, 0, 0, 0);
    }
    // ---- online softmax, rows r = 0..3 (head 4g + r), column = token col ----
    // Probabilities are taken against a reference max m_run that moves only
    // when a tile's max exceeds it by more than 2^8 (then l and the
    // accumulator are rescaled, a rare, wave-uniform branch).  p <= 2^8 stays
    // exact in range for bf16 and fp32, and the result O / l does not depend
    // on the reference.
    const int tile_t0 = j * kBS;
    const bool valid = tile_t0 + col < t1;
    float z[4], tmax[4];
    bool grow = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      z[r] = valid ? sc[r] * qk_mult : -INFINITY;
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
        for (int m = 0; m < kNLoad; ++m) acc[m][r] *= c;
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
      if (col < kHPW) {
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
    for (int m = 0; m < kNLoad; ++m) {
      acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          pa[0], fp8x8_to_bf16(vr[m].x & vmask[0][0], vr[m].y & vmask[0][1]), acc[m], 0, 0, 0);
      acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          pa[1], fp8x8_to_bf16(vr[m].z & vmask[1][0], vr[m].w & vmask[1][1]), acc[m], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  }

  // Rows r = 0..3 are head 4g + r; lane holds dims 32m + col.  final_out:
  // the normalised output rows of sequence s; else the partial rows
  // prow0 + h (h = 0..7) of ws_o / ws_ml.
  __device__ __forceinline__ void finish(const DecodeArgs& a, int s, int qh0, bool bad,
                                         bool final_out, size_t prow0, float* ws_o, float* ws_ml,
                                         int col, int g) const {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float lt = sum_xor16(row16_sum(l_run[r]));
      const int hh = 4 * g + r;
      if (final_out) {
        const float inv = lt > 0.f ? a.v_mult / lt : 0.f;
        uint16_t* o = (uint16_t*)a.out + ((size_t)s * a.Hq + qh0 + hh) * kD + col;
#pragma unroll
        for (int m = 0; m < kNLoad; ++m) o[32 * m] = f32_to_bf16(bad ? NAN : acc[m][r] * inv);
      } else {
        const size_t pi = prow0 + hh;
        float* o = ws_o + pi * kD + col;
#pragma unroll
        for (int m = 0; m < kNLoad; ++m) o[32 * m] = bad ? NAN : acc[m][r] * a.v_mult;
        if (col == 0) {
          ws_ml[pi * 2] = m_run[r];
          ws_ml[pi * 2 + 1] = bad ? NAN : lt;
        }
      }
    }
  }
};

// One wave's work on tiles [jfirst, jend) of sequence s (tokens end at t1)
// for the 8 query heads qh0 .. qh0+7 of kv head hkv, then the output rows
// (final_out) or the partial rows prow0 + h (h = 0..7) of ws_o / ws_ml.
// prow: this wave's LDS rows.  store_new: first store the sequence's new
// token (decode step; the wave reads the block that receives it).  NBUF:
// tiles in flight per wave.
template <int NBUF = kMfmaBufs>
__device__ __forceinline__ void mfma_item(const DecodeArgs& a, int s, int hkv, int qh0, int jfirst,
                                          int jend, int t1, bool bad, bool final_out, size_t prow0,
                                          float* ws_o, float* ws_ml, uint16_t (*prow)[kBS],
                                          int lane, bool store_new = false, int L = 0) {
  const int col = lane & 31, g = lane >> 5;
  const int32_t* __restrict__ tbl = a.tables + (size_t)s * a.max_blocks;
  const size_t head_off = (size_t)hkv * kTile;
  const size_t blk_stride = (size_t)a.Hkv * kTile;
  MfmaHeads h;
  h.set_q((const uint16_t*)a.q + ((size_t)s * a.Hq + qh0) * kD, col, g);
  h.reset();
  tile_loop<NBUF, kNLoad, 1>(
      tbl, jfirst, jend, a.nb, (const uint8_t*)a.kc + head_off + lane * 16,
      (const uint8_t*)a.vc + head_off + col * 32 + g * 16, blk_stride, lane, bad,
      [&](int j, const u32x4* kr, const u32x4* vr) { h.tile(a.qk_mult, j, t1, kr, vr, prow, col, g); },
      store_new ? jend - 1 : -1, [&] {
        if (store_new) store_new_token<PKV_FP8_E4M3, kD, kBS>(a, s, hkv, L, lane);
      });
  h.finish(a, s, qh0, bad, final_out, prow0, ws_o, ws_ml, col, g);
}

// A split-K work item: partition `part` of sequence s, kv head hkv.
struct MItem {
  int s, hkv, qh0;
  int j0, jend;   // tiles [j0, jend)
  int t1, L;      // tokens end at t1; context length (clamped to the table)
  int row;        // partial row of the workspace (p0 + part)
  bool bad;       // length out of range or offsets stale: NaN output
  bool final_out; // the only partition of its sequence: write the output
  bool store;     // decode step: this item reads the block of the new token
};

// Item x of the split-K schedule: head group x % nhg, launch slot x / nhg
// mapped to (sequence, partition) longest first (split_slot).  off / lens:
// the partition offsets and lengths to read (device arrays or an LDS copy).
template <bool STORE>
__device__ __forceinline__ MItem split_item(const DecodeArgs& a, int x, int nhg, int lane,
                                            const int32_t* off, const int32_t* lens) {
  MItem it;
  const int G = a.Hq / a.Hkv, groups = G / kHPW;
  const int hg = x % nhg;
  int part;
  split_slot<kBS>(a, x / nhg, lane, it.s, part, off, lens);
  it.hkv = hg / groups;
  it.qh0 = it.hkv * G + (hg % groups) * kHPW;
  const int p0 = off[it.s];
  const int nparts = off[it.s + 1] - p0;
  it.row = p0 + part;
  int L = lens[it.s];
  it.bad = false;
  if (L < 0) { L = 0; it.bad = true; }
  if (L > a.max_blocks * kBS) { L = a.max_blocks * kBS; it.bad = true; }
  if (nparts != split_parts(L, a.partition)) it.bad = true;   // stale offsets
  it.L = L;
  const int t0 = part * a.partition;
  it.t1 = min(L, t0 + a.partition);
  it.j0 = t0 / kBS;
  it.jend = max((it.t1 + kBS - 1) / kBS, it.j0);
  it.final_out = nparts == 1;
  it.store = STORE && !it.bad && L > 0 && t0 < L && it.t1 == L;
  return it;
}

// Split-K schedule, one wave per item dispatched by the hardware: item
// (blockIdx.x / nhg) * NW + wave of head group blockIdx.x % nhg (the head
// group is the id's low part, so with 8 head groups every XCD serves one kv
// head).  One pass (SPLIT = false): item = sequence.  STORE (decode step,
// one group of 8 query heads per kv head): the wave that reads a sequence's
// last block first stores the sequence's new token; it is that block's only
// reader.  NBUF: tiles in flight per wave (two for split-K partitions shorter
// than kDeepBelow tokens, whose items are short enough that the first
// tiles' latency is a large share of each).
template <int NW, bool SPLIT, bool STORE = false, int NBUF = kMfmaBufs>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_mfma_fp8_kernel(const DecodeArgs a) {
  __shared__ uint16_t p_lds[NW][kHPW][kBS];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.Hq / a.Hkv;
  const int nhg = a.Hkv * (G / kHPW);
  const int hg = blockIdx.x % nhg;
  const int item = (blockIdx.x / nhg) * NW + w;
  const int n_items = SPLIT ? a.total_parts : a.S;
  if (item >= n_items) return;
  float* ws_ml = a.ws + (size_t)a.total_parts * a.Hq * kD;
  if constexpr (SPLIT) {
    const MItem it = split_item<STORE>(a, item * nhg + hg, nhg, lane, a.part_off, a.lens);
    mfma_item<NBUF>(a, it.s, it.hkv, it.qh0, it.j0, it.jend, it.t1, it.bad, it.final_out,
              (size_t)it.row * a.Hq + it.qh0, a.ws, ws_ml, p_lds[w], lane, it.store, it.L);
  } else {
    const int s = item, hkv = hg / (G / kHPW);
    const int qh0 = hkv * G + (hg % (G / kHPW)) * kHPW;
    int L = a.lens[s];
    bool bad = false;
    if (L < 0) { L = 0; bad = true; }
    if (L > a.max_blocks * kBS) { L = a.max_blocks * kBS; bad = true; }
    mfma_item<NBUF>(a, s, hkv, qh0, 0, (L + kBS - 1) / kBS, L, bad, true, 0, a.ws, ws_ml, p_lds[w],
              lane, STORE && !bad && L > 0, L);
  }
}

// Paged read probe for this kernel's shape (a measurement aid): the split-K
// kernel above without its arithmetic -- same grid, item mapping
// (split_item), block-table walk, tile ring and per-lane addresses (value
// rows permuted as the products need them) -- every tile folded into a
// checksum that is stored only on a value nobody expects.
template <int NW, int NBUF>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void paged_read_probe_mfma_kernel(const DecodeArgs a, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, g = lane >> 5;
  const int nhg = a.Hkv * (a.Hq / a.Hkv / kHPW);
  const int hg = blockIdx.x % nhg;
  const int item = (blockIdx.x / nhg) * NW + w;
  if (item >= a.total_parts) return;
  const MItem it = split_item<false>(a, item * nhg + hg, nhg, lane, a.part_off, a.lens);
  bool bad = it.bad;
  const int32_t* __restrict__ tbl = a.tables + (size_t)it.s * a.max_blocks;
  const size_t head_off = (size_t)it.hkv * kTile;
  uint32_t acc = 0;
  tile_loop<NBUF, kNLoad, 1>(
      tbl, it.j0, it.jend, a.nb, (const uint8_t*)a.kc + head_off + lane * 16,
      (const uint8_t*)a.vc + head_off + col * 32 + g * 16, (size_t)a.Hkv * kTile, lane, bad,
      [&](int, const u32x4* kr, const u32x4* vr) {
#pragma unroll
        for (int l = 0; l < kNLoad; ++l)
          acc ^= kr[l].x ^ kr[l].y ^ kr[l].z ^ kr[l].w ^ vr[l].x ^ vr[l].y ^ vr[l].z ^ vr[l].w;
      });
  if (acc == 0x9e3779b9u && !bad) sink[0] = acc;
}

// ---- persistent split-K with a work counter --------------------------------
// The counter is one 64-bit word after the partials in the workspace: the
// launch's epoch (a host-side number unique to each launch) in bits 24..63
// and the count of items taken beyond the static first ones in bits 0..23.
// The first wave of the grid writes (epoch, 0) at its start; a wave's add
// that returns another epoch ran before that write (its increment is lost
// with the old value), so the wave waits for the epoch to appear and adds
// again.  Workgroup 0 is dispatched first and resident, so the write comes;
// the wait is still bounded (below), so every wave ends.  The atomics are
// agent-scope read-modify-writes, which the hardware performs coherently for
// all XCDs of the device.
constexpr int kCountBits = 24;
constexpr unsigned long long kCountMask = (1ull << kCountBits) - 1;
constexpr int kMaxCachedSeqs = 64 * kOrderChunks;   // sequences whose offsets fit the LDS copy

// Taking an item is split in two so that the atomic's round trip overlaps a
// tile: grab_issue adds to the counter (lane 0) and returns the old value
// unread; grab_finish, once a tile later, turns it into an item index (R +
// count, or n_items when the work is exhausted).  A value of another epoch
// means this launch's first write has not landed yet: wait for it (at most
// ~14 ms per try, 8 tries, then take no further item) and add again.
__device__ __forceinline__ unsigned long long grab_issue(unsigned long long* ctr, int lane) {
  unsigned long long v = 0;
  if (lane == 0) v = atomicAdd(ctr, 1ull);
  return v;
}

__device__ __forceinline__ int grab_finish(unsigned long long v, unsigned long long* ctr,
                                          unsigned long long epoch, int R, int n_items, int lane) {
  int x = n_items;
  if (lane == 0) {
    for (int tries = 0;; ++tries) {
      if ((v >> kCountBits) == epoch) {
        const unsigned long long c = v & kCountMask;
        x = c < (unsigned long long)(n_items - R) ? R + (int)c : n_items;
        break;
      }
      if (tries == 8) break;
      for (int spin = 0;
           spin < (1 << 16) &&
           (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> kCountBits) != epoch;
           ++spin)
        __builtin_amdgcn_s_sleep(8);
      v = atomicAdd(ctr, 1ull);
    }
  }
  return __builtin_amdgcn_readfirstlane(x);
}

// Load tile j of an item into kd / vd: block id from lane (j - j0) of tv (the
// item's table entries, one per lane), bad set (and block 0 read) when the id
// is out of range.
__device__ __forceinline__ void load_mfma_tile(const DecodeArgs& a, int tv, int k, int hkv,
                                               int lane, bool& bad, u32x4* kd, u32x4* vd) {
  int b = __builtin_amdgcn_readlane(tv, k);
  if ((unsigned)b >= (unsigned)a.nb) { bad = true; b = 0; }
  const int col = lane & 31, g = lane >> 5;
  const size_t base = ((size_t)b * a.Hkv + hkv) * kTile;
  const uint8_t* kt = (const uint8_t*)a.kc + base + lane * 16;
  const uint8_t* vt = (const uint8_t*)a.vc + base + col * 32 + g * 16;
#pragma unroll
  for (int l = 0; l < kNLoad; ++l) kd[l] = load16(kt + l * 1024);
#pragma unroll
  for (int l = 0; l < kNLoad; ++l) vd[l] = load16(vt + l * 1024);
}

// Work-counter split-K decode: R = gridDim.x * NW persistent waves; wave gw
// takes item gw, then items R, R + 1, ... from the counter, in split_item's
// order.  While item i streams, the wave has claimed item i+1 (the claim
// goes out when item i becomes current and is read a tile later), then
// loads item i+1's table entries (one per lane: items have at most 64
// tiles, partitions of <= 2048 tokens) and query rows (2 KB, 32 bytes per
// lane, moved through LDS into the MFMA layout at the switch); item i+1's
// first tile is loaded as soon as item i's last tile is in registers,
// before item i's epilogue.
template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_mfma_queue_kernel(const DecodeArgs a) {
  __shared__ uint16_t p_lds[NW][kHPW][kBS];
  __shared__ u32x4 q_lds[NW][kQBytes / 16];
  const int lane = threadIdx.x & 63, col = lane & 31, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = blockIdx.x * NW + w;
  const int R = gridDim.x * NW;
  const int nhg = a.Hkv * (a.Hq / a.Hkv / kHPW);
  const int n_items = a.total_parts * nhg;
  float* ws_ml = a.ws + (size_t)a.total_parts * a.Hq * kD;
  unsigned long long* ctr = (unsigned long long*)(ws_ml + (size_t)a.total_parts * a.Hq * 2);
  if (gw == 0 && lane == 0)
    __hip_atomic_store(ctr, a.epoch << kCountBits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // the lengths and partition offsets, copied to LDS once (the host sends
  // at most kMaxCachedSeqs sequences here): describing an item then costs no
  // memory round trip in the middle of a stream
  __shared__ int32_t off[kMaxCachedSeqs + 1], lens[kMaxCachedSeqs];
  for (int i = threadIdx.x; i <= a.S; i += NW * 64) {
    off[i] = a.part_off[i];
    if (i < a.S) lens[i] = a.lens[i];
  }
  __syncthreads();
  if (gw >= n_items) return;

  MItem cur = split_item<false>(a, gw, nhg, lane, off, lens);
  int ctv = lane < cur.jend - cur.j0 ? a.tables[(size_t)cur.s * a.max_blocks + cur.j0 + lane] : 0;
  MfmaHeads h;
  h.set_q((const uint16_t*)a.q + ((size_t)cur.s * a.Hq + cur.qh0) * kD, col, g);
  unsigned long long gv = grab_issue(ctr, lane);   // the next item, read a tile later
  u32x4 kb[kNLoad], vb[kNLoad];
  bool cbad = cur.bad;
  if (cur.jend > cur.j0) load_mfma_tile(a, ctv, 0, cur.hkv, lane, cbad, kb, vb);

  for (;;) {
    h.reset();
    bool has_nxt = false, nxt_ahead = false, nbad = false;
    MItem nxt{};
    int ntv = 0;
    u32x4 nq0 = {0, 0, 0, 0}, nq1 = {0, 0, 0, 0};
    // the next item: description, table entries and query rows
    auto fetch_next = [&] {
      const int nx = grab_finish(gv, ctr, a.epoch, R, n_items, lane);
      if (nx >= n_items) return;
      has_nxt = true;
      nxt = split_item<false>(a, nx, nhg, lane, off, lens);
      nbad = nxt.bad;
      if (lane < nxt.jend - nxt.j0) ntv = a.tables[(size_t)nxt.s * a.max_blocks + nxt.j0 + lane];
      const u32x4* qsrc = (const u32x4*)((const uint16_t*)a.q + ((size_t)nxt.s * a.Hq + nxt.qh0) * kD);
      nq0 = qsrc[2 * lane];
      nq1 = qsrc[2 * lane + 1];
      nxt_ahead = nxt.jend > nxt.j0;
    };
    const int n = cur.jend - cur.j0;
    if (n == 0) fetch_next();
    for (int k = 0; k < n; ++k) {
      h.tile(a.qk_mult, cur.j0 + k, cur.t1, kb, vb, p_lds[w], col, g);
      if (k + 1 < n) load_mfma_tile(a, ctv, k + 1, cur.hkv, lane, cbad, kb, vb);
      if (k == 0) fetch_next();
      if (k + 1 == n && nxt_ahead) load_mfma_tile(a, ntv, 0, nxt.hkv, lane, nbad, kb, vb);
    }
    h.finish(a, cur.s, cur.qh0, cbad, cur.final_out, (size_t)cur.row * a.Hq + cur.qh0, a.ws, ws_ml,
             col, g);
    if (!has_nxt) break;
    // switch to the next item: its query rows through LDS into the A layout
    q_lds[w][2 * lane] = nq0;
    q_lds[w][2 * lane + 1] = nq1;
    __builtin_amdgcn_wave_barrier();
    h.set_q((const uint16_t*)q_lds[w], col, g);
    __builtin_amdgcn_wave_barrier();
    cur = nxt;
    ctv = ntv;
    cbad = nbad;
    gv = grab_issue(ctr, lane);
  }
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

// Resident workgroups of a kernel on the current device (at least 1), or -1.
int resident_wgs(const void* kernel, int threads) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
    return -1;
  return (per_cu > 1 ? per_cu : 1) * cus;
}

// resident_wgs of the work-counter kernel on the current device, looked up once per device.
int queue_resident_wgs() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return -1;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  c = resident_wgs(reinterpret_cast<const void*>(&decode_mfma_queue_kernel<kWaves>), kWaves * 64);
  if (c > 0) cache[dev].store(c, std::memory_order_relaxed);
  return c;
}

// Epoch of a work-counter launch: unique per launch within the process, and
// started from the clock so that a counter word left in reused memory by
// another process is unlikely to carry it.
unsigned long long next_epoch() {
  static std::atomic<unsigned long long> ctr{
      (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count() * 2654435761ull};
  return (ctr.fetch_add(1) + 1) & ((1ull << (64 - kCountBits)) - 1);
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

bool decode_queue_supported(const DecodeArgs& a) {
  const long long n_items = (long long)a.total_parts * (a.Hq / 8);
  return decode_mfma_eligible(a) && a.partition > 0 && a.partition <= 64 * kBS &&
         a.S <= kMaxCachedSeqs && n_items < (1ll << kCountBits) - (1ll << 20);
}

int launch_paged_read_probe_mfma(const DecodeArgs& a, uint32_t* sink, void* stream) {
  if (a.partition <= 0) return (int)hipErrorInvalidValue;
  const int nhg = a.Hkv * (a.Hq / a.Hkv / 8);
  dim3 block(kWaves * 64), grid((a.total_parts + kWaves - 1) / kWaves * nhg);
  if (a.partition < kDeepBelow)
    hipLaunchKernelGGL((paged_read_probe_mfma_kernel<kWaves, 2>), grid, block, 0,
                       (hipStream_t)stream, a, sink);
  else
    hipLaunchKernelGGL((paged_read_probe_mfma_kernel<kWaves, kMfmaBufs>), grid, block, 0,
                       (hipStream_t)stream, a, sink);
  return (int)hipGetLastError();
}

int launch_decode_mfma(const DecodeArgs& a, void* stream, bool store) {
  hipStream_t st = (hipStream_t)stream;
  const int groups = a.Hq / a.Hkv / 8;
  if (store && groups != 1) return (int)hipErrorInvalidValue;
  dim3 block(kWaves * 64);
  const int nhg = a.Hkv * groups;
  const int items = a.partition > 0 ? a.total_parts : a.S;
  dim3 grid((items + kWaves - 1) / kWaves * nhg);
  if (a.partition > 0 && a.partition < kDeepBelow) {
    if (store)
      hipLaunchKernelGGL((decode_mfma_fp8_kernel<kWaves, true, true, 2>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((decode_mfma_fp8_kernel<kWaves, true, false, 2>), grid, block, 0, st, a);
  } else if (a.partition > 0) {
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

// Work-counter schedule (paged_attention_decode_queue): as many resident
// workgroups as the items need, each launch with its own epoch.  Shapes
// outside decode_queue_supported are refused before this is called.
int launch_decode_mfma_queue(const DecodeArgs& a0, void* stream) {
  if (!decode_queue_supported(a0)) return (int)hipErrorInvalidValue;
  const int c = queue_resident_wgs();
  if (c <= 0) return (int)hipErrorInvalidValue;
  DecodeArgs a = a0;
  a.epoch = next_epoch();
  const long long need = ((long long)a.total_parts * (a.Hq / 8) + kWaves - 1) / kWaves;
  dim3 block(kWaves * 64), grid((unsigned)std::min<long long>(c, need));
  hipLaunchKernelGGL((decode_mfma_queue_kernel<kWaves>), grid, block, 0, (hipStream_t)stream, a);
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
  const int wgs = resident_wgs(reinterpret_cast<const void*>(&decode_mfma_sk_kernel<kSkWaves, false>),
                               kSkWaves * 64);
  return wgs > 0 ? wgs * kSkWaves : -1;
}

}  // namespace pkv
