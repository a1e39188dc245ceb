// Block-pool maintenance kernels: the per-step slot scatter of new key/value
// rows, whole-block copies for copy-on-write, and a gather of sequences back
// into dense rows.
//
// "Day 6/90 of Inference Engineering" (PagedAttention notes): each decode
// step writes its token into whichever block the manager handed out, and a
// prompt that diverges from a shared prefix continues in a fresh block.
//
// Pool layout (elements of E bytes, X = 16 / E):
//   key   [NB][H][D/X][BS][X]    value [NB][H][D][BS]

#include <hip/hip_runtime.h>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

// One thread per (token, kv head, 16-byte key unit of the cache): it writes
// that key unit and the X value elements of the same dims.
template <int SRC, int CACHE>
__global__ __launch_bounds__(256) void kv_write_kernel(const void* __restrict__ key,
                                                       const void* __restrict__ value,
                                                       uint8_t* __restrict__ kc,
                                                       uint8_t* __restrict__ vc,
                                                       const int32_t* __restrict__ slots, int T,
                                                       int H, int D, int BS, int nb, float k_inv,
                                                       float v_inv) {
  constexpr int E = CACHE == PKV_F32 ? 4 : CACHE == PKV_BF16 ? 2 : 1;
  constexpr int X = 16 / E;
  const int units = D / X;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long)T * H * units) return;
  const int c = (int)(gid % units);
  const int h = (int)((gid / units) % H);
  const int t = (int)(gid / ((long)units * H));
  const int slot = slots[t];
  if (slot < 0 || slot >= nb * BS) return;
  write_kv_unit<CACHE>(key, value, kc, vc, t, h, c, slot, H, D, BS, k_inv, v_inv);
}

// Block-wise scatter (bf16 rows into a bf16 or fp8 cache).  Workgroup (g, h)
// owns input rows g*BS .. g*BS + BS - 1 of kv head h.  A row is covered when
// the BS rows around it that its slot's block needs (its block's slots, in
// order, on consecutive input rows) are all present -- the usual case inside
// the chunk of a prefill, wherever the chunk starts.  The workgroup whose
// rows hold a covered block's first slot writes that whole block: key units
// as contiguous 16-byte runs, value rows staged in LDS and written as whole
// dim rows of the block's value tile (16-byte pieces, full lines) instead of
// one element per dim row per token.  Rows that are not covered are
// scattered one unit at a time as kv_write_kernel does.  The stored bits are
// the same either way.
template <int CACHE, int D, int BS>
__global__ __launch_bounds__(256) void kv_write_block_kernel(const uint16_t* __restrict__ key,
                                                             const uint16_t* __restrict__ value,
                                                             uint8_t* __restrict__ kc,
                                                             uint8_t* __restrict__ vc,
                                                             const int32_t* __restrict__ slots,
                                                             int T, int H, int nb, float k_inv,
                                                             float v_inv) {
  constexpr int E = CACHE == PKV_BF16 ? 2 : 1;   // cache element bytes
  constexpr int X = 16 / E;                       // elements per 16-byte cache unit
  constexpr int UNITS = D / X;                    // key units per token
  constexpr int PER = 16 / E;                     // tokens per 16-byte piece of a value row
  __shared__ uint32_t vt[BS][D / 2 + 1];          // a block's value rows (bf16 pairs)
  __shared__ int covered[BS];
  __shared__ int start;                           // row of a covered block's first slot
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * BS, h = blockIdx.y;
  const int nslots = nb * BS;
  if (tid < BS) covered[tid] = 1;
  if (tid == 0) start = -1;
  __syncthreads();
  // coverage: pair (row r, offset k) checks that input row r - o + k holds
  // slot (slot_r - o) + k, o being row r's offset in its block
  for (int i = tid; i < BS * BS; i += 256) {
    const int r = i / BS, k = i % BS, t = t0 + r;
    bool ok = false;
    if (t < T) {
      const int sr = slots[t];
      if (sr >= 0 && sr < nslots) {
        const int o = sr % BS, ts = t - o;
        ok = ts >= 0 && ts + BS <= T && slots[ts + k] == sr - o + k;
      }
    }
    if (!ok) covered[r] = 0;
  }
  __syncthreads();
  // a covered row at offset 0 starts its block; two such rows are at least
  // BS rows apart, so at most one lies here
  if (tid < BS && covered[tid] && slots[t0 + tid] % BS == 0) start = tid;
  // rows that are not covered: one unit at a time
  for (int i = tid; i < BS * UNITS; i += 256) {
    const int r = i / UNITS, c = i % UNITS, t = t0 + r;
    if (t >= T || covered[r]) continue;
    const int slot = slots[t];
    if (slot < 0 || slot >= nslots) continue;
    write_kv_unit<CACHE>(key, value, kc, vc, t, h, c, slot, H, D, BS, k_inv, v_inv);
  }
  __syncthreads();
  const int r0 = start;
  if (r0 < 0) return;                     // no whole block starts in these rows
  const int ts = t0 + r0;                 // its rows: ts .. ts + BS - 1
  const size_t tile = (size_t)(slots[ts] / BS) * H + h;   // (block, kv head) tile index
  // keys: unit (c, token k) at ((tile * UNITS + c) * BS + k) * 16
  for (int i = tid; i < BS * UNITS; i += 256) {
    const int c = i / BS, k = i % BS;
    const uint16_t* src = key + ((size_t)(ts + k) * H + h) * D + c * X;
    uint8_t* dst = kc + ((tile * UNITS + c) * BS + k) * 16;
    if constexpr (CACHE == PKV_BF16) {
      *(u32x4*)dst = *(const u32x4*)src;
    } else {
      const u32x4 ka = *(const u32x4*)src, kb = *(const u32x4*)(src + 8);
      const uint32_t kw[8] = {ka.x, ka.y, ka.z, ka.w, kb.x, kb.y, kb.z, kb.w};
      uint32_t kout[4] = {0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t k0 = f32_to_e4m3(bf16_lo(kw[j]) * k_inv);
        const uint32_t k1 = f32_to_e4m3(bf16_hi(kw[j]) * k_inv);
        kout[j / 2] |= (k0 | (k1 << 8)) << (16 * (j % 2));
      }
      *(u32x4*)dst = u32x4{kout[0], kout[1], kout[2], kout[3]};
    }
  }
  // values: stage the rows, then write dim row d's tokens PER at a time
  for (int i = tid; i < BS * (D / 8); i += 256) {
    const int k = i / (D / 8), q = i % (D / 8);
    const u32x4 v = *(const u32x4*)(value + ((size_t)(ts + k) * H + h) * D + q * 8);
    vt[k][4 * q] = v.x;
    vt[k][4 * q + 1] = v.y;
    vt[k][4 * q + 2] = v.z;
    vt[k][4 * q + 3] = v.w;
  }
  __syncthreads();
  for (int i = tid; i < D * (BS / PER); i += 256) {
    const int d = i / (BS / PER), piece = i % (BS / PER);
    uint32_t out[4] = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint32_t w = vt[piece * PER + j][d / 2];
      const float f = (d & 1) ? bf16_hi(w) : bf16_lo(w);
      const uint32_t code = CACHE == PKV_BF16 ? ((d & 1) ? w >> 16 : w & 0xffffu)
                                              : f32_to_e4m3(f * v_inv);
      out[j * E / 4] |= code << (8 * ((j * E) % 4));
    }
    *(u32x4*)(vc + ((tile * D + d) * BS + piece * PER) * E) = u32x4{out[0], out[1], out[2], out[3]};
  }
}

// Decode-step scatter: one thread per (sequence, kv head, key unit); row s
// of key/value is sequence s's new token, stored at position lens[s] - 1 in
// the slot its block table gives.  Sequences of length 0, beyond the table or
// with an out-of-range block id are skipped, and so, with t_start (the
// shared-prefix decode step), is a sequence whose new token lies before its
// own blocks (lens[s] <= t_start[s]).
template <int CACHE>
__global__ __launch_bounds__(256) void kv_write_tail_kernel(const void* __restrict__ key,
                                                            const void* __restrict__ value,
                                                            uint8_t* __restrict__ kc,
                                                            uint8_t* __restrict__ vc,
                                                            const int32_t* __restrict__ tables,
                                                            int max_blocks,
                                                            const int32_t* __restrict__ lens, int S,
                                                            int H, int D, int BS, int nb,
                                                            float k_inv, float v_inv,
                                                            const int32_t* __restrict__ t_start) {
  constexpr int X = 16 / (CACHE == PKV_F32 ? 4 : CACHE == PKV_BF16 ? 2 : 1);
  const int units = D / X;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long)S * H * units) return;
  const int c = (int)(gid % units);
  const int h = (int)((gid / units) % H);
  const int s = (int)(gid / ((long)units * H));
  const int L = lens[s];
  if (L <= 0 || L > max_blocks * BS) return;
  if (t_start && L <= t_start[s]) return;
  const int pos = L - 1;
  const int blk = tables[(size_t)s * max_blocks + pos / BS];
  if ((unsigned)blk >= (unsigned)nb) return;
  write_kv_unit<CACHE>(key, value, kc, vc, s, h, c, blk * BS + pos % BS, H, D, BS, k_inv, v_inv);
}

// One workgroup per (pair, pool): copies block_bytes from block src to dst.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t* __restrict__ kc,
                                                          uint8_t* __restrict__ vc,
                                                          const int32_t* __restrict__ pairs,
                                                          size_t block_bytes, int nb) {
  const int src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
  if ((unsigned)src >= (unsigned)nb || (unsigned)dst >= (unsigned)nb) return;
  uint8_t* pool = blockIdx.y == 0 ? kc : vc;
  const u32x4* s = (const u32x4*)(pool + (size_t)src * block_bytes);
  u32x4* d = (u32x4*)(pool + (size_t)dst * block_bytes);
  const size_t n = block_bytes / 16;
  for (size_t i = threadIdx.x; i < n; i += 256) d[i] = s[i];
}

// Whole-block moves between two pools: unit u = (pair u / 2, pool u % 2)
// copies src block pairs[i][0] to dst block pairs[i][1] of the key (pool 0)
// or value (pool 1) pool.  A bounded grid walks the units (grid stride),
// four 16-byte units per thread in flight, and leaves most wave slots to
// kernels of other streams.  Ids out of range skip the pair.
__global__ __launch_bounds__(256) void swap_blocks_kernel(uint8_t* __restrict__ dk,
                                                          uint8_t* __restrict__ dv,
                                                          const uint8_t* __restrict__ sk,
                                                          const uint8_t* __restrict__ sv,
                                                          const int32_t* __restrict__ pairs,
                                                          int n_pairs, size_t block_bytes,
                                                          int src_nb, int dst_nb) {
  const size_t n = block_bytes / 16;
  for (int unit = blockIdx.x; unit < 2 * n_pairs; unit += gridDim.x) {
    const int i = unit >> 1, pool = unit & 1;
    const int src = pairs[2 * i], dst = pairs[2 * i + 1];
    if ((unsigned)src >= (unsigned)src_nb || (unsigned)dst >= (unsigned)dst_nb) continue;
    const u32x4* s = (const u32x4*)((pool == 0 ? sk : sv) + (size_t)src * block_bytes);
    u32x4* d = (u32x4*)((pool == 0 ? dk : dv) + (size_t)dst * block_bytes);
    for (size_t i0 = threadIdx.x; i0 < n; i0 += 4 * 256) {
      u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const size_t j = i0 + (size_t)u * 256;
        if (j < n) v[u] = s[j];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const size_t j = i0 + (size_t)u * 256;
        if (j < n) d[j] = v[u];
      }
    }
  }
}

// One thread per (output row, kv head, 16-byte unit of the dense row).
template <int CACHE>
__global__ __launch_bounds__(256) void gather_kernel(uint8_t* __restrict__ k_out,
                                                     uint8_t* __restrict__ v_out,
                                                     const uint8_t* __restrict__ kc,
                                                     const uint8_t* __restrict__ vc,
                                                     const int32_t* __restrict__ tables,
                                                     int max_blocks,
                                                     const int32_t* __restrict__ cu_ctx, int S,
                                                     int T, int H, int D, int BS, int nb) {
  constexpr int E = CACHE == PKV_F32 ? 4 : CACHE == PKV_BF16 ? 2 : 1;
  constexpr int X = 16 / E;
  const int units = D / X;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long)T * H * units) return;
  const int c = (int)(gid % units);
  const int h = (int)((gid / units) % H);
  const int r = (int)(gid / ((long)units * H));
  int lo = 0, hi = S;  // largest s with cu_ctx[s] <= r
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (cu_ctx[mid] <= r) lo = mid; else hi = mid;
  }
  const int s = lo, t = r - cu_ctx[s];
  const int jb = t / BS, o = t % BS;
  const size_t dst = (((size_t)r * H + h) * D + (size_t)c * X) * E;
  u32x4 kz = {0, 0, 0, 0}, vz = {0, 0, 0, 0};
  const int b = jb < max_blocks ? tables[(size_t)s * max_blocks + jb] : -1;
  if ((unsigned)b < (unsigned)nb) {
    kz = *(const u32x4*)(kc + ((((size_t)b * H + h) * (D / X) + c) * BS + o) * 16);
    const size_t v0 = (((size_t)b * H + h) * D + (size_t)c * X) * BS + o;  // element index
    uint32_t wv[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < X; ++i) {
      uint32_t e;
      if constexpr (E == 4) e = ((const uint32_t*)vc)[v0 + (size_t)i * BS];
      else if constexpr (E == 2) e = ((const uint16_t*)vc)[v0 + (size_t)i * BS];
      else e = vc[v0 + (size_t)i * BS];
      wv[(i * E) / 4] |= e << (8 * ((i * E) % 4));
    }
    vz = u32x4{wv[0], wv[1], wv[2], wv[3]};
  }
  *(u32x4*)(k_out + dst) = kz;
  *(u32x4*)(v_out + dst) = vz;
}

}  // namespace

int launch_kv_write(const void* key, const void* value, void* kc, void* vc, const int32_t* slots,
                    int T, int H, int D, int BS, int nb, pkv_dtype src, pkv_dtype cache,
                    float k_inv, float v_inv, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int X = 16 / elem_bytes(cache);
  const long n = (long)T * H * (D / X);
  if (n == 0) return 0;
  dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (cache != PKV_F32 && src == PKV_BF16) {
    // block-wise: one workgroup per (BS input rows, kv head)
    dim3 bgrid((unsigned)((T + BS - 1) / BS), (unsigned)H);
    auto k16 = (const uint16_t*)key, v16 = (const uint16_t*)value;
    auto kc8 = (uint8_t*)kc, vc8 = (uint8_t*)vc;
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, bgrid, block, 0, st, k16, v16, kc8, vc8, slots, T, H, nb, k_inv,
                         v_inv);
    };
    const bool f8 = cache == PKV_FP8_E4M3;
    if (D == 128 && BS == 16)
      f8 ? go(kv_write_block_kernel<PKV_FP8_E4M3, 128, 16>) : go(kv_write_block_kernel<PKV_BF16, 128, 16>);
    else if (D == 128)
      f8 ? go(kv_write_block_kernel<PKV_FP8_E4M3, 128, 32>) : go(kv_write_block_kernel<PKV_BF16, 128, 32>);
    else if (BS == 16)
      f8 ? go(kv_write_block_kernel<PKV_FP8_E4M3, 64, 16>) : go(kv_write_block_kernel<PKV_BF16, 64, 16>);
    else
      f8 ? go(kv_write_block_kernel<PKV_FP8_E4M3, 64, 32>) : go(kv_write_block_kernel<PKV_BF16, 64, 32>);
    return (int)hipGetLastError();
  }
  if (cache == PKV_F32)
    hipLaunchKernelGGL((kv_write_kernel<PKV_F32, PKV_F32>), grid, block, 0, st, key, value,
                       (uint8_t*)kc, (uint8_t*)vc, slots, T, H, D, BS, nb, k_inv, v_inv);
  else if (cache == PKV_BF16)
    hipLaunchKernelGGL((kv_write_kernel<PKV_BF16, PKV_BF16>), grid, block, 0, st, key, value,
                       (uint8_t*)kc, (uint8_t*)vc, slots, T, H, D, BS, nb, k_inv, v_inv);
  else
    hipLaunchKernelGGL((kv_write_kernel<PKV_BF16, PKV_FP8_E4M3>), grid, block, 0, st, key, value,
                       (uint8_t*)kc, (uint8_t*)vc, slots, T, H, D, BS, nb, k_inv, v_inv);
  return (int)hipGetLastError();
}

int launch_kv_write_tail(const void* key, const void* value, void* kc, void* vc,
                         const int32_t* tables, int max_blocks, const int32_t* lens, int S, int H,
                         int D, int BS, int nb, pkv_dtype cache, float k_inv, float v_inv,
                         void* stream, const int32_t* t_start) {
  hipStream_t st = (hipStream_t)stream;
  const int X = 16 / elem_bytes(cache);
  const long n = (long)S * H * (D / X);
  if (n == 0) return 0;
  dim3 grid((unsigned)((n + 255) / 256)), block(256);
  auto k8 = (uint8_t*)kc, v8 = (uint8_t*)vc;
  if (cache == PKV_F32)
    hipLaunchKernelGGL((kv_write_tail_kernel<PKV_F32>), grid, block, 0, st, key, value, k8, v8,
                       tables, max_blocks, lens, S, H, D, BS, nb, k_inv, v_inv, t_start);
  else if (cache == PKV_BF16)
    hipLaunchKernelGGL((kv_write_tail_kernel<PKV_BF16>), grid, block, 0, st, key, value, k8, v8,
                       tables, max_blocks, lens, S, H, D, BS, nb, k_inv, v_inv, t_start);
  else
    hipLaunchKernelGGL((kv_write_tail_kernel<PKV_FP8_E4M3>), grid, block, 0, st, key, value, k8,
                       v8, tables, max_blocks, lens, S, H, D, BS, nb, k_inv, v_inv, t_start);
  return (int)hipGetLastError();
}

int launch_copy_blocks(void* kc, void* vc, const int32_t* pairs, int n, size_t block_bytes, int nb,
                       void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n, 2), dim3(256), 0, (hipStream_t)stream,
                     (uint8_t*)kc, (uint8_t*)vc, pairs, block_bytes, nb);
  return (int)hipGetLastError();
}

// Workgroups of a swap launch: 256 x 16 KiB in flight, which streams an
// HBM-to-HBM move (the staging copy of a swap) at HBM rates and covers the
// host link's bandwidth-delay product many times over.  With a host pool on
// one side, 8 to 256 workgroups all reach ~55 GB/s on MI355X and all slow a
// decode running beside them (1.9x to 2.3x); whole-run asynchronous copies
// of a staged sequence do not (paged_kv_swap_blocks_memcpy).
constexpr int kSwapWorkgroups = 256;

int launch_swap_blocks(void* dk, void* dv, const void* sk, const void* sv, const int32_t* pairs,
                       int n, size_t block_bytes, int src_nb, int dst_nb, void* stream) {
  if (n == 0) return 0;
  const int wgs = (int)std::min<long long>(2ll * n, kSwapWorkgroups);
  hipLaunchKernelGGL(swap_blocks_kernel, dim3(wgs), dim3(256), 0, (hipStream_t)stream,
                     (uint8_t*)dk, (uint8_t*)dv, (const uint8_t*)sk, (const uint8_t*)sv, pairs, n,
                     block_bytes, src_nb, dst_nb);
  return (int)hipGetLastError();
}

int launch_gather(void* k_out, void* v_out, const void* kc, const void* vc, const int32_t* tables,
                  int max_blocks, const int32_t* cu_ctx, int S, int T, int H, int D, int BS,
                  int nb, pkv_dtype cache, void* stream) {
  const int X = 16 / elem_bytes(cache);
  const long n = (long)T * H * (D / X);
  if (n == 0) return 0;
  dim3 grid((unsigned)((n + 255) / 256)), block(256);
  hipStream_t st = (hipStream_t)stream;
  auto ko = (uint8_t*)k_out, vo = (uint8_t*)v_out;
  auto kcc = (const uint8_t*)kc, vcc = (const uint8_t*)vc;
  if (cache == PKV_F32)
    hipLaunchKernelGGL((gather_kernel<PKV_F32>), grid, block, 0, st, ko, vo, kcc, vcc, tables,
                       max_blocks, cu_ctx, S, T, H, D, BS, nb);
  else if (cache == PKV_BF16)
    hipLaunchKernelGGL((gather_kernel<PKV_BF16>), grid, block, 0, st, ko, vo, kcc, vcc, tables,
                       max_blocks, cu_ctx, S, T, H, D, BS, nb);
  else
    hipLaunchKernelGGL((gather_kernel<PKV_FP8_E4M3>), grid, block, 0, st, ko, vo, kcc, vcc, tables,
                       max_blocks, cu_ctx, S, T, H, D, BS, nb);
  return (int)hipGetLastError();
}

}  // namespace pkv

// ---------------------------------------------------------------------------
// Streaming-read probe: every lane reads 16-byte units of a buffer with
// UNROLL loads in flight, folds them into a checksum and stores nothing
// unless the checksum hits a sentinel.  Measures the attainable HBM read
// rate of this GPU, the ceiling the decode kernel's KV stream is held to.
namespace pkv {
namespace {
// Streaming read: workgroup g reads one contiguous run of 256 * UNROLL
// 16-byte units (lane t: units base + t, base + t + 256, ...), all loads in
// flight before any is used, non-temporal.  Of the layouts measured on
// MI355X (a grid-stride sweep with 4 to 8 loads per lane, contiguous runs of
// 4 to 16 loads per lane, plain and non-temporal loads, direct-to-LDS loads)
// this one streamed fastest.
template <int UNROLL>
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink) {
  constexpr size_t RUN = 256 * UNROLL;
  uint32_t acc = 0;
  for (size_t base = (size_t)blockIdx.x * RUN; base < n16; base += (size_t)gridDim.x * RUN) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const size_t i = base + (size_t)u * 256 + threadIdx.x;
      v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}
}  // namespace

int launch_read_probe(const void* src, size_t bytes, void* sink, int blocks, void* stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return 0;
  hipLaunchKernelGGL((read_probe_kernel<8>), dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)src, n16, (uint32_t*)sink);
  return (int)hipGetLastError();
}
}  // namespace pkv
