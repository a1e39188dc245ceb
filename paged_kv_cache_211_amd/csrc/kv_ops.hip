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

// Decode-step scatter: one thread per (sequence, kv head, key unit); row s
// of key/value is sequence s's new token, stored at position lens[s] - 1 in
// the slot its block table gives.  Sequences of length 0, beyond the table or
// with an out-of-range block id are skipped.
template <int CACHE>
__global__ __launch_bounds__(256) void kv_write_tail_kernel(const void* __restrict__ key,
                                                            const void* __restrict__ value,
                                                            uint8_t* __restrict__ kc,
                                                            uint8_t* __restrict__ vc,
                                                            const int32_t* __restrict__ tables,
                                                            int max_blocks,
                                                            const int32_t* __restrict__ lens, int S,
                                                            int H, int D, int BS, int nb,
                                                            float k_inv, float v_inv) {
  constexpr int X = 16 / (CACHE == PKV_F32 ? 4 : CACHE == PKV_BF16 ? 2 : 1);
  const int units = D / X;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long)S * H * units) return;
  const int c = (int)(gid % units);
  const int h = (int)((gid / units) % H);
  const int s = (int)(gid / ((long)units * H));
  const int L = lens[s];
  if (L <= 0 || L > max_blocks * BS) return;
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

// Whole blocks between two pools of one layout (a device pool and a pinned
// host pool reached through its device pointer): workgroup (i, pool) copies
// src block pairs[i][0] to dst block pairs[i][1], four 16-byte units per
// thread in flight (loads from host memory cross the host link, so many
// must be outstanding).  Ids out of range skip the pair.
__global__ __launch_bounds__(256) void swap_blocks_kernel(uint8_t* __restrict__ dk,
                                                          uint8_t* __restrict__ dv,
                                                          const uint8_t* __restrict__ sk,
                                                          const uint8_t* __restrict__ sv,
                                                          const int32_t* __restrict__ pairs,
                                                          size_t block_bytes, int src_nb,
                                                          int dst_nb) {
  const int src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
  if ((unsigned)src >= (unsigned)src_nb || (unsigned)dst >= (unsigned)dst_nb) return;
  const u32x4* s = (const u32x4*)((blockIdx.y == 0 ? sk : sv) + (size_t)src * block_bytes);
  u32x4* d = (u32x4*)((blockIdx.y == 0 ? dk : dv) + (size_t)dst * block_bytes);
  const size_t n = block_bytes / 16;
  for (size_t i0 = threadIdx.x; i0 < n; i0 += 4 * 256) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t i = i0 + (size_t)u * 256;
      if (i < n) v[u] = s[i];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t i = i0 + (size_t)u * 256;
      if (i < n) d[i] = v[u];
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
                         void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int X = 16 / elem_bytes(cache);
  const long n = (long)S * H * (D / X);
  if (n == 0) return 0;
  dim3 grid((unsigned)((n + 255) / 256)), block(256);
  auto k8 = (uint8_t*)kc, v8 = (uint8_t*)vc;
  if (cache == PKV_F32)
    hipLaunchKernelGGL((kv_write_tail_kernel<PKV_F32>), grid, block, 0, st, key, value, k8, v8,
                       tables, max_blocks, lens, S, H, D, BS, nb, k_inv, v_inv);
  else if (cache == PKV_BF16)
    hipLaunchKernelGGL((kv_write_tail_kernel<PKV_BF16>), grid, block, 0, st, key, value, k8, v8,
                       tables, max_blocks, lens, S, H, D, BS, nb, k_inv, v_inv);
  else
    hipLaunchKernelGGL((kv_write_tail_kernel<PKV_FP8_E4M3>), grid, block, 0, st, key, value, k8,
                       v8, tables, max_blocks, lens, S, H, D, BS, nb, k_inv, v_inv);
  return (int)hipGetLastError();
}

int launch_copy_blocks(void* kc, void* vc, const int32_t* pairs, int n, size_t block_bytes, int nb,
                       void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n, 2), dim3(256), 0, (hipStream_t)stream,
                     (uint8_t*)kc, (uint8_t*)vc, pairs, block_bytes, nb);
  return (int)hipGetLastError();
}

int launch_swap_blocks(void* dk, void* dv, const void* sk, const void* sv, const int32_t* pairs,
                       int n, size_t block_bytes, int src_nb, int dst_nb, void* stream) {
  if (n == 0) return 0;
  hipLaunchKernelGGL(swap_blocks_kernel, dim3(n, 2), dim3(256), 0, (hipStream_t)stream,
                     (uint8_t*)dk, (uint8_t*)dv, (const uint8_t*)sk, (const uint8_t*)sv, pairs,
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
template <int UNROLL>
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink) {
  const size_t tid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  uint32_t acc = 0;
  size_t i = tid;
  for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
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
