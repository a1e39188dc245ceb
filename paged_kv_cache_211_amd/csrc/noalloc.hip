// paged_attention_decode without a caller-provided workspace, for callers
// that cannot allocate device memory: the split-K partials go to a
// file-scope device array instead.  The kernels are those of
// paged_attention_decode; only where their workspace lives differs.
//
// The array exists once per GPU the library runs on (each device holds its
// own copy at its own address, for the life of the process).  Its address
// is resolved once per device, with that device current, on the first call
// there, and every later call passes that address to the kernels as their
// workspace.  Calls that overlap on one GPU share the array and race.

#include <hip/hip_runtime.h>

#include <mutex>

#include "pkv.h"
#include "pkv_internal.h"

namespace {

constexpr size_t kScratchBytes = PKV_NOALLOC_WORKSPACE_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

// Split-K partials of paged_attention_decode_noalloc.  In host code this
// name is only a stand-in for the symbol: the device address comes from
// hipGetSymbolAddress.
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device (resolved once per device).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return pkv::fail(PKV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return pkv::fail(PKV_ERR_HIP, "device %d beyond the %d devices this library tracks", dev,
                     kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return pkv::fail(PKV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                       hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return PKV_OK;
}

}  // namespace

extern "C" int paged_attention_decode_noalloc(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
    float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype, float k_scale, float v_scale,
    int partition_tokens, const int32_t* partition_offsets, int total_partitions, void* stream) {
  pkv::DecodeCall c{out, query, key_cache, value_cache, block_tables, max_blocks_per_seq,
                    context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                    num_blocks, scale, q_dtype, cache_dtype, k_scale, v_scale, partition_tokens,
                    partition_offsets, total_partitions, nullptr, 0};
  if (partition_tokens > 0 && num_seqs > 0) {
    const size_t need =
        paged_attention_workspace_bytes(total_partitions, num_q_heads, head_dim);
    if (need > kScratchBytes)
      return pkv::fail(PKV_ERR_WORKSPACE,
                       "split-K partials need %zu bytes, more than the %zu-byte static workspace "
                       "(use longer partitions, or paged_attention_decode with a workspace)",
                       need, kScratchBytes);
    if (need > 0) {
      void* p = nullptr;
      const int rc = scratch_address(&p);
      if (rc) return rc;
      c.workspace = p;
      c.workspace_bytes = kScratchBytes;
    }
  }
  return pkv::decode_common(c, true, stream);
}
