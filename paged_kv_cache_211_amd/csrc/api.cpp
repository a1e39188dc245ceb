// C ABI of libpkv: argument checks, dtype dispatch and launches on the
// caller's stream.  Only what the host can see is checked; device contents
// are trusted (the kernels themselves refuse out-of-range block ids).

#include <cmath>
#include <cstring>

#include <hip/hip_runtime.h>

#include "pkv.h"
#include "pkv_internal.h"

namespace pkv {

static bool valid_dtype(int t) { return t == PKV_F32 || t == PKV_BF16 || t == PKV_FP8_E4M3; }

static int hip_status(int e, const char* what) {
  if (e != hipSuccess)
    return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString((hipError_t)e));
  clear_error();
  return PKV_OK;
}

static int check_decode(const DecodeCall& c, DecodeArgs* a) {
  if (!c.out || !c.query || !c.key_cache || !c.value_cache || !c.block_tables || !c.context_lens)
    return fail(PKV_ERR_INVALID, "null pointer argument");
  if (c.num_seqs < 0 || c.num_q_heads <= 0 || c.num_kv_heads <= 0 || c.max_blocks_per_seq <= 0 ||
      c.num_blocks <= 0)
    return fail(PKV_ERR_INVALID, "sizes must be positive");
  if (c.num_q_heads % c.num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "num_q_heads %% num_kv_heads != 0");
  if (!valid_dtype(c.q_dtype) || !valid_dtype(c.cache_dtype))
    return fail(PKV_ERR_INVALID, "unknown dtype");
  if (!std::isfinite(c.scale)) return fail(PKV_ERR_INVALID, "scale must be finite");
  const int G = c.num_q_heads / c.num_kv_heads;
  if (!decode_supported(c.q_dtype, c.cache_dtype, c.head_dim, c.block_size, G))
    return fail(PKV_ERR_UNSUPPORTED, "unsupported (q %d, cache %d, head_dim %d, block_size %d)",
                (int)c.q_dtype, (int)c.cache_dtype, c.head_dim, c.block_size);
  const bool fp8 = c.cache_dtype == PKV_FP8_E4M3;
  if (fp8 && (!(c.k_scale > 0.f) || !(c.v_scale > 0.f) || !std::isfinite(c.k_scale) ||
              !std::isfinite(c.v_scale)))
    return fail(PKV_ERR_INVALID, "fp8 scales must be positive and finite");
  if (c.partition_tokens < 0 || (c.partition_tokens % c.block_size) != 0)
    return fail(PKV_ERR_INVALID, "partition_tokens must be 0 or a positive multiple of block_size");
  if (c.partition_tokens > 0) {
    if (!c.partition_offsets) return fail(PKV_ERR_INVALID, "partition_offsets is null");
    if (c.total_partitions < c.num_seqs) return fail(PKV_ERR_INVALID, "total_partitions < num_seqs");
    const size_t need = paged_attention_workspace_bytes(c.total_partitions, c.num_q_heads, c.head_dim);
    if (!c.workspace || c.workspace_bytes < need)
      return fail(PKV_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, c.workspace_bytes);
    if ((uintptr_t)c.workspace % 16 != 0)
      return fail(PKV_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  }
  if ((size_t)c.num_blocks * c.block_size > (size_t)INT32_MAX)
    return fail(PKV_ERR_INVALID, "num_blocks * block_size exceeds int32 slots");

  a->out = c.out;
  a->q = c.query;
  a->kc = c.key_cache;
  a->vc = c.value_cache;
  a->tables = c.block_tables;
  a->lens = c.context_lens;
  a->part_off = c.partition_tokens > 0 ? c.partition_offsets : nullptr;
  a->ws = (float*)c.workspace;
  a->max_blocks = c.max_blocks_per_seq;
  a->S = c.num_seqs;
  a->Hq = c.num_q_heads;
  a->Hkv = c.num_kv_heads;
  a->D = c.head_dim;
  a->BS = c.block_size;
  a->nb = c.num_blocks;
  a->partition = c.partition_tokens;
  a->total_parts = c.partition_tokens > 0 ? c.total_partitions : 0;
  a->qk_mult = c.scale * (fp8 ? c.k_scale : 1.f) * kLog2eHost;
  a->v_mult = fp8 ? c.v_scale : 1.f;
  a->q_dtype = c.q_dtype;
  a->kv_dtype = c.cache_dtype;
  return PKV_OK;
}

int decode_common(const DecodeCall& c, bool reduce, void* stream) {
  DecodeArgs a;
  int rc = check_decode(c, &a);
  if (rc) return rc;
  if (c.queue && !decode_queue_supported(a))
    return fail(PKV_ERR_UNSUPPORTED,
                "the work-counter decode needs an fp8 E4M3 cache, bf16 queries, head_dim 128, "
                "block_size 32, a multiple of 8 query heads per kv head, split-K partitions of "
                "at most 2048 tokens and at most 512 sequences");
  if (c.num_seqs == 0) return PKV_OK;
  rc = hip_status(c.queue ? launch_decode_mfma_queue(a, stream) : launch_decode(a, stream),
                  "paged_attention_decode launch");
  if (rc || !reduce || c.partition_tokens == 0) return rc;
  return hip_status(launch_splitk_reduce(c.out, a.ws, c.partition_offsets, c.num_seqs,
                                         c.num_q_heads, c.head_dim, c.total_partitions,
                                         c.q_dtype, stream, 2,
                                         max_partitions(a.max_blocks, a.BS, a.partition)),
                    "paged_attention_splitk_reduce launch");
}

}  // namespace pkv

using namespace pkv;

extern "C" {

int paged_kv_write(const void* key, const void* value, void* key_cache, void* value_cache,
                   const int32_t* slot_mapping, int num_tokens, int num_kv_heads, int head_dim,
                   int block_size, int num_blocks, pkv_dtype src_dtype, pkv_dtype cache_dtype,
                   float k_scale, float v_scale, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0)
    return fail(PKV_ERR_INVALID, "sizes must be positive");
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return fail(PKV_ERR_INVALID, "null pointer argument");
  if (!valid_dtype(src_dtype) || !valid_dtype(cache_dtype))
    return fail(PKV_ERR_INVALID, "unknown dtype");
  const bool ok = (src_dtype == PKV_F32 && cache_dtype == PKV_F32) ||
                  (src_dtype == PKV_BF16 && cache_dtype == PKV_BF16) ||
                  (src_dtype == PKV_BF16 && cache_dtype == PKV_FP8_E4M3);
  if (!ok) return fail(PKV_ERR_UNSUPPORTED, "unsupported write %d -> %d", (int)src_dtype, (int)cache_dtype);
  if ((head_dim != 64 && head_dim != 128) || (block_size != 16 && block_size != 32))
    return fail(PKV_ERR_UNSUPPORTED, "head_dim must be 64/128 and block_size 16/32");
  if ((size_t)num_blocks * block_size > (size_t)INT32_MAX)
    return fail(PKV_ERR_INVALID, "num_blocks * block_size exceeds int32 slots");
  float k_inv = 1.f, v_inv = 1.f;
  if (cache_dtype == PKV_FP8_E4M3) {
    if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
      return fail(PKV_ERR_INVALID, "fp8 scales must be positive and finite");
    k_inv = 1.f / k_scale;  // one correctly rounded fp32 division
    v_inv = 1.f / v_scale;
  }
  return hip_status(launch_kv_write(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                                    num_kv_heads, head_dim, block_size, num_blocks, src_dtype,
                                    cache_dtype, k_inv, v_inv, stream),
                    "paged_kv_write launch");
}

int paged_attention_decode(void* out, const void* query, const void* key_cache,
                           const void* value_cache, const int32_t* block_tables,
                           int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                           int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                           int num_blocks, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                           float k_scale, float v_scale, int partition_tokens,
                           const int32_t* partition_offsets, int total_partitions,
                           void* workspace, size_t workspace_bytes, void* stream) {
  DecodeCall c{out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
               num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
               q_dtype, cache_dtype, k_scale, v_scale, partition_tokens, partition_offsets,
               total_partitions, workspace, workspace_bytes};
  return decode_common(c, true, stream);
}

int paged_attention_decode_queue(void* out, const void* query, const void* key_cache,
                                 const void* value_cache, const int32_t* block_tables,
                                 int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                                 int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                 int num_blocks, float scale, pkv_dtype q_dtype,
                                 pkv_dtype cache_dtype, float k_scale, float v_scale,
                                 int partition_tokens, const int32_t* partition_offsets,
                                 int total_partitions, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  DecodeCall c{out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
               num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
               q_dtype, cache_dtype, k_scale, v_scale, partition_tokens, partition_offsets,
               total_partitions, workspace, workspace_bytes, true};
  return decode_common(c, true, stream);
}

int paged_attention_decode_partials(void* out, const void* query, const void* key_cache,
                                    const void* value_cache, const int32_t* block_tables,
                                    int max_blocks_per_seq, const int32_t* context_lens,
                                    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                    int block_size, int num_blocks, float scale, pkv_dtype q_dtype,
                                    pkv_dtype cache_dtype, float k_scale, float v_scale,
                                    int partition_tokens, const int32_t* partition_offsets,
                                    int total_partitions, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  if (partition_tokens <= 0) return fail(PKV_ERR_INVALID, "partition_tokens must be > 0");
  DecodeCall c{out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
               num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
               q_dtype, cache_dtype, k_scale, v_scale, partition_tokens, partition_offsets,
               total_partitions, workspace, workspace_bytes};
  return decode_common(c, false, stream);
}

int paged_attention_decode_step(void* out, const void* query, const void* new_key,
                                const void* new_value, void* key_cache, void* value_cache,
                                const int32_t* block_tables, int max_blocks_per_seq,
                                const int32_t* context_lens, int num_seqs, int num_q_heads,
                                int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                float k_scale, float v_scale, int partition_tokens,
                                const int32_t* partition_offsets, int total_partitions,
                                void* workspace, size_t workspace_bytes, void* stream) {
  DecodeCall c{out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
               num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
               q_dtype, cache_dtype, k_scale, v_scale, partition_tokens, partition_offsets,
               total_partitions, workspace, workspace_bytes};
  DecodeArgs a;
  int rc = check_decode(c, &a);
  if (rc) return rc;
  if (!new_key || !new_value) return fail(PKV_ERR_INVALID, "null pointer argument");
  if (num_seqs == 0) return PKV_OK;
  a.new_k = new_key;
  a.new_v = new_value;
  if (cache_dtype == PKV_FP8_E4M3) {
    a.k_inv = 1.f / k_scale;  // the same correctly rounded division as paged_kv_write
    a.v_inv = 1.f / v_scale;
  }
  if (decode_step_stores_in_kernel(a)) {
    rc = hip_status(launch_decode_step(a, stream), "paged_attention_decode_step launch");
  } else {
    // the slots of position context_lens[s] - 1 come from the tables, as in
    // the one-launch form
    rc = hip_status(launch_kv_write_tail(new_key, new_value, key_cache, value_cache, block_tables,
                                         max_blocks_per_seq, context_lens, num_seqs, num_kv_heads,
                                         head_dim, block_size, num_blocks, cache_dtype, a.k_inv,
                                         a.v_inv, stream),
                    "paged_attention_decode_step store launch");
    if (!rc) rc = hip_status(launch_decode(a, stream), "paged_attention_decode_step launch");
  }
  if (rc || partition_tokens == 0) return rc;
  return hip_status(launch_splitk_reduce(out, a.ws, partition_offsets, num_seqs, num_q_heads,
                                         head_dim, total_partitions, q_dtype, stream, 2,
                                         max_partitions(a.max_blocks, a.BS, a.partition)),
                    "paged_attention_splitk_reduce launch");
}

int paged_attention_decode_step_launches(int num_q_heads, int num_kv_heads, int head_dim,
                                         int block_size, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                         int partition_tokens) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
      partition_tokens < 0 || !valid_dtype(q_dtype) || !valid_dtype(cache_dtype))
    return fail(PKV_ERR_INVALID, "bad arguments");
  if (!decode_supported(q_dtype, cache_dtype, head_dim, block_size, num_q_heads / num_kv_heads))
    return fail(PKV_ERR_UNSUPPORTED, "unsupported decode shape");
  DecodeArgs a{};
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.D = head_dim;
  a.BS = block_size;
  a.partition = partition_tokens;
  a.q_dtype = q_dtype;
  a.kv_dtype = cache_dtype;
  clear_error();
  return (decode_step_stores_in_kernel(a) ? 1 : 2) + (partition_tokens > 0 ? 1 : 0);
}

static bool shape_args(int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                       pkv_dtype q_dtype, pkv_dtype cache_dtype, DecodeArgs* a) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
      !valid_dtype(q_dtype) || !valid_dtype(cache_dtype)) {
    fail(PKV_ERR_INVALID, "bad arguments");
    return false;
  }
  if (!decode_supported(q_dtype, cache_dtype, head_dim, block_size, num_q_heads / num_kv_heads)) {
    fail(PKV_ERR_UNSUPPORTED, "unsupported decode shape");
    return false;
  }
  *a = DecodeArgs{};
  a->Hq = num_q_heads;
  a->Hkv = num_kv_heads;
  a->D = head_dim;
  a->BS = block_size;
  a->q_dtype = q_dtype;
  a->kv_dtype = cache_dtype;
  return true;
}

int paged_attention_streamk_workers(int num_q_heads, int num_kv_heads, int head_dim,
                                    int block_size, pkv_dtype q_dtype, pkv_dtype cache_dtype) {
  DecodeArgs a;
  if (!shape_args(num_q_heads, num_kv_heads, head_dim, block_size, q_dtype, cache_dtype, &a))
    return PKV_ERR_INVALID;
  const int r = decode_sk_workers(a);
  if (r <= 0) return fail(PKV_ERR_HIP, "occupancy query failed");
  clear_error();
  return r;
}

static int streamk_common(const DecodeCall& c, const void* new_key, const void* new_value,
                          const int32_t* tile_offsets, int total_tiles, int workers,
                          bool reduce, void* stream) {
  DecodeArgs a;
  int rc = check_decode(c, &a);
  if (rc) return rc;
  const bool step = new_key || new_value;
  if (step && !(new_key && new_value)) return fail(PKV_ERR_INVALID, "null pointer argument");
  if (!tile_offsets || total_tiles < 0) return fail(PKV_ERR_INVALID, "bad tile offsets");
  if (workers <= 0) return fail(PKV_ERR_INVALID, "workers must be > 0");
  const size_t need = paged_attention_streamk_workspace_bytes(workers, c.num_seqs, c.num_q_heads,
                                                              c.num_kv_heads, c.head_dim);
  if (!c.workspace || c.workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, c.workspace_bytes);
  if (c.num_seqs == 0) return PKV_OK;
  a.ws = (float*)c.workspace;
  a.tile_off = tile_offsets;
  a.sk_cu = total_tiles;
  a.sk_workers = workers;
  if (step) {
    a.new_k = new_key;
    a.new_v = new_value;
    if (c.cache_dtype == PKV_FP8_E4M3) {
      a.k_inv = 1.f / c.k_scale;  // the same correctly rounded division as paged_kv_write
      a.v_inv = 1.f / c.v_scale;
    }
  }
  const bool store_in_kernel = step && decode_sk_heads_per_wave(a) == c.num_q_heads / c.num_kv_heads;
  if (step && !store_in_kernel) {
    rc = hip_status(launch_kv_write_tail(new_key, new_value, (void*)c.key_cache,
                                         (void*)c.value_cache, c.block_tables,
                                         c.max_blocks_per_seq, c.context_lens, c.num_seqs,
                                         c.num_kv_heads, c.head_dim, c.block_size, c.num_blocks,
                                         c.cache_dtype, a.k_inv, a.v_inv, stream),
                    "paged_attention_decode_step_streamk store launch");
    if (rc) return rc;
  }
  if (total_tiles > 0) {
    rc = hip_status(launch_decode_sk(a, store_in_kernel, stream), "stream-K decode launch");
    if (rc) return rc;
  }
  if (!reduce) return PKV_OK;
  return hip_status(launch_sk_reduce(a, stream), "stream-K reduce launch");
}

int paged_attention_decode_streamk(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   int max_blocks_per_seq, const int32_t* context_lens,
                                   const int32_t* tile_offsets, int total_tiles, int num_seqs,
                                   int num_q_heads, int num_kv_heads, int head_dim,
                                   int block_size, int num_blocks, float scale,
                                   pkv_dtype q_dtype, pkv_dtype cache_dtype, float k_scale,
                                   float v_scale, int workers, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  DecodeCall c{out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
               num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
               q_dtype, cache_dtype, k_scale, v_scale, 0, nullptr, 0, workspace, workspace_bytes};
  return streamk_common(c, nullptr, nullptr, tile_offsets, total_tiles, workers, true, stream);
}

int paged_attention_decode_streamk_partials(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* tile_offsets, int total_tiles, int num_seqs, int num_q_heads, int num_kv_heads,
    int head_dim, int block_size, int num_blocks, float scale, pkv_dtype q_dtype,
    pkv_dtype cache_dtype, float k_scale, float v_scale, int workers, void* workspace,
    size_t workspace_bytes, void* stream) {
  DecodeCall c{out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
               num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
               q_dtype, cache_dtype, k_scale, v_scale, 0, nullptr, 0, workspace, workspace_bytes};
  return streamk_common(c, nullptr, nullptr, tile_offsets, total_tiles, workers, false, stream);
}

int paged_attention_streamk_reduce(void* out, const void* workspace, size_t workspace_bytes,
                                   const int32_t* tile_offsets, int total_tiles, int num_seqs,
                                   int num_q_heads, int num_kv_heads, int head_dim,
                                   int block_size, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                   int workers, void* stream) {
  DecodeArgs a;
  if (!shape_args(num_q_heads, num_kv_heads, head_dim, block_size, q_dtype, cache_dtype, &a))
    return PKV_ERR_INVALID;
  if (!out || !workspace || !tile_offsets) return fail(PKV_ERR_INVALID, "null pointer argument");
  if (num_seqs < 0 || total_tiles < 0 || workers <= 0) return fail(PKV_ERR_INVALID, "bad sizes");
  const size_t need = paged_attention_streamk_workspace_bytes(workers, num_seqs, num_q_heads,
                                                              num_kv_heads, head_dim);
  if (workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  if (num_seqs == 0) return PKV_OK;
  a.out = out;
  a.ws = (float*)workspace;
  a.S = num_seqs;
  a.tile_off = tile_offsets;
  a.sk_cu = total_tiles;
  a.sk_workers = workers;
  return hip_status(launch_sk_reduce(a, stream), "stream-K reduce launch");
}

int paged_attention_decode_step_streamk(void* out, const void* query, const void* new_key,
                                        const void* new_value, void* key_cache, void* value_cache,
                                        const int32_t* block_tables, int max_blocks_per_seq,
                                        const int32_t* context_lens, const int32_t* tile_offsets,
                                        int total_tiles, int num_seqs, int num_q_heads,
                                        int num_kv_heads, int head_dim, int block_size,
                                        int num_blocks, float scale, pkv_dtype q_dtype,
                                        pkv_dtype cache_dtype, float k_scale, float v_scale,
                                        int workers, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  if (!new_key || !new_value) return fail(PKV_ERR_INVALID, "null pointer argument");
  DecodeCall c{out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
               num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
               q_dtype, cache_dtype, k_scale, v_scale, 0, nullptr, 0, workspace, workspace_bytes};
  return streamk_common(c, new_key, new_value, tile_offsets, total_tiles, workers, true, stream);
}

// The shared-prefix decode, and with new_key / new_value its decode step.
static int prefix_common(void* out, const void* query, const void* new_key,
                         const void* new_value, const void* key_cache, const void* value_cache,
                         const int32_t* block_tables, int max_blocks_per_seq,
                         const int32_t* context_lens, int num_seqs, int num_q_heads,
                         int num_kv_heads, int head_dim, int block_size, int num_blocks,
                         float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype, float k_scale,
                         float v_scale, int partition_tokens, const int32_t* group_offsets,
                         const int32_t* group_prefix_blocks, int num_groups,
                         const int32_t* row_offsets, const int32_t* suffix_offsets,
                         const int32_t* token_start, const int32_t* prefix_item_offsets,
                         int total_rows, int total_suffix_partitions, int total_prefix_items,
                         void* workspace, size_t workspace_bytes, bool step, void* stream) {
  if (partition_tokens <= 0) return fail(PKV_ERR_INVALID, "partition_tokens must be > 0");
  if (total_rows < num_seqs || total_suffix_partitions < 0 || total_prefix_items < 0 ||
      num_groups < 0)
    return fail(PKV_ERR_INVALID, "bad plan totals");
  if (!group_offsets || !group_prefix_blocks || !row_offsets || !suffix_offsets ||
      !token_start || !prefix_item_offsets)
    return fail(PKV_ERR_INVALID, "null pointer argument");
  if (step && (!new_key || !new_value)) return fail(PKV_ERR_INVALID, "null pointer argument");
  // validate as a split-K call over total_rows partial rows
  DecodeCall c{out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
               num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
               q_dtype, cache_dtype, k_scale, v_scale, partition_tokens, suffix_offsets,
               total_rows, workspace, workspace_bytes};
  DecodeArgs a;
  int rc = check_decode(c, &a);
  if (rc) return rc;
  if (!decode_prefix_supported(a))
    return fail(PKV_ERR_UNSUPPORTED, "shared-prefix decode needs bf16 q and cache, head_dim 128, "
                                     "block_size 16");
  if (num_seqs == 0) return PKV_OK;
  a.ws_rows = total_rows;
  PrefixArgs p;
  p.group_off = group_offsets;
  p.group_blocks = group_prefix_blocks;
  p.pre_off = prefix_item_offsets;
  p.row_off = row_offsets;
  p.suf_off = suffix_offsets;
  p.n_groups = num_groups;
  p.total_items = total_prefix_items;
  p.total_rows = total_rows;
  p.step = step ? 1 : 0;
  DecodeArgs b = a;   // the split-K pass over each sequence's own tokens
  b.part_off = suffix_offsets;
  b.total_parts = total_suffix_partitions;
  b.t_start = token_start;
  b.row_off = row_offsets;
  // decode step: the suffix wave that reads a sequence's last block stores
  // its new token, else a store launch goes first
  const bool in_kernel = step && total_suffix_partitions > 0 && decode_prefix_step_in_kernel(a);
  if (step) {
    b.new_k = new_key;
    b.new_v = new_value;
    if (!in_kernel) {
      rc = hip_status(launch_kv_write_tail(new_key, new_value, (void*)key_cache,
                                           (void*)value_cache, block_tables, max_blocks_per_seq,
                                           context_lens, num_seqs, num_kv_heads, head_dim,
                                           block_size, num_blocks, cache_dtype, 1.f, 1.f, stream,
                                           token_start),
                      "shared-prefix decode step store launch");
      if (rc) return rc;
    }
  }
  if (total_suffix_partitions > 0) {
    // the prefix pass and the split-K pass over each sequence's own tokens
    // in one launch (they write disjoint partial rows)
    rc = hip_status(launch_decode_prefix_fused(a, b, p, stream, in_kernel),
                    "shared-prefix decode launch");
  } else {
    rc = hip_status(launch_decode_prefix(a, p, stream), "shared-prefix decode launch");
  }
  if (rc) return rc;
  return hip_status(launch_splitk_reduce(out, a.ws, row_offsets, num_seqs, num_q_heads, head_dim,
                                         total_rows, q_dtype, stream, 1),
                    "shared-prefix reduce launch");
}

int paged_attention_decode_prefix(void* out, const void* query, const void* key_cache,
                                  const void* value_cache, const int32_t* block_tables,
                                  int max_blocks_per_seq, const int32_t* context_lens,
                                  int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                  int block_size, int num_blocks, float scale, pkv_dtype q_dtype,
                                  pkv_dtype cache_dtype, float k_scale, float v_scale,
                                  int partition_tokens, const int32_t* group_offsets,
                                  const int32_t* group_prefix_blocks, int num_groups,
                                  const int32_t* row_offsets, const int32_t* suffix_offsets,
                                  const int32_t* token_start, const int32_t* prefix_item_offsets,
                                  int total_rows, int total_suffix_partitions,
                                  int total_prefix_items, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return prefix_common(out, query, nullptr, nullptr, key_cache, value_cache, block_tables,
                       max_blocks_per_seq, context_lens, num_seqs, num_q_heads, num_kv_heads,
                       head_dim, block_size, num_blocks, scale, q_dtype, cache_dtype, k_scale,
                       v_scale, partition_tokens, group_offsets, group_prefix_blocks, num_groups,
                       row_offsets, suffix_offsets, token_start, prefix_item_offsets, total_rows,
                       total_suffix_partitions, total_prefix_items, workspace, workspace_bytes,
                       false, stream);
}

int paged_attention_decode_prefix_step(
    void* out, const void* query, const void* new_key, const void* new_value, void* key_cache,
    void* value_cache, const int32_t* block_tables, int max_blocks_per_seq,
    const int32_t* context_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
    int block_size, int num_blocks, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
    float k_scale, float v_scale, int partition_tokens, const int32_t* group_offsets,
    const int32_t* group_prefix_blocks, int num_groups, const int32_t* row_offsets,
    const int32_t* suffix_offsets, const int32_t* token_start, const int32_t* prefix_item_offsets,
    int total_rows, int total_suffix_partitions, int total_prefix_items, void* workspace,
    size_t workspace_bytes, void* stream) {
  return prefix_common(out, query, new_key, new_value, key_cache, value_cache, block_tables,
                       max_blocks_per_seq, context_lens, num_seqs, num_q_heads, num_kv_heads,
                       head_dim, block_size, num_blocks, scale, q_dtype, cache_dtype, k_scale,
                       v_scale, partition_tokens, group_offsets, group_prefix_blocks, num_groups,
                       row_offsets, suffix_offsets, token_start, prefix_item_offsets, total_rows,
                       total_suffix_partitions, total_prefix_items, workspace, workspace_bytes,
                       true, stream);
}

int paged_attention_prefill(void* out, const void* query, const void* key_cache,
                            const void* value_cache, const int32_t* block_tables,
                            int max_blocks_per_seq, const int32_t* context_lens,
                            const int32_t* query_start, int num_seqs, int max_query_len,
                            int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                            int num_blocks, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                            float k_scale, float v_scale, void* stream) {
  (void)k_scale;
  (void)v_scale;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens ||
      !query_start)
    return fail(PKV_ERR_INVALID, "null pointer argument");
  if (num_seqs < 0 || max_query_len < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0)
    return fail(PKV_ERR_INVALID, "bad sizes");
  if (num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "num_q_heads %% num_kv_heads != 0");
  if (!valid_dtype(q_dtype) || !valid_dtype(cache_dtype)) return fail(PKV_ERR_INVALID, "unknown dtype");
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID, "scale must be finite");
  if (!prefill_supported(q_dtype, cache_dtype, head_dim, block_size))
    return fail(PKV_ERR_UNSUPPORTED, "prefill needs bf16 query and cache, head_dim 128, "
                                     "block_size 16");
  const int G = num_q_heads / num_kv_heads;
  const long long qblocks = prefill_query_blocks(max_query_len, G);
  const long long total = qblocks * num_kv_heads * (long long)num_seqs;
  if (total > (long long)INT32_MAX - 8) return fail(PKV_ERR_INVALID, "too many query blocks");
  if ((long long)max_blocks_per_seq * block_size > (long long)INT32_MAX)
    return fail(PKV_ERR_INVALID, "max_blocks_per_seq * block_size exceeds int32");
  if (num_seqs == 0 || max_query_len == 0) {
    clear_error();
    return PKV_OK;
  }
  PrefillArgs a;
  a.out = out;
  a.q = query;
  a.kc = key_cache;
  a.vc = value_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.q_start = query_start;
  a.S = num_seqs;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.nb = num_blocks;
  a.qblocks = (int)qblocks;
  a.total_wg = (int)total;
  a.qk_mult = scale * kLog2eHost;
  return hip_status(launch_prefill(a, stream), "prefill launch");
}

int paged_attention_splitk_reduce(void* out, const void* workspace, size_t workspace_bytes,
                                  const int32_t* partition_offsets, int num_seqs,
                                  int num_q_heads, int head_dim, int total_partitions,
                                  int max_partitions_per_seq, pkv_dtype out_dtype, void* stream) {
  if (!out || !workspace || !partition_offsets) return fail(PKV_ERR_INVALID, "null pointer argument");
  if (num_seqs < 0 || num_q_heads <= 0 || total_partitions < num_seqs)
    return fail(PKV_ERR_INVALID, "bad sizes");
  if (head_dim != 64 && head_dim != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim must be 64/128");
  if (out_dtype != PKV_F32 && out_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "output dtype must be F32 or BF16");
  const size_t need = paged_attention_workspace_bytes(total_partitions, num_q_heads, head_dim);
  if (workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  if (num_seqs == 0) return PKV_OK;
  return hip_status(launch_splitk_reduce(out, (const float*)workspace, partition_offsets, num_seqs,
                                         num_q_heads, head_dim, total_partitions, out_dtype, stream,
                                         2, max_partitions_per_seq),
                    "paged_attention_splitk_reduce launch");
}

int paged_kv_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs, int num_pairs,
                         size_t block_bytes, int num_blocks, void* stream) {
  if (num_pairs < 0 || num_blocks <= 0) return fail(PKV_ERR_INVALID, "bad sizes");
  if (num_pairs == 0) return PKV_OK;
  if (!key_cache || !value_cache || !pairs) return fail(PKV_ERR_INVALID, "null pointer argument");
  if (block_bytes == 0 || block_bytes % 16 != 0)
    return fail(PKV_ERR_INVALID, "block_bytes must be a positive multiple of 16");
  return hip_status(launch_copy_blocks(key_cache, value_cache, pairs, num_pairs, block_bytes,
                                       num_blocks, stream),
                    "paged_kv_copy_blocks launch");
}

int paged_kv_swap_blocks(void* dst_key_cache, void* dst_value_cache, const void* src_key_cache,
                         const void* src_value_cache, const int32_t* pairs, int num_pairs,
                         size_t block_bytes, int src_blocks, int dst_blocks, void* stream) {
  if (num_pairs < 0 || src_blocks <= 0 || dst_blocks <= 0) return fail(PKV_ERR_INVALID, "bad sizes");
  if (num_pairs == 0) {
    clear_error();
    return PKV_OK;
  }
  if (!dst_key_cache || !dst_value_cache || !src_key_cache || !src_value_cache || !pairs)
    return fail(PKV_ERR_INVALID, "null pointer argument");
  if (block_bytes == 0 || block_bytes % 16 != 0)
    return fail(PKV_ERR_INVALID, "block_bytes must be a positive multiple of 16");
  return hip_status(launch_swap_blocks(dst_key_cache, dst_value_cache, src_key_cache,
                                       src_value_cache, pairs, num_pairs, block_bytes, src_blocks,
                                       dst_blocks, stream),
                    "paged_kv_swap_blocks launch");
}

int paged_kv_swap_blocks_memcpy(void* dst_key_cache, void* dst_value_cache,
                             const void* src_key_cache, const void* src_value_cache,
                             const int32_t* pairs_host, int num_pairs, size_t block_bytes,
                             int src_blocks, int dst_blocks, void* stream) {
  if (num_pairs < 0 || src_blocks <= 0 || dst_blocks <= 0) return fail(PKV_ERR_INVALID, "bad sizes");
  if (num_pairs == 0) {
    clear_error();
    return PKV_OK;
  }
  if (!dst_key_cache || !dst_value_cache || !src_key_cache || !src_value_cache || !pairs_host)
    return fail(PKV_ERR_INVALID, "null pointer argument");
  if (block_bytes == 0 || block_bytes % 16 != 0)
    return fail(PKV_ERR_INVALID, "block_bytes must be a positive multiple of 16");
  hipStream_t st = (hipStream_t)stream;
  // runs of pairs whose source and destination ids both step by one: one
  // copy per run and pool
  int i = 0;
  while (i < num_pairs) {
    const int s0 = pairs_host[2 * i], d0 = pairs_host[2 * i + 1];
    if ((unsigned)s0 >= (unsigned)src_blocks || (unsigned)d0 >= (unsigned)dst_blocks) {
      ++i;
      continue;
    }
    int n = 1;
    while (i + n < num_pairs && pairs_host[2 * (i + n)] == s0 + n &&
           pairs_host[2 * (i + n) + 1] == d0 + n && s0 + n < src_blocks && d0 + n < dst_blocks)
      ++n;
    const size_t off_s = (size_t)s0 * block_bytes, off_d = (size_t)d0 * block_bytes;
    const size_t bytes = (size_t)n * block_bytes;
    int rc = hip_status(hipMemcpyAsync((uint8_t*)dst_key_cache + off_d,
                                       (const uint8_t*)src_key_cache + off_s, bytes,
                                       hipMemcpyDefault, st),
                        "paged_kv_swap_blocks_memcpy copy");
    if (!rc)
      rc = hip_status(hipMemcpyAsync((uint8_t*)dst_value_cache + off_d,
                                     (const uint8_t*)src_value_cache + off_s, bytes,
                                     hipMemcpyDefault, st),
                      "paged_kv_swap_blocks_memcpy copy");
    if (rc) return rc;
    i += n;
  }
  clear_error();
  return PKV_OK;
}

int pkv_paged_read_probe(const void* key_cache, const void* value_cache,
                         const int32_t* block_tables, int max_blocks_per_seq,
                         const int32_t* context_lens, int num_seqs, int num_q_heads,
                         int num_kv_heads, int head_dim, int block_size, int num_blocks,
                         pkv_dtype q_dtype, pkv_dtype cache_dtype, int partition_tokens,
                         const int32_t* partition_offsets, int total_partitions, void* sink,
                         void* stream) {
  // the decode's checks, with the sink standing in for the buffers the
  // probe does not touch (query, output, workspace)
  DecodeCall c{sink, sink, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
               num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, 1.f,
               q_dtype, cache_dtype, 1.f, 1.f, partition_tokens, partition_offsets,
               total_partitions, sink, (size_t)-1};
  if (partition_tokens <= 0) return fail(PKV_ERR_INVALID, "partition_tokens must be > 0");
  if (!sink || (uintptr_t)sink % 16 != 0) return fail(PKV_ERR_INVALID, "sink must be 16-byte aligned");
  DecodeArgs a;
  const int rc = check_decode(c, &a);
  if (rc) return rc;
  if (num_seqs == 0) return PKV_OK;
  return hip_status(launch_paged_read_probe(a, (uint32_t*)sink, stream), "pkv_paged_read_probe launch");
}

int pkv_host_device_pointer(const void* host, void** device_out) {
  if (!host || !device_out) return fail(PKV_ERR_INVALID, "null pointer argument");
  void* d = nullptr;
  const int rc = hip_status(hipHostGetDevicePointer(&d, const_cast<void*>(host), 0),
                            "hipHostGetDevicePointer (is the memory pinned?)");
  if (rc) return rc;
  if (!d) return fail(PKV_ERR_HIP, "hipHostGetDevicePointer returned null");
  *device_out = d;
  return PKV_OK;
}

int paged_kv_gather(void* k_out, void* v_out, const void* key_cache, const void* value_cache,
                    const int32_t* block_tables, int max_blocks_per_seq, const int32_t* cu_ctx,
                    int num_seqs, int total_tokens, int num_kv_heads, int head_dim, int block_size,
                    int num_blocks, pkv_dtype cache_dtype, void* stream) {
  if (num_seqs < 0 || total_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0)
    return fail(PKV_ERR_INVALID, "bad sizes");
  if (total_tokens == 0 || num_seqs == 0) return PKV_OK;
  if (!k_out || !v_out || !key_cache || !value_cache || !block_tables || !cu_ctx)
    return fail(PKV_ERR_INVALID, "null pointer argument");
  if (!valid_dtype(cache_dtype)) return fail(PKV_ERR_INVALID, "unknown dtype");
  if ((head_dim != 64 && head_dim != 128) || (block_size != 16 && block_size != 32))
    return fail(PKV_ERR_UNSUPPORTED, "head_dim must be 64/128 and block_size 16/32");
  return hip_status(launch_gather(k_out, v_out, key_cache, value_cache, block_tables,
                                  max_blocks_per_seq, cu_ctx, num_seqs, total_tokens, num_kv_heads,
                                  head_dim, block_size, num_blocks, cache_dtype, stream),
                    "paged_kv_gather launch");
}

int pkv_hbm_read_probe(const void* buffer, size_t bytes, void* sink, int workgroups,
                       void* stream) {
  if (!buffer || !sink || bytes < 16 || workgroups <= 0)
    return fail(PKV_ERR_INVALID, "bad arguments");
  return hip_status(launch_read_probe(buffer, bytes, sink, workgroups, stream),
                    "pkv_hbm_read_probe launch");
}

}  // extern "C"
