// Host-only parts of the C ABI of libpkv: the thread-local error message,
// split-K partition offsets, stream-K tile offsets, workspace sizes and the
// shared-prefix plan.  Nothing here touches a device, so this file builds
// with a plain C++ compiler too (the sanitizer build of the host code uses
// it with the block allocator).

#include <cstdarg>
#include <cstdio>

#include "pkv.h"
#include "pkv_internal.h"

namespace pkv {

static thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = 0; }

}  // namespace pkv

using namespace pkv;

extern "C" {

const char* pkv_last_error(void) { return g_err; }

int pkv_abi_version(void) { return PKV_ABI_VERSION; }

int paged_attention_partition_offsets(const int32_t* context_lens_host, int num_seqs,
                                      int partition_tokens, int32_t* offsets_host_out,
                                      int* total_partitions_out) {
  if (num_seqs < 0 || partition_tokens <= 0 || !offsets_host_out || (num_seqs > 0 && !context_lens_host))
    return fail(PKV_ERR_INVALID, "bad arguments");
  int64_t acc = 0;
  offsets_host_out[0] = 0;
  for (int s = 0; s < num_seqs; ++s) {
    const int64_t L = context_lens_host[s];
    if (L < 0) return fail(PKV_ERR_INVALID, "negative context length at %d", s);
    const int64_t n = L == 0 ? 1 : (L + partition_tokens - 1) / partition_tokens;
    acc += n;
    if (acc > INT32_MAX) return fail(PKV_ERR_INVALID, "too many partitions");
    offsets_host_out[s + 1] = (int32_t)acc;
  }
  if (total_partitions_out) *total_partitions_out = (int)acc;
  return PKV_OK;
}

size_t paged_attention_workspace_bytes(int total_partitions, int num_q_heads, int head_dim) {
  if (total_partitions <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  return (size_t)total_partitions * num_q_heads * (head_dim + 2) * sizeof(float) + kWorkspaceTail;
}

int paged_attention_tile_offsets(const int32_t* context_lens_host, int num_seqs, int block_size,
                                 int32_t* offsets_host_out, int* total_tiles_out) {
  if (num_seqs < 0 || block_size <= 0 || !offsets_host_out || (num_seqs > 0 && !context_lens_host))
    return fail(PKV_ERR_INVALID, "bad arguments");
  int64_t acc = 0;
  offsets_host_out[0] = 0;
  for (int s = 0; s < num_seqs; ++s) {
    const int64_t L = context_lens_host[s];
    if (L < 0) return fail(PKV_ERR_INVALID, "negative context length at %d", s);
    acc += (L + block_size - 1) / block_size;
    if (acc > INT32_MAX) return fail(PKV_ERR_INVALID, "too many tiles");
    offsets_host_out[s + 1] = (int32_t)acc;
  }
  if (total_tiles_out) *total_tiles_out = (int)acc;
  clear_error();
  return PKV_OK;
}

size_t paged_attention_streamk_workspace_bytes(int workers, int num_seqs, int num_q_heads,
                                               int num_kv_heads, int head_dim) {
  if (workers <= 0 || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_q_heads % num_kv_heads != 0)
    return 0;
  const size_t G = (size_t)(num_q_heads / num_kv_heads);
  return ((size_t)workers * G + (size_t)num_seqs * num_q_heads) * (head_dim + 2) * sizeof(float);
}

int paged_attention_prefix_plan(const int32_t* context_lens_host, int num_seqs,
                                const int32_t* group_offsets_host,
                                const int32_t* group_prefix_blocks_host, int num_groups,
                                int block_size, int partition_tokens, int num_q_heads,
                                int num_kv_heads, int32_t* row_offsets_out,
                                int32_t* suffix_offsets_out, int32_t* token_start_out,
                                int32_t* prefix_item_offsets_out, int32_t* totals_out) {
  if (num_seqs < 0 || num_groups < 0 || block_size <= 0 || partition_tokens <= 0 ||
      partition_tokens % block_size != 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || !row_offsets_out || !suffix_offsets_out ||
      !prefix_item_offsets_out || !totals_out || (num_seqs > 0 && (!context_lens_host || !token_start_out)) ||
      !group_offsets_host || (num_groups > 0 && !group_prefix_blocks_host))
    return fail(PKV_ERR_INVALID, "bad arguments");
  if (group_offsets_host[0] != 0 || group_offsets_host[num_groups] != num_seqs)
    return fail(PKV_ERR_INVALID, "group offsets must run from 0 to num_seqs");
  const int G = num_q_heads / num_kv_heads;
  int64_t rows = 0, suf = 0, items = 0;
  row_offsets_out[0] = 0;
  suffix_offsets_out[0] = 0;
  prefix_item_offsets_out[0] = 0;
  for (int g = 0; g < num_groups; ++g) {
    const int a0 = group_offsets_host[g], a1 = group_offsets_host[g + 1];
    const int pb = group_prefix_blocks_host[g];
    if (a1 < a0 || pb < 0) return fail(PKV_ERR_INVALID, "bad group %d", g);
    const int64_t pt = (int64_t)pb * block_size;
    const int npre = (pb + kPrefixPieceBlocks - 1) / kPrefixPieceBlocks;
    for (int s = a0; s < a1; ++s) {
      const int64_t L = context_lens_host[s];
      if (L < pt) return fail(PKV_ERR_INVALID, "sequence %d is shorter than its group's prefix", s);
      int64_t nsuf = (L - pt + partition_tokens - 1) / partition_tokens;
      if (nsuf + npre == 0) nsuf = 1;   // an empty sequence still gets its (zero) row
      suf += nsuf;
      rows += nsuf + npre;
      if (rows > INT32_MAX) return fail(PKV_ERR_INVALID, "too many rows");
      suffix_offsets_out[s + 1] = (int32_t)suf;
      row_offsets_out[s + 1] = (int32_t)rows;
      token_start_out[s] = (int32_t)pt;
    }
    const int64_t rb = ((int64_t)(a1 - a0) * G + 31) / 32;
    items += (int64_t)num_kv_heads * rb * npre;
    if (items > INT32_MAX) return fail(PKV_ERR_INVALID, "too many prefix items");
    prefix_item_offsets_out[g + 1] = (int32_t)items;
  }
  totals_out[0] = (int32_t)rows;
  totals_out[1] = (int32_t)suf;
  totals_out[2] = (int32_t)items;
  clear_error();
  return PKV_OK;
}

}  // extern "C"
