// Internal declarations shared by the host-side translation units of libpkv.
#pragma once

#include <algorithm>
#include <cstddef>
#include <cstdint>

#include "pkv.h"

namespace pkv {

// Records a thread-local error message and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

constexpr float kLog2eHost = 1.4426950408889634f;

inline int elem_bytes(pkv_dtype t) { return t == PKV_F32 ? 4 : t == PKV_BF16 ? 2 : 1; }

// Everything the decode kernels need, resolved on the host.
struct DecodeArgs {
  void* out;
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* tables;
  const int32_t* lens;
  const int32_t* part_off;  // null in one-pass mode
  float* ws;                // partial outputs [total_parts][Hq][D] then (m, l) [total_parts][Hq][2]
  int max_blocks;
  int S, Hq, Hkv, D, BS, nb;
  int partition;            // tokens; 0 = one pass
  int total_parts;
  float qk_mult;            // scale * k_scale * log2(e): scores in the log2 domain
  float v_mult;             // v_scale for fp8, else 1
  pkv_dtype q_dtype, kv_dtype;
  // Decode step (paged_attention_decode_step): row s of new_k / new_v is the
  // new token of sequence s (position lens[s] - 1), stored by the workgroup
  // that reads the sequence's last block.  Null otherwise.
  const void* new_k = nullptr;
  const void* new_v = nullptr;
  float k_inv = 1.f, v_inv = 1.f;
  // Stream-K schedule: tile_off [S+1] prefix sums of ceil(lens/BS) (device),
  // sk_cu = tile_off[S] (host copy), sk_workers = waves launched.
  const int32_t* tile_off = nullptr;
  int sk_cu = 0, sk_workers = 0;
  // Shared-prefix decode (suffix pass): sequence s's own tokens start at
  // t_start[s] (device), its split-K partitions are part_off rows (suffix
  // numbering), written as partial rows row_off[s] + part.  Null otherwise.
  const int32_t* t_start = nullptr;
  const int32_t* row_off = nullptr;
  int ws_rows = 0;   // partial rows of the workspace when not total_parts
  // Work-counter split-K launches: a number unique to the launch, which tags
  // the counter in the workspace's last bytes (after the partials).
  unsigned long long epoch = 0;
};

// Bytes after the split-K partials in a workspace: the work counter of the
// work-counter decode (one 64-bit word, padded).
constexpr size_t kWorkspaceTail = 256;

// The arguments of a decode entry point, as the C ABI receives them.
struct DecodeCall {
  void* out;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* context_lens;
  int num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks;
  float scale;
  pkv_dtype q_dtype, cache_dtype;
  float k_scale, v_scale;
  int partition_tokens;
  const int32_t* partition_offsets;
  int total_partitions;
  void* workspace;
  size_t workspace_bytes;
  bool queue = false;   // paged_attention_decode_queue: the work-counter schedule
};

// paged_attention_decode's checks and launches (api.cpp): the decode
// kernel, then (reduce, partition_tokens > 0) the split-K reduce.
int decode_common(const DecodeCall& c, bool reduce, void* stream);

// Shared-prefix decode: groups of consecutive sequences (group_off[g] ..
// group_off[g+1]) share their first group_blocks[g] blocks; prefix work items
// (waves) of group g are pre_off[g] .. pre_off[g+1]; per sequence, rows
// row_off[s] .. row_off[s+1] hold its suffix partitions (suf_off numbering)
// then one prefix piece of kPrefixPieceBlocks blocks each.  All device.
constexpr int kPrefixPieceBlocks = 8;
struct PrefixArgs {
  const int32_t* group_off = nullptr;
  const int32_t* group_blocks = nullptr;
  const int32_t* pre_off = nullptr;
  const int32_t* row_off = nullptr;
  const int32_t* suf_off = nullptr;
  int n_groups = 0, total_items = 0, total_rows = 0;
  // decode step: members whose new token lies in the shared blocks
  // (lens <= group_blocks * BS) get NaN rows
  int step = 0;
};

// Chunked prefill (prefill.hip): sequence s owns query rows q_start[s] ..
// q_start[s+1]-1, its last C positions; qblocks workgroups per (sequence, kv
// head) cover up to qblocks * 128 (position, head) rows; total_wg = S * Hkv *
// qblocks.  Pointers are device pointers.
struct PrefillArgs {
  void* out = nullptr;
  const void* q = nullptr;
  const void* kc = nullptr;
  const void* vc = nullptr;
  const int32_t* tables = nullptr;
  const int32_t* lens = nullptr;
  const int32_t* q_start = nullptr;
  int S = 0, Hq = 0, Hkv = 0, max_blocks = 0, nb = 0;
  int qblocks = 0, total_wg = 0;
  float qk_mult = 0.f;   // scale * log2(e)
};

// Kernel launchers (decode.hip, kv_ops.hip).  Return hipError_t as int.
int launch_decode(const DecodeArgs& a, void* stream);
// Decode step (decode.hip): whether the decode launch itself can store the
// new tokens (one workgroup -- one wave on the matrix-core path -- per kv
// head and partition), and that launch; otherwise the caller stores them
// with launch_kv_write_tail first.
bool decode_step_stores_in_kernel(const DecodeArgs& a);
int launch_decode_step(const DecodeArgs& a, void* stream);
// Stream-K decode (decode.hip): resident waves for this shape on the current
// device (< 0 on error), the decode launch (store: also the decode step's
// new-token store, when decode_step_stores_in_kernel) and its reduce.
int decode_sk_workers(const DecodeArgs& a);
int decode_sk_heads_per_wave(const DecodeArgs& a);
int launch_decode_sk(const DecodeArgs& a, bool store, void* stream);
int launch_sk_reduce(const DecodeArgs& a, void* stream);
// Shared-prefix decode (decode_prefix.hip): bf16 query and cache, head_dim
// 128, block size 16.
bool decode_prefix_supported(const DecodeArgs& a);
// whether the suffix pass has one wave per (sequence, kv head, partition), so
// that the decode step can store the new tokens inside the launch
bool decode_prefix_step_in_kernel(const DecodeArgs& a);
int launch_decode_prefix(const DecodeArgs& a, const PrefixArgs& p, void* stream);
// the prefix pass (a) and the suffix split-K pass (b) in one launch; store:
// the decode step's new-token store (b.new_k / b.new_v), only where
// decode_prefix_step_in_kernel
int launch_decode_prefix_fused(const DecodeArgs& a, const DecodeArgs& b, const PrefixArgs& p,
                               void* stream, bool store = false);
int launch_swap_blocks(void* dk, void* dv, const void* sk, const void* sv, const int32_t* pairs,
                       int n, size_t block_bytes, int src_nb, int dst_nb, void* stream);
bool prefill_supported(pkv_dtype q, pkv_dtype kv, int D, int BS);
int prefill_query_blocks(int max_query_len, int G);
int launch_prefill(const PrefillArgs& a, void* stream);
// Matrix-core decode for fp8 key/value tiles with query heads in groups of 8
// (decode_mfma.hip); launch_decode routes eligible calls there.
bool decode_mfma_eligible(const DecodeArgs& a);
int launch_decode_mfma(const DecodeArgs& a, void* stream, bool store = false);
// Paged read probe (paged_probe.hip): the split-K decode's reads for this
// shape (vector-ALU kernel, or the matrix-core kernel's through
// launch_paged_read_probe_mfma in decode_mfma.hip), no arithmetic; at most
// one word stored to sink.
int launch_paged_read_probe(const DecodeArgs& a, uint32_t* sink, void* stream);
int launch_paged_read_probe_mfma(const DecodeArgs& a, uint32_t* sink, void* stream);
// The work-counter split-K schedule (fp8 matrix-core shape only): whether a
// call qualifies, and its launch.
bool decode_queue_supported(const DecodeArgs& a);
int launch_decode_mfma_queue(const DecodeArgs& a, void* stream);
int launch_decode_mfma_sk(const DecodeArgs& a, void* stream, bool store);
int decode_mfma_sk_workers();
// min_parts: sequences with fewer rows are left alone (2 for split-K, whose
// single-partition sequences write their output directly; 1 when every
// sequence has partials only).  max_rows: an upper bound on one sequence's
// rows (0 = small); past four per piece lane the kernel that holds more rows
// in flight is launched (either kernel is correct for any count).
int launch_splitk_reduce(void* out, const float* ws, const int32_t* part_off, int S, int Hq, int D,
                         int total_parts, pkv_dtype out_dtype, void* stream, int min_parts = 2,
                         int max_rows = 0);
// Upper bound on the split-K partitions of one sequence whose table holds
// max_blocks blocks of bs tokens.
inline int max_partitions(int max_blocks, int bs, int partition) {
  if (partition <= 0) return 1;
  const long long t = (long long)max_blocks * bs;
  return (int)std::min<long long>((t + partition - 1) / partition, 1 << 30);
}
bool decode_supported(pkv_dtype q, pkv_dtype kv, int D, int BS, int G);

int launch_kv_write(const void* key, const void* value, void* kc, void* vc, const int32_t* slots,
                    int T, int H, int D, int BS, int nb, pkv_dtype src, pkv_dtype cache,
                    float k_inv, float v_inv, void* stream);
// t_start (device, optional): sequence s is skipped when lens[s] <= t_start[s]
int launch_kv_write_tail(const void* key, const void* value, void* kc, void* vc,
                         const int32_t* tables, int max_blocks, const int32_t* lens, int S, int H,
                         int D, int BS, int nb, pkv_dtype cache, float k_inv, float v_inv,
                         void* stream, const int32_t* t_start = nullptr);
int launch_copy_blocks(void* kc, void* vc, const int32_t* pairs, int n, size_t block_bytes,
                       int nb, void* stream);
int launch_read_probe(const void* src, size_t bytes, void* sink, int blocks, void* stream);
int launch_gather(void* k_out, void* v_out, const void* kc, const void* vc, const int32_t* tables,
                  int max_blocks, const int32_t* cu_ctx, int S, int T, int H, int D, int BS,
                  int nb, pkv_dtype cache, void* stream);

}  // namespace pkv
