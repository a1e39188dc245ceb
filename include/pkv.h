/* pkv.h -- PagedAttention decode for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpkv.so.  The library computes single-query attention for many
 * sequences at once over a key/value cache that lives in fixed-size blocks
 * scattered through device memory and reached only through a per-sequence
 * block table, plus the scatter of each decode step's new key/value token
 * into the slot the block manager handed out, and a host-side block manager
 * with shared prefix blocks.
 *
 * Sources: "Day 6/90 of Inference Engineering" (PagedAttention notes: blocks
 * handed out one at a time, fill before allocate, prefix sharing, block
 * table); "PagedAttention Kernel：大模型推理优化的显存管理革新" §1 (fixed-size
 * pages scattered through device memory), §2.2 (coalesced access, prefetch of
 * the next page), §3.1 (QK^T per block, softmax, PV accumulated block by
 * block), §3.2 (balancing uneven work), §6 (fp32 accumulation).
 *
 * Conventions shared by every device entry point
 * ----------------------------------------------
 *  - Every pointer argument of a device entry point is a DEVICE pointer
 *    owned by the caller.  The library never allocates, frees or copies
 *    device memory and never synchronises; all work is enqueued on `stream`
 *    (a hipStream_t passed as void*; NULL = the null stream).
 *  - Return value: PKV_OK (0) or a negative PKV_ERR_* code; on error nothing
 *    has been enqueued and pkv_last_error() returns a message (thread-local).
 *  - Only arguments visible on the host are checked (null pointers, sizes,
 *    supported dtype / head_dim / block_size combinations, workspace size).
 *    Device contents (block ids, lengths, slots) are trusted; a kernel that
 *    meets a block id outside [0, num_blocks) or a length beyond the table
 *    width skips the offending data and writes NaN for that sequence's heads
 *    instead of reading out of bounds.
 *  - Element types: PKV_F32 (fp32), PKV_BF16 (bfloat16), PKV_FP8_E4M3 (OCP
 *    E4M3FN, stored as one byte).  Supported (query, cache) pairs:
 *    (F32, F32), (BF16, BF16), (BF16, FP8_E4M3).  head_dim is 64 or 128,
 *    block_size 16 or 32.
 *
 * Block pool layout (one pool for keys, one for values)
 * ------------------------------------------------------
 *  x = 16 / sizeof(element)            (4 fp32, 8 bf16, 16 fp8)
 *  key_cache   [num_blocks][num_kv_heads][head_dim / x][block_size][x]
 *  value_cache [num_blocks][num_kv_heads][head_dim][block_size]
 *  Token position t of sequence s lives in block block_tables[s][t / bs] at
 *  slot t % bs; a slot id is block * block_size + slot.  One (block, kv head)
 *  tile of each pool is block_size*head_dim*sizeof(element) contiguous bytes.
 *
 *  Query, output and new-token rows are dense row-major:
 *  query/out [num_seqs][num_q_heads][head_dim]; key/value
 *  [num_tokens][num_kv_heads][head_dim].  Query head g reads kv head
 *  g / (num_q_heads / num_kv_heads).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2 } pkv_dtype;

enum {
  PKV_OK = 0,
  PKV_ERR_INVALID = -1,     /* bad argument (null pointer, size, combination)   */
  PKV_ERR_UNSUPPORTED = -2, /* valid but not built (dtype, head_dim, block_size) */
  PKV_ERR_WORKSPACE = -3,   /* workspace missing or too small                   */
  PKV_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed       */
  PKV_ERR_NO_BLOCKS = -5,   /* allocator: not enough free blocks                */
  PKV_ERR_SEQ = -6          /* allocator: unknown or duplicate sequence id      */
};

/* Message for the last error returned on this thread ("" if none). */
const char* pkv_last_error(void);

/* ABI version of this header (bumped on incompatible change). */
int pkv_abi_version(void);
#define PKV_ABI_VERSION 2

/* ---------------------------------------------------------------------------
 * paged_kv_write -- scatter new key/value rows into their slots.
 * Each step's new token goes wherever the block manager put it ("Day 6/90 of
 * Inference Engineering", PagedAttention notes).
 *
 *  key, value     [num_tokens][num_kv_heads][head_dim] of src_dtype (device)
 *  key_cache,
 *  value_cache    block pools of cache_dtype in the layout above (device)
 *  slot_mapping   [num_tokens] int32 (device); token i goes to slot
 *                 slot_mapping[i]; a negative slot skips the token, and so
 *                 does a slot >= num_blocks * block_size.
 *  src/cache      (F32 -> F32) and (BF16 -> BF16) copy bits; (BF16 -> FP8)
 *                 stores E4M3FN(fp32(x) * fp32(1 / scale)) rounded to nearest
 *                 even and saturated to +-448 (NaN -> 0x7F), with
 *                 scale = k_scale for keys and v_scale for values (the
 *                 dequantisation multipliers; ignored unless cache is FP8).
 *  Two tokens mapped to the same slot race (the result is one of them).
 * ------------------------------------------------------------------------- */
int paged_kv_write(const void* key, const void* value, void* key_cache, void* value_cache,
                   const int32_t* slot_mapping, int num_tokens, int num_kv_heads, int head_dim,
                   int block_size, int num_blocks, pkv_dtype src_dtype, pkv_dtype cache_dtype,
                   float k_scale, float v_scale, void* stream);

/* ---------------------------------------------------------------------------
 * Split-K partitions ("PagedAttention Kernel：大模型推理优化的显存管理革新"
 * §3.2: sequences of very different lengths leave compute units idle unless
 * the work is cut into balanced pieces; here a long sequence's blocks are cut
 * into partitions that separate workgroups decode, and a reduce combines
 * them).  With partition_tokens = P > 0, sequence s is cut into
 * n_s = max(1, ceil(context_lens[s] / P)) partitions of logical tokens
 * [p*P, (p+1)*P); partition_offsets[s] = sum_{r<s} n_r, partition_offsets[S]
 * = total_partitions.
 *
 * paged_attention_partition_offsets computes those offsets on the host.
 *  context_lens_host [num_seqs] int32 (host, caller-owned, read only)
 *  offsets_host_out  [num_seqs + 1] int32 (host, caller-owned, written)
 *  *total_partitions_out  (host, may be NULL) = offsets_host_out[num_seqs]
 * Returns PKV_ERR_INVALID for a null array, P <= 0, a negative length or a
 * total above INT32_MAX (nothing useful is written then).  Touches no device.
 * ------------------------------------------------------------------------- */
int paged_attention_partition_offsets(const int32_t* context_lens_host, int num_seqs,
                                      int partition_tokens, int32_t* offsets_host_out,
                                      int* total_partitions_out);

/* Workspace bytes the split-K decode needs for total_partitions partitions
 * (the partials of "PagedAttention Kernel：大模型推理优化的显存管理革新"
 * §3.2's split work, combined by the reduce): one fp32 row of head_dim
 * unnormalised outputs and one (max, sum) pair per (partition, query head),
 * then 256 bytes for the work counter of the persistent decode (§3.2's
 * atomic page counter):
 * total_partitions * num_q_heads * (head_dim + 2) * 4 + 256 bytes.  The
 * workspace must be 16-byte aligned.  Returns 0 when an argument is not
 * positive.  Pure arithmetic, no device access. */
size_t paged_attention_workspace_bytes(int total_partitions, int num_q_heads, int head_dim);

/* ---------------------------------------------------------------------------
 * paged_attention_decode -- out[s, g, :] = softmax(scale * K_s q_{s,g}) V_s
 * over the context_lens[s] tokens of sequence s, with K_s, V_s read block by
 * block through block_tables ("PagedAttention Kernel：大模型推理优化的显存管理
 * 革新" §3.1: QK^T per block, softmax, PV; fp32 accumulation per §6).
 *
 *  out            [num_seqs][num_q_heads][head_dim] of q_dtype (device)
 *  query          [num_seqs][num_q_heads][head_dim] of q_dtype (device)
 *  key_cache,
 *  value_cache    block pools of cache_dtype (device)
 *  block_tables   [num_seqs][max_blocks_per_seq] int32 physical block ids
 *                 (device); only the first ceil(context_lens[s]/block_size)
 *                 entries of row s are read
 *  context_lens   [num_seqs] int32 (device); 0 gives a zero output row
 *  scale          softmax scale applied to q.k (fp32)
 *  k_scale,v_scale dequantisation multipliers of an FP8 cache (else ignored)
 *  partition_tokens 0 = one pass per sequence (no workspace needed);
 *                 else P > 0, a multiple of block_size: split-K over
 *                 partitions of P tokens, partials in `workspace`, then the
 *                 split-K reduce (both launched here, in order, on `stream`)
 *  partition_offsets [num_seqs + 1] int32 (device), as described above;
 *                 NULL when partition_tokens == 0.  A sequence whose entry
 *                 count disagrees with its device length (stale offsets, say
 *                 from the lengths before a step) gets NaN output rows, and
 *                 so does a sequence given no partition; with such offsets
 *                 whether the decode step stores that sequence's new row is
 *                 unspecified
 *  total_partitions host copy of partition_offsets[num_seqs]
 *  workspace      device scratch of >= paged_attention_workspace_bytes()
 *                 bytes, 16-byte aligned (caller-owned; contents need no
 *                 initialisation; two calls that run at the same time need
 *                 two workspaces)
 * ------------------------------------------------------------------------- */
int paged_attention_decode(void* out, const void* query, const void* key_cache,
                           const void* value_cache, const int32_t* block_tables,
                           int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                           int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                           int num_blocks, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                           float k_scale, float v_scale, int partition_tokens,
                           const int32_t* partition_offsets, int total_partitions,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * paged_attention_decode_noalloc -- paged_attention_decode for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, result and
 * launches as paged_attention_decode without workspace / workspace_bytes:
 * the split-K partials go to a device array inside the library,
 * PKV_NOALLOC_WORKSPACE_BYTES (64 MiB) per GPU, which each GPU the library
 * runs on holds until the process ends.  The call allocates nothing: its
 * first call on a device looks up that device's copy of the array
 * (hipGetSymbolAddress), every call launches the decode and the reduce on
 * `stream`.
 *  - partition_tokens > 0 with paged_attention_workspace_bytes(
 *    total_partitions, num_q_heads, head_dim) > PKV_NOALLOC_WORKSPACE_BYTES
 *    returns PKV_ERR_WORKSPACE and launches nothing; other errors as
 *    paged_attention_decode.
 *  - All calls on one GPU share the array, which keeps the last call's
 *    partials; nothing in it needs clearing (every partial a call reads, the
 *    same call writes first).  Calls that overlap on one GPU (two streams,
 *    two threads) race: order them on one stream or with events.
 * ------------------------------------------------------------------------- */
#define PKV_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
int paged_attention_decode_noalloc(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   int max_blocks_per_seq, const int32_t* context_lens,
                                   int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                   int block_size, int num_blocks, float scale, pkv_dtype q_dtype,
                                   pkv_dtype cache_dtype, float k_scale, float v_scale,
                                   int partition_tokens, const int32_t* partition_offsets,
                                   int total_partitions, void* stream);

/* ---------------------------------------------------------------------------
 * paged_attention_decode_queue -- paged_attention_decode's split-K with its
 * work items handed out by a device work counter: a grid of resident waves,
 * each taking (sequence, partition, kv head) items one after another in the
 * same longest-first order, and loading the next item's table entries, query
 * and first tile while the current one streams ("PagedAttention Kernel：大模型
 * 推理优化的显存管理革新" §3.2: an atomic page counter in a persistent loop;
 * §2.2: prefetch of the next page).  Same arguments, result (bit for bit)
 * and errors as paged_attention_decode, plus:
 *  - only an fp8 E4M3 cache with bf16 queries, head_dim 128, block_size 32,
 *    a multiple of 8 query heads per kv head, 0 < partition_tokens <= 2048
 *    and num_seqs <= 512; anything else returns PKV_ERR_UNSUPPORTED and
 *    launches nothing;
 *  - the counter lives in the workspace's last bytes (inside
 *    paged_attention_workspace_bytes) and is reset by the launch itself, so
 *    the workspace still needs no initialisation.
 * paged_attention_decode's hardware-dispatched waves are faster on MI355X;
 * this schedule exists for comparison and for callers that want it.
 * ------------------------------------------------------------------------- */
int paged_attention_decode_queue(void* out, const void* query, const void* key_cache,
                                 const void* value_cache, const int32_t* block_tables,
                                 int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                                 int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                 int num_blocks, float scale, pkv_dtype q_dtype,
                                 pkv_dtype cache_dtype, float k_scale, float v_scale,
                                 int partition_tokens, const int32_t* partition_offsets,
                                 int total_partitions, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* paged_attention_decode_partials -- the first of the two launches above on
 * its own: writes `out` for sequences with a single partition and partials
 * (m, l, unnormalised o) into `workspace` for the others.  Same arguments as
 * paged_attention_decode; partition_tokens must be > 0. */
int paged_attention_decode_partials(void* out, const void* query, const void* key_cache,
                                    const void* value_cache, const int32_t* block_tables,
                                    int max_blocks_per_seq, const int32_t* context_lens,
                                    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                    int block_size, int num_blocks, float scale, pkv_dtype q_dtype,
                                    pkv_dtype cache_dtype, float k_scale, float v_scale,
                                    int partition_tokens, const int32_t* partition_offsets,
                                    int total_partitions, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* paged_attention_decode_step -- one whole decode step: store each
 * sequence's new key/value row, then attend over the context that now holds
 * it ("Day 6/90 of Inference Engineering": a decode step appends its token to
 * the sequence's last block, then attention reads every block of the table).
 * The result equals paged_kv_write of the new rows followed by
 * paged_attention_decode, with these differences:
 *  new_key, new_value [num_seqs][num_kv_heads][head_dim] of q_dtype (device):
 *                 row s is the token at position context_lens[s] - 1 of
 *                 sequence s, stored into the slot that block_tables gives
 *                 for that position (so the caller has already grown the
 *                 table); a sequence of length 0, longer than its table or
 *                 with an out-of-range block id gets no store.  bf16 rows
 *                 go to an FP8 cache as E4M3FN(fp32(x) / k_scale) (v_scale
 *                 for values), rounded as paged_kv_write rounds them.
 *  key_cache, value_cache are written.
 * When one workgroup reads each (sequence, kv head) partition -- the
 * vector-ALU kernel with all G query heads of a kv head in one workgroup --
 * that workgroup stores the new token before it reads the last block, so
 * store and decode are one launch; otherwise a store launch precedes the
 * decode.  With partitions the split-K reduce follows, as in
 * paged_attention_decode.  Returns PKV_ERR_INVALID for a null new_key or
 * new_value, else as paged_attention_decode. */
int paged_attention_decode_step(void* out, const void* query, const void* new_key,
                                const void* new_value, void* key_cache, void* value_cache,
                                const int32_t* block_tables, int max_blocks_per_seq,
                                const int32_t* context_lens, int num_seqs, int num_q_heads,
                                int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                float k_scale, float v_scale, int partition_tokens,
                                const int32_t* partition_offsets, int total_partitions,
                                void* workspace, size_t workspace_bytes, void* stream);

/* paged_attention_decode_step_launches -- how many kernel launches
 * paged_attention_decode_step makes for this shape: 1 (store inside the
 * decode, no partitions) to 3 (store, decode, split-K reduce).  Returns a
 * negative PKV_ERR_* for bad or unsupported arguments.  Host only; touches
 * no device. */
int paged_attention_decode_step_launches(int num_q_heads, int num_kv_heads, int head_dim,
                                         int block_size, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                         int partition_tokens);

/* ---------------------------------------------------------------------------
 * Stream-K decode: the same result as paged_attention_decode, scheduled for
 * uneven lengths ("PagedAttention Kernel：大模型推理优化的显存管理革新" §3.2:
 * sequences of very different lengths leave workers idle unless the work is
 * rebalanced).  The (block, kv head) tiles of all sequences are laid end to
 * end, per group of query heads, and each of `workers` persistent waves takes
 * an equal contiguous slice; a sequence cut between waves is recombined by a
 * reduce launch with the split-K rule.  Each wave streams the same number of
 * tiles whatever the length mix.
 *
 *  tile_offsets   [num_seqs + 1] int32 (device): 0, then running sums of
 *                 ceil(context_lens[s] / block_size)
 *                 (paged_attention_tile_offsets computes them on the host);
 *                 a sequence whose entry disagrees with its device length
 *                 gets a NaN output row
 *  total_tiles    host copy of tile_offsets[num_seqs]
 *  workers        waves to launch, > 0; paged_attention_streamk_workers
 *                 gives the number resident on the current device
 *  workspace      device scratch of >= paged_attention_streamk_workspace_bytes
 *                 (workers, ...) bytes (caller-owned; no initialisation)
 * Other arguments as paged_attention_decode.  Two launches on `stream`
 * (decode, reduce); the reduce also writes the zero rows of empty sequences.
 * ------------------------------------------------------------------------- */
int paged_attention_tile_offsets(const int32_t* context_lens_host, int num_seqs, int block_size,
                                 int32_t* offsets_host_out, int* total_tiles_out);

/* Waves of the stream-K kernel resident at once on the current device for
 * this shape (workgroups per CU at full occupancy x CUs x waves per
 * workgroup); a negative PKV_ERR_* on bad arguments. */
int paged_attention_streamk_workers(int num_q_heads, int num_kv_heads, int head_dim,
                                    int block_size, pkv_dtype q_dtype, pkv_dtype cache_dtype);

/* Workspace of the stream-K decode:
 * (workers * (num_q_heads / num_kv_heads) + num_seqs * num_q_heads)
 * * (head_dim + 2) * 4 bytes; 0 for bad arguments. */
size_t paged_attention_streamk_workspace_bytes(int workers, int num_seqs, int num_q_heads,
                                               int num_kv_heads, int head_dim);

int paged_attention_decode_streamk(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   int max_blocks_per_seq, const int32_t* context_lens,
                                   const int32_t* tile_offsets, int total_tiles, int num_seqs,
                                   int num_q_heads, int num_kv_heads, int head_dim,
                                   int block_size, int num_blocks, float scale,
                                   pkv_dtype q_dtype, pkv_dtype cache_dtype, float k_scale,
                                   float v_scale, int workers, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* The two launches of paged_attention_decode_streamk on their own: the
 * decode writes the outputs of sequences that one wave covered whole and the
 * partials of the others; the reduce combines those partials and writes the
 * zero rows of empty sequences.  Arguments as above. */
int paged_attention_decode_streamk_partials(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* tile_offsets, int total_tiles, int num_seqs, int num_q_heads, int num_kv_heads,
    int head_dim, int block_size, int num_blocks, float scale, pkv_dtype q_dtype,
    pkv_dtype cache_dtype, float k_scale, float v_scale, int workers, void* workspace,
    size_t workspace_bytes, void* stream);
int paged_attention_streamk_reduce(void* out, const void* workspace, size_t workspace_bytes,
                                   const int32_t* tile_offsets, int total_tiles, int num_seqs,
                                   int num_q_heads, int num_kv_heads, int head_dim,
                                   int block_size, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                   int workers, void* stream);

/* paged_attention_decode_step_streamk -- paged_attention_decode_step with the
 * stream-K schedule: new_key/new_value as there; the wave that reads a
 * sequence's last block stores the new token first when one wave covers all
 * query heads of a kv head, else a store launch precedes the decode. */
int paged_attention_decode_step_streamk(void* out, const void* query, const void* new_key,
                                        const void* new_value, void* key_cache, void* value_cache,
                                        const int32_t* block_tables, int max_blocks_per_seq,
                                        const int32_t* context_lens, const int32_t* tile_offsets,
                                        int total_tiles, int num_seqs, int num_q_heads,
                                        int num_kv_heads, int head_dim, int block_size,
                                        int num_blocks, float scale, pkv_dtype q_dtype,
                                        pkv_dtype cache_dtype, float k_scale, float v_scale,
                                        int workers, void* workspace, size_t workspace_bytes,
                                        void* stream);

/* ---------------------------------------------------------------------------
 * Shared-prefix decode ("Day 6/90 of Inference Engineering": prompts that
 * begin alike share their prefix blocks by reference and continue in blocks
 * of their own).  The same result as paged_attention_decode, scheduled so
 * that the blocks a group of sequences shares are read once per 32 query
 * rows ((sequence, query head) pairs of a kv head) instead of once per
 * sequence: a matrix-core pass over each group's shared blocks leaves
 * partials, the split-K decode covers every sequence's own tokens from the
 * end of its group's prefix, and the split-K reduce combines both.
 * bf16 query and cache, head_dim 128, block_size 16 (else
 * PKV_ERR_UNSUPPORTED).
 *
 * paged_attention_prefix_plan (host only): groups are runs of consecutive
 * sequences, group g = sequences group_offsets[g] .. group_offsets[g+1]-1
 * (group_offsets[0] = 0, group_offsets[num_groups] = num_seqs), whose tables
 * all begin with the same group_prefix_blocks[g] block ids (0 = nothing
 * shared).  Every member must be at least that many blocks long.  Outputs
 * (caller-owned host arrays): row_offsets_out [num_seqs+1] (partial rows of
 * each sequence: its suffix partitions, then one row per 8 prefix blocks),
 * suffix_offsets_out [num_seqs+1] (suffix partitions), token_start_out
 * [num_seqs] (first own token), prefix_item_offsets_out [num_groups+1]
 * (waves of the prefix pass), totals_out [3] = (rows, suffix partitions,
 * prefix waves).  PKV_ERR_INVALID on inconsistent groups.
 *
 * paged_attention_decode_prefix: the usual decode arguments, then
 * partition_tokens (> 0) and the plan's arrays uploaded to the device
 * (group_offsets, group_prefix_blocks, row_offsets, suffix_offsets,
 * token_start, prefix_item_offsets) with its three totals; workspace of
 * paged_attention_workspace_bytes(total_rows, num_q_heads, head_dim) bytes.
 * Two launches on `stream` (both passes in one, then the reduce).  A block
 * id out of range in a group's prefix makes every member's output NaN; a
 * sequence whose context length gives another count of suffix partitions
 * than suffix_offsets (a plan made for other lengths) gets a NaN output
 * row.
 * ------------------------------------------------------------------------- */
int paged_attention_prefix_plan(const int32_t* context_lens_host, int num_seqs,
                                const int32_t* group_offsets_host,
                                const int32_t* group_prefix_blocks_host, int num_groups,
                                int block_size, int partition_tokens, int num_q_heads,
                                int num_kv_heads, int32_t* row_offsets_out,
                                int32_t* suffix_offsets_out, int32_t* token_start_out,
                                int32_t* prefix_item_offsets_out, int32_t* totals_out);

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
                                  size_t workspace_bytes, void* stream);

/* paged_attention_decode_prefix_step -- the shared-prefix decode's whole
 * decode step ("Day 6/90 of Inference Engineering": a step appends its token
 * to the sequence's own last block, then attention reads every block of the
 * table): store each sequence's new key/value row, then decode as
 * paged_attention_decode_prefix.  The plan comes from the step's context
 * lengths (the new token included).  new_key, new_value as in
 * paged_attention_decode_step (row s is the token at position
 * context_lens[s] - 1, stored into the slot the table gives; bf16);
 * key_cache and value_cache are written.  A sequence whose new token lies in
 * its group's shared blocks (context_lens[s] <= token_start[s], which a cache
 * that copies shared blocks on write never produces) gets a NaN output row
 * and no store.  The result is paged_kv_write of the new rows followed by
 * paged_attention_decode_prefix, bit for bit.  Where the suffix pass gives
 * each (sequence, kv head) one workgroup (query heads per kv head of 1, 2 or
 * 4), the suffix workgroup that reads a sequence's last block stores the
 * token first and the step is two launches (decode, reduce); otherwise a
 * store launch precedes them.  Returns PKV_ERR_INVALID for a null new_key or
 * new_value, else as paged_attention_decode_prefix. */
int paged_attention_decode_prefix_step(
    void* out, const void* query, const void* new_key, const void* new_value, void* key_cache,
    void* value_cache, const int32_t* block_tables, int max_blocks_per_seq,
    const int32_t* context_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
    int block_size, int num_blocks, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
    float k_scale, float v_scale, int partition_tokens, const int32_t* group_offsets,
    const int32_t* group_prefix_blocks, int num_groups, const int32_t* row_offsets,
    const int32_t* suffix_offsets, const int32_t* token_start, const int32_t* prefix_item_offsets,
    int total_rows, int total_suffix_partitions, int total_prefix_items, void* workspace,
    size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * paged_attention_prefill -- chunked prefill over the paged cache.
 * The block table makes a sequence's scattered blocks read as one contiguous
 * cache ("Day 6/90 of Inference Engineering", PagedAttention notes), and
 * attention is QK^T, softmax, PV block by block ("PagedAttention Kernel：大
 * 模型推理优化的显存管理革新" §3.1, fp32 accumulation per §6).  The pages
 * only describe decode; for a chunk of new tokens this takes the plain
 * causal reading: sequence s holds context_lens[s] = L tokens (the chunk's
 * keys and values already stored, e.g. by paged_kv_write), its last
 * C = query_start[s+1] - query_start[s] positions are the chunk, and chunk
 * row i, at position L - C + i, attends tokens 0 .. L - C + i:
 *   out[query_start[s] + i, g, :] = softmax_t(scale * q . k_t) v_t  over
 *   those tokens, kv head g / (num_q_heads / num_kv_heads).
 *
 *  out, query     [total rows][num_q_heads][head_dim] bf16 (device), rows of
 *                 all chunks in sequence order
 *  query_start    [num_seqs + 1] int32 (device), non-decreasing, [0] = 0
 *  max_query_len  >= every chunk length (sizes the grid); rows of a longer
 *                 chunk past max_query_len are left unwritten
 *  other arguments as paged_attention_decode; bf16 query and cache,
 *  head_dim 128, block_size 16 (else PKV_ERR_UNSUPPORTED); k_scale and
 *  v_scale are ignored.  A chunk longer than its context, or a block id out
 *  of range among the blocks a row block reads, gives NaN rows.  One launch
 *  on `stream`, no workspace.
 * ------------------------------------------------------------------------- */
int paged_attention_prefill(void* out, const void* query, const void* key_cache,
                            const void* value_cache, const int32_t* block_tables,
                            int max_blocks_per_seq, const int32_t* context_lens,
                            const int32_t* query_start, int num_seqs, int max_query_len,
                            int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                            int num_blocks, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                            float k_scale, float v_scale, void* stream);

/* paged_attention_splitk_reduce -- combine the partials of every sequence
 * with more than one partition ("PagedAttention Kernel" article §3.2: uneven
 * pages need the work split): with running maxima m_p (log2 domain), sums
 * l_p and unnormalised outputs o_p, out = sum_p 2^(m_p - M) o_p /
 * sum_p 2^(m_p - M) l_p, M = max_p m_p.  Sequences with one partition are
 * left untouched.  max_partitions_per_seq: the caller's bound on one
 * sequence's partition count, or 0 if unknown; it only selects the launch
 * shape (past 4 partials per piece lane of the reduce, a kernel that holds
 * more partial rows in flight), and every value gives the same result. */
int paged_attention_splitk_reduce(void* out, const void* workspace, size_t workspace_bytes,
                                  const int32_t* partition_offsets, int num_seqs,
                                  int num_q_heads, int head_dim, int total_partitions,
                                  int max_partitions_per_seq, pkv_dtype out_dtype, void* stream);

/* ---------------------------------------------------------------------------
 * paged_kv_copy_blocks -- copy whole key and value blocks (all kv heads):
 * for i < num_pairs, block pairs[2i] -> block pairs[2i+1], in both pools.
 * Serves the allocator's copy-on-write of a shared, partly filled last block
 * (prefix sharing, "Day 6/90 of Inference Engineering").  pairs is device
 * int32 [num_pairs][2]; block_bytes = num_kv_heads*block_size*head_dim*elem.
 * Destinations must be distinct and no destination may be a source.
 * ------------------------------------------------------------------------- */
int paged_kv_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs, int num_pairs,
                         size_t block_bytes, int num_blocks, void* stream);

/* ---------------------------------------------------------------------------
 * paged_kv_swap_blocks -- move whole blocks between two pools of the same
 * layout, for swapping a sequence to host memory and back (the pairs come
 * from pkv_alloc_swap_out / pkv_alloc_swap_in).  For each pair (s, d):
 * dst_key_cache block d = src_key_cache block s, same for values.
 *  pools          block-major pools, block_bytes per block per pool; each
 *                 either a device pool or a pinned host pool passed as the
 *                 device pointer pkv_host_device_pointer returned for it
 *  pairs          [num_pairs][2] int32 (device): (src block, dst block);
 *                 ids outside [0, src_blocks) / [0, dst_blocks) skip the pair
 *  Two destinations of one call must differ (else they race).  One launch
 *  on `stream`; reads from a host pool cross the host link.
 * ------------------------------------------------------------------------- */
int paged_kv_swap_blocks(void* dst_key_cache, void* dst_value_cache, const void* src_key_cache,
                         const void* src_value_cache, const int32_t* pairs, int num_pairs,
                         size_t block_bytes, int src_blocks, int dst_blocks, void* stream);

/* ---------------------------------------------------------------------------
 * paged_kv_swap_blocks_memcpy -- paged_kv_swap_blocks as asynchronous copies
 * of whole runs: each run of pairs whose source and destination ids both
 * step by one becomes one hipMemcpyAsync per pool on `stream` ("PagedAttention
 * Kernel：大模型推理优化的显存管理革新" §6: asynchronous copies on a stream of
 * their own, beside the compute stream).  For a swap, the engine first
 * gathers a sequence's scattered blocks into a contiguous device staging
 * pool with paged_kv_swap_blocks (HBM to HBM), so the host-link copy is a
 * few long runs; on MI355X a decode running beside those copies keeps its
 * speed, where beside paged_kv_swap_blocks straight to the host it slows
 * down 2.3x.  Same pools, pair semantics (ids out of range skip the pair)
 * and errors as paged_kv_swap_blocks, except:
 *  pairs_host     [num_pairs][2] int32 in HOST memory, read during the call
 *  The call returns once the copies are queued; the pools must stay alive
 *  until `stream` reaches them.  How the runtime carries out a copy (its
 *  copy kernels or a DMA engine) is the runtime's choice.
 * ------------------------------------------------------------------------- */
int paged_kv_swap_blocks_memcpy(void* dst_key_cache, void* dst_value_cache,
                             const void* src_key_cache, const void* src_value_cache,
                             const int32_t* pairs_host, int num_pairs, size_t block_bytes,
                             int src_blocks, int dst_blocks, void* stream);

/* Device pointer of pinned host memory (hipHostGetDevicePointer); fails with
 * PKV_ERR_HIP for memory that is not pinned.  Host memory is only ever
 * handed to a kernel through this pointer. */
int pkv_host_device_pointer(const void* host, void** device_out);

/* paged_kv_gather -- read every sequence back through its block table into
 * dense rows, i.e. the contiguous cache the block table makes the scattered
 * blocks look like ("Day 6/90 of Inference Engineering", PagedAttention
 * notes: the block table maps logical blocks to physical ones).  A test aid
 * for bit-exact checks of the cache contents.
 *  k_out, v_out   [total_tokens][num_kv_heads][head_dim] of cache_dtype bits
 *                 (device, caller-owned, written); sequence s occupies rows
 *                 cu_ctx[s] .. cu_ctx[s+1]-1, token t of it in row
 *                 cu_ctx[s] + t, read from block block_tables[s][t / bs],
 *                 slot t % bs
 *  cu_ctx         [num_seqs + 1] int32 (device): 0, then running sums of the
 *                 lengths; total_tokens = cu_ctx[num_seqs], passed from the
 *                 host (it sizes the launch)
 *  block_tables   [num_seqs][max_blocks_per_seq] int32 (device)
 * Host-visible errors as paged_kv_write; a block id outside [0, num_blocks),
 * or a position past the table width, gives rows of zero bits instead of a
 * read outside the pool or the table. */
int paged_kv_gather(void* k_out, void* v_out, const void* key_cache, const void* value_cache,
                    const int32_t* block_tables, int max_blocks_per_seq, const int32_t* cu_ctx,
                    int num_seqs, int total_tokens, int num_kv_heads, int head_dim, int block_size,
                    int num_blocks, pkv_dtype cache_dtype, void* stream);

/* pkv_hbm_read_probe -- measurement aid: `workgroups` workgroups of 256
 * lanes stream-read `bytes` (rounded down to 16) of device memory at
 * `buffer`, each workgroup a contiguous 32 KiB run at a time (16-byte
 * non-temporal loads, eight in flight per lane), and store at most
 * one word to device `sink` (4 bytes).  Timing it gives the attainable HBM
 * read rate, the ceiling for the decode kernel's key/value stream (an HBM
 * bound kernel is measured by bytes moved, "Memory Systems" notes, core idea
 * 1). */
int pkv_hbm_read_probe(const void* buffer, size_t bytes, void* sink, int workgroups, void* stream);

/* pkv_paged_read_probe -- measurement aid: the reads of the split-K kernel
 * paged_attention_decode runs for this shape (the vector-ALU kernel, or the
 * matrix-core kernel of fp8 caches with 8 query heads per kv head) and
 * nothing else (same grid, workgroup order, block-table walk and tile ring;
 * no arithmetic, no partials, no reduce).  Arguments as paged_attention_decode without out, query, scale
 * and the workspace (k/v scales do not matter); partition_tokens must be > 0.
 * sink: 16-byte aligned device memory of which at most 4 bytes are written.
 * Timing it gives the rate that the decode's access pattern (scattered
 * blocks reached through the block table, 1 KiB-contiguous loads) reaches
 * on the device ("Memory Systems" notes, core idea 1). */
int pkv_paged_read_probe(const void* key_cache, const void* value_cache,
                         const int32_t* block_tables, int max_blocks_per_seq,
                         const int32_t* context_lens, int num_seqs, int num_q_heads,
                         int num_kv_heads, int head_dim, int block_size, int num_blocks,
                         pkv_dtype q_dtype, pkv_dtype cache_dtype, int partition_tokens,
                         const int32_t* partition_offsets, int total_partitions, void* sink,
                         void* stream);

/* ---------------------------------------------------------------------------
 * Host block allocator ("Day 6/90 of Inference Engineering", PagedAttention
 * notes): hands out one block at a time, takes a new block only when the
 * last one is full, shares prefix blocks by reference count and starts a
 * new block where prompts diverge.  Host memory only; not thread-safe.
 * Every call either succeeds or returns an error leaving the state as it
 * was.  Policy, fixed so tables are reproducible:
 *   - free list: FIFO queue initialised from free_order (NULL = 0..n-1);
 *     allocation pops the front; a block whose refcount reaches 0 is pushed
 *     to the back;
 *   - fork(parent, child): child gets a copy of the parent's table and
 *     length; every block gains one reference;
 *   - append(seq, n): token by token -- if the sequence has no block or its
 *     last block is full, pop a new block; else if the last block's refcount
 *     is > 1, pop a new block, emit a copy-on-write pair (old, new), drop a
 *     reference to old and replace it in the table; the token takes slot
 *     table[pos / bs] * bs + pos % bs;
 *   - free_seq: drop one reference per table entry, in table order.
 *  Swapping to host memory ("PagedAttention Kernel：大模型推理优化的显存管理革
 *  新" §4.1 weighs page replacement policies; its table of them is missing,
 *  so least-recently-used is a reading):
 *   - a host pool of num_host_blocks slots with its own FIFO free list
 *     (initially 0, 1, ...);
 *   - swap_out(seq): every block must be unshared (refcount 1), else
 *     PKV_ERR_INVALID; table entry by entry, pop a host slot, emit the pair
 *     (device block, host slot), drop the block's reference and put the
 *     slot in the table;
 *   - swap_in(seq): table entry by entry, pop a device block, emit the pair
 *     (host slot, device block), return the slot to the back of the host
 *     free list and put the block in the table;
 *   - a swapped-out sequence may only be swapped in or freed (its slots go
 *     back in table order); append, fork from it and fill_tables give
 *     PKV_ERR_INVALID; block_table returns its host slots;
 *   - a clock ticks on add, fork (the child), append, swap_in and touch,
 *     stamping that sequence; lru names the resident sequence with at least
 *     one block, all unshared, whose stamp is oldest (PKV_ERR_SEQ if none);
 *   - the same events count a sequence's uses (a new or forked sequence
 *     starts at 1); lfu names, among the same candidates, the one with the
 *     fewest uses, the oldest stamp among equals (least frequently used:
 *     §4.1 advises LRU for document processing and LFU for batch work; its
 *     comparison table is missing, so the choice stays with the caller).
 *  The pairs drive paged_kv_swap_blocks, which moves the data.
 * ------------------------------------------------------------------------- */
typedef struct pkv_alloc pkv_alloc;

/* NULL on invalid arguments (see pkv_last_error): num_blocks or block_size
 * not positive, num_blocks * block_size above INT32_MAX (slot ids are int32),
 * or a free_order that is not a permutation of 0..num_blocks-1 (host memory,
 * copied). */
pkv_alloc* pkv_alloc_create(int num_blocks, int block_size, const int32_t* free_order);
void pkv_alloc_destroy(pkv_alloc* a);
int pkv_alloc_add_seq(pkv_alloc* a, int64_t seq);
int pkv_alloc_fork(pkv_alloc* a, int64_t parent, int64_t child);
/* slots_out: host int32 [n_tokens]; cow_pairs_out: host int32 [2*cow_cap]
 * receiving (src, dst) pairs; *n_cow_out = pairs written (at most 1 per
 * call).  cow_cap < 1 is an error only if a copy is needed. */
int pkv_alloc_append(pkv_alloc* a, int64_t seq, int n_tokens, int32_t* slots_out,
                     int32_t* cow_pairs_out, int cow_cap, int* n_cow_out);
int pkv_alloc_free_seq(pkv_alloc* a, int64_t seq);
/* Copies the table of seq into out (host, capacity cap); *n_out = its length. */
int pkv_alloc_block_table(const pkv_alloc* a, int64_t seq, int32_t* out, int cap, int* n_out);
/* Fills out[num_seqs][width] (host) with the tables of seqs[i], padded with
 * pad; fails if a table is wider than width. */
int pkv_alloc_fill_tables(const pkv_alloc* a, const int64_t* seqs, int num_seqs, int32_t* out,
                          int width, int32_t pad);
/* Length in tokens of seq, or a negative error (PKV_ERR_SEQ for an unknown
 * sequence).  A length never exceeds num_blocks * block_size, which
 * pkv_alloc_create keeps within INT32_MAX, so the int result is exact.
 * pkv_alloc_seq_len is the same value as int64_t. */
int pkv_alloc_len(const pkv_alloc* a, int64_t seq);
int64_t pkv_alloc_seq_len(const pkv_alloc* a, int64_t seq);
/* Refcount of a block, or a negative error. */
int pkv_alloc_refcount(const pkv_alloc* a, int32_t block);
int pkv_alloc_num_free(const pkv_alloc* a);
/* Copies the free list, front first, into out (capacity cap); returns count. */
int pkv_alloc_free_list(const pkv_alloc* a, int32_t* out, int cap);
/* Sets the host pool to num_host_blocks slots (free list 0, 1, ...); fails
 * while any sequence is swapped out. */
int pkv_alloc_set_host_pool(pkv_alloc* a, int num_host_blocks);
/* pairs_out: host int32 [2*cap], (device block, host slot) per table entry;
 * *n_out = pairs written (the table length).  cap below the table length is
 * PKV_ERR_INVALID; too few host slots PKV_ERR_NO_BLOCKS. */
int pkv_alloc_swap_out(pkv_alloc* a, int64_t seq, int32_t* pairs_out, int cap, int* n_out);
/* pairs_out: (host slot, device block) per table entry; too few free device
 * blocks is PKV_ERR_NO_BLOCKS. */
int pkv_alloc_swap_in(pkv_alloc* a, int64_t seq, int32_t* pairs_out, int cap, int* n_out);
/* Marks seq as used now. */
int pkv_alloc_touch(pkv_alloc* a, int64_t seq);
/* *seq_out = the least recently used sequence that can be swapped out. */
int pkv_alloc_lru(const pkv_alloc* a, int64_t* seq_out);
/* *seq_out = the least frequently used sequence that can be swapped out. */
int pkv_alloc_lfu(const pkv_alloc* a, int64_t* seq_out);
/* 1 if seq is swapped out, 0 if resident, or a negative error. */
int pkv_alloc_is_swapped(const pkv_alloc* a, int64_t seq);
int pkv_alloc_num_host_free(const pkv_alloc* a);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
