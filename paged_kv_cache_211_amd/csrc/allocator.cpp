// Host block allocator for the paged KV cache.
//
// "Day 6/90 of Inference Engineering" (PagedAttention notes): during decode
// the cache manager hands out one block at a time and only takes a new block
// when the current one is full, so every block is filled before the next is
// allocated and the decision is just "is the last block full?"; prompts with a
// common prefix share its blocks, and writing resumes in a new block where
// they diverge; a block table maps each sequence's logical blocks to scattered
// physical blocks.  The unstated policy (FIFO free list, copy-on-write of a
// shared, partly filled last block, all-or-nothing calls) is spelled out in
// pkv.h, and so are swapping to a host pool and the least-recently-used
// choice of a sequence to swap ("PagedAttention Kernel：大模型推理优化的显存管
// 理革新" §4.1 compares replacement policies; its table is missing, so the
// policy is a reading).
//
// Single-threaded by contract: callers serialise access to one allocator.

#include <deque>
#include <unordered_map>
#include <vector>

#include "pkv.h"
#include "pkv_internal.h"

struct pkv_alloc {
  int num_blocks = 0;
  int bs = 0;
  std::deque<int32_t> free_q;
  std::vector<int32_t> ref;
  std::deque<int32_t> host_free;   // host pool slots, FIFO
  int num_host = 0;
  int64_t clock = 0;                // ticks on add, fork, append, swap_in, touch
  struct Seq {
    std::vector<int32_t> table;     // device blocks, or host slots when swapped
    int64_t len = 0;
    bool swapped = false;
    int64_t stamp = 0;              // clock at the last use
    int64_t uses = 0;               // uses counted on the same events
  };
  std::unordered_map<int64_t, Seq> seqs;
};

namespace {

int no_seq(int64_t seq) { return pkv::fail(PKV_ERR_SEQ, "unknown sequence %lld", (long long)seq); }

void drop_ref(pkv_alloc* a, int32_t b) {
  if (--a->ref[b] == 0) a->free_q.push_back(b);
}

int swapped_out(int64_t seq) {
  return pkv::fail(PKV_ERR_INVALID, "sequence %lld is swapped out", (long long)seq);
}

// The resident sequence with at least one block, all unshared, that is
// smallest in (by_uses ? uses : 0, stamp): the victim of either policy.
int pick_victim(const pkv_alloc* a, bool by_uses, int64_t* seq_out) {
  if (!a || !seq_out) return pkv::fail(PKV_ERR_INVALID, "null argument");
  bool found = false;
  int64_t best = 0, best_uses = 0, best_stamp = 0;
  for (const auto& kv : a->seqs) {
    const pkv_alloc::Seq& s = kv.second;
    if (s.swapped || s.table.empty()) continue;
    bool shared = false;
    for (int32_t b : s.table) shared = shared || a->ref[b] != 1;
    if (shared) continue;
    const int64_t u = by_uses ? s.uses : 0;
    if (!found || u < best_uses || (u == best_uses && s.stamp < best_stamp)) {
      found = true;
      best = kv.first;
      best_uses = u;
      best_stamp = s.stamp;
    }
  }
  if (!found) return pkv::fail(PKV_ERR_SEQ, "no sequence can be swapped out");
  *seq_out = best;
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_alloc* pkv_alloc_create(int num_blocks, int block_size, const int32_t* free_order) {
  if (num_blocks <= 0 || block_size <= 0) {
    pkv::fail(PKV_ERR_INVALID, "num_blocks and block_size must be positive");
    return nullptr;
  }
  // slot ids (block * block_size + offset) are int32 in every interface
  if ((int64_t)num_blocks * block_size > (int64_t)INT32_MAX) {
    pkv::fail(PKV_ERR_INVALID, "num_blocks * block_size = %lld exceeds int32 slot ids",
              (long long)num_blocks * block_size);
    return nullptr;
  }
  auto* a = new pkv_alloc;
  a->num_blocks = num_blocks;
  a->bs = block_size;
  a->ref.assign(num_blocks, 0);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete a;
        pkv::fail(PKV_ERR_INVALID, "free_order is not a permutation of 0..num_blocks-1");
        return nullptr;
      }
      seen[b] = 1;
      a->free_q.push_back(b);
    }
  } else {
    for (int i = 0; i < num_blocks; ++i) a->free_q.push_back(i);
  }
  pkv::clear_error();
  return a;
}

void pkv_alloc_destroy(pkv_alloc* a) { delete a; }

int pkv_alloc_add_seq(pkv_alloc* a, int64_t seq) {
  if (!a) return pkv::fail(PKV_ERR_INVALID, "null allocator");
  if (a->seqs.count(seq)) return pkv::fail(PKV_ERR_SEQ, "sequence %lld exists", (long long)seq);
  pkv_alloc::Seq s;
  s.stamp = ++a->clock;
  s.uses = 1;
  a->seqs.emplace(seq, std::move(s));
  return PKV_OK;
}

int pkv_alloc_fork(pkv_alloc* a, int64_t parent, int64_t child) {
  if (!a) return pkv::fail(PKV_ERR_INVALID, "null allocator");
  auto it = a->seqs.find(parent);
  if (it == a->seqs.end()) return no_seq(parent);
  if (a->seqs.count(child)) return pkv::fail(PKV_ERR_SEQ, "sequence %lld exists", (long long)child);
  if (it->second.swapped) return swapped_out(parent);
  pkv_alloc::Seq c = it->second;  // copy before emplace may rehash
  for (int32_t b : c.table) ++a->ref[b];
  c.stamp = ++a->clock;
  c.uses = 1;   // a new sequence: its own count
  a->seqs.emplace(child, std::move(c));
  return PKV_OK;
}

int pkv_alloc_append(pkv_alloc* a, int64_t seq, int n_tokens, int32_t* slots_out,
                     int32_t* cow_pairs_out, int cow_cap, int* n_cow_out) {
  if (!a) return pkv::fail(PKV_ERR_INVALID, "null allocator");
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return no_seq(seq);
  if (it->second.swapped) return swapped_out(seq);
  if (n_tokens < 0) return pkv::fail(PKV_ERR_INVALID, "negative token count");
  if (n_tokens > 0 && !slots_out) return pkv::fail(PKV_ERR_INVALID, "null slots_out");
  pkv_alloc::Seq& s = it->second;
  const int64_t bs = a->bs;

  // Count what the call needs before touching anything, so a failure leaves
  // the state unchanged.  Only the first token can find a shared, partly
  // filled last block; after the copy the block is private.
  const bool partial = !s.table.empty() && (s.len % bs) != 0;
  const bool cow = n_tokens > 0 && partial && a->ref[s.table.back()] > 1;
  const int64_t have = (int64_t)s.table.size();
  const int64_t need_total = (s.len + n_tokens + bs - 1) / bs;
  const int64_t fresh = need_total - have + (cow ? 1 : 0);
  if (fresh > (int64_t)a->free_q.size())
    return pkv::fail(PKV_ERR_NO_BLOCKS, "need %lld free blocks, have %zu", (long long)fresh,
                     a->free_q.size());
  if (cow && (cow_cap < 1 || !cow_pairs_out))
    return pkv::fail(PKV_ERR_INVALID, "copy-on-write needed but cow_pairs_out has no room");

  int n_cow = 0;
  for (int i = 0; i < n_tokens; ++i) {
    const int64_t pos = s.len;
    if (s.table.empty() || pos % bs == 0) {
      int32_t b = a->free_q.front();
      a->free_q.pop_front();
      a->ref[b] = 1;
      s.table.push_back(b);
    } else if (a->ref[s.table.back()] > 1) {
      int32_t b = a->free_q.front();
      a->free_q.pop_front();
      a->ref[b] = 1;
      int32_t old = s.table.back();
      cow_pairs_out[2 * n_cow] = old;
      cow_pairs_out[2 * n_cow + 1] = b;
      ++n_cow;
      drop_ref(a, old);
      s.table.back() = b;
    }
    slots_out[i] = (int32_t)(s.table[pos / bs] * bs + pos % bs);
    s.len = pos + 1;
  }
  if (n_cow_out) *n_cow_out = n_cow;
  s.stamp = ++a->clock;
  ++s.uses;
  return PKV_OK;
}

int pkv_alloc_free_seq(pkv_alloc* a, int64_t seq) {
  if (!a) return pkv::fail(PKV_ERR_INVALID, "null allocator");
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return no_seq(seq);
  if (it->second.swapped) {
    for (int32_t h : it->second.table) a->host_free.push_back(h);
  } else {
    for (int32_t b : it->second.table) drop_ref(a, b);
  }
  a->seqs.erase(it);
  return PKV_OK;
}

int pkv_alloc_set_host_pool(pkv_alloc* a, int num_host_blocks) {
  if (!a) return pkv::fail(PKV_ERR_INVALID, "null allocator");
  if (num_host_blocks < 0) return pkv::fail(PKV_ERR_INVALID, "negative host pool size");
  for (const auto& kv : a->seqs)
    if (kv.second.swapped) return pkv::fail(PKV_ERR_INVALID, "sequences are swapped out");
  a->num_host = num_host_blocks;
  a->host_free.clear();
  for (int i = 0; i < num_host_blocks; ++i) a->host_free.push_back(i);
  return PKV_OK;
}

int pkv_alloc_swap_out(pkv_alloc* a, int64_t seq, int32_t* pairs_out, int cap, int* n_out) {
  if (!a) return pkv::fail(PKV_ERR_INVALID, "null allocator");
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return no_seq(seq);
  pkv_alloc::Seq& s = it->second;
  if (s.swapped) return swapped_out(seq);
  for (int32_t b : s.table)
    if (a->ref[b] != 1)
      return pkv::fail(PKV_ERR_INVALID, "sequence %lld holds shared blocks", (long long)seq);
  const size_t n = s.table.size();
  if (n > a->host_free.size())
    return pkv::fail(PKV_ERR_NO_BLOCKS, "need %zu host slots, have %zu", n, a->host_free.size());
  if ((int64_t)n > cap || (n > 0 && !pairs_out))
    return pkv::fail(PKV_ERR_INVALID, "pairs_out holds %d pairs, need %zu", cap, n);
  for (size_t i = 0; i < n; ++i) {
    const int32_t b = s.table[i];
    const int32_t h = a->host_free.front();
    a->host_free.pop_front();
    pairs_out[2 * i] = b;
    pairs_out[2 * i + 1] = h;
    drop_ref(a, b);
    s.table[i] = h;
  }
  s.swapped = true;
  if (n_out) *n_out = (int)n;
  return PKV_OK;
}

int pkv_alloc_swap_in(pkv_alloc* a, int64_t seq, int32_t* pairs_out, int cap, int* n_out) {
  if (!a) return pkv::fail(PKV_ERR_INVALID, "null allocator");
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return no_seq(seq);
  pkv_alloc::Seq& s = it->second;
  if (!s.swapped) return pkv::fail(PKV_ERR_INVALID, "sequence %lld is resident", (long long)seq);
  const size_t n = s.table.size();
  if (n > a->free_q.size())
    return pkv::fail(PKV_ERR_NO_BLOCKS, "need %zu free blocks, have %zu", n, a->free_q.size());
  if ((int64_t)n > cap || (n > 0 && !pairs_out))
    return pkv::fail(PKV_ERR_INVALID, "pairs_out holds %d pairs, need %zu", cap, n);
  for (size_t i = 0; i < n; ++i) {
    const int32_t h = s.table[i];
    const int32_t b = a->free_q.front();
    a->free_q.pop_front();
    a->ref[b] = 1;
    pairs_out[2 * i] = h;
    pairs_out[2 * i + 1] = b;
    a->host_free.push_back(h);
    s.table[i] = b;
  }
  s.swapped = false;
  s.stamp = ++a->clock;
  ++s.uses;
  if (n_out) *n_out = (int)n;
  return PKV_OK;
}

int pkv_alloc_touch(pkv_alloc* a, int64_t seq) {
  if (!a) return pkv::fail(PKV_ERR_INVALID, "null allocator");
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return no_seq(seq);
  it->second.stamp = ++a->clock;
  ++it->second.uses;
  return PKV_OK;
}

int pkv_alloc_lru(const pkv_alloc* a, int64_t* seq_out) { return pick_victim(a, false, seq_out); }

int pkv_alloc_lfu(const pkv_alloc* a, int64_t* seq_out) { return pick_victim(a, true, seq_out); }

int pkv_alloc_is_swapped(const pkv_alloc* a, int64_t seq) {
  if (!a) return pkv::fail(PKV_ERR_INVALID, "null allocator");
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return no_seq(seq);
  return it->second.swapped ? 1 : 0;
}

int pkv_alloc_num_host_free(const pkv_alloc* a) {
  if (!a) return pkv::fail(PKV_ERR_INVALID, "null allocator");
  return (int)a->host_free.size();
}

int pkv_alloc_block_table(const pkv_alloc* a, int64_t seq, int32_t* out, int cap, int* n_out) {
  if (!a) return pkv::fail(PKV_ERR_INVALID, "null allocator");
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return no_seq(seq);
  const auto& t = it->second.table;
  if ((int64_t)t.size() > cap) return pkv::fail(PKV_ERR_INVALID, "table wider than cap");
  for (size_t i = 0; i < t.size(); ++i) out[i] = t[i];
  if (n_out) *n_out = (int)t.size();
  return PKV_OK;
}

int pkv_alloc_fill_tables(const pkv_alloc* a, const int64_t* seqs, int num_seqs, int32_t* out,
                          int width, int32_t pad) {
  if (!a || (num_seqs > 0 && (!seqs || !out)) || num_seqs < 0 || width < 0)
    return pkv::fail(PKV_ERR_INVALID, "bad arguments");
  for (int i = 0; i < num_seqs; ++i) {
    auto it = a->seqs.find(seqs[i]);
    if (it == a->seqs.end()) return no_seq(seqs[i]);
    if (it->second.swapped) return swapped_out(seqs[i]);
    if ((int64_t)it->second.table.size() > width)
      return pkv::fail(PKV_ERR_INVALID, "table of sequence %lld wider than %d",
                       (long long)seqs[i], width);
  }
  for (int i = 0; i < num_seqs; ++i) {
    const auto& t = a->seqs.find(seqs[i])->second.table;
    int32_t* row = out + (size_t)i * width;
    for (int j = 0; j < width; ++j) row[j] = j < (int)t.size() ? t[j] : pad;
  }
  return PKV_OK;
}

int64_t pkv_alloc_seq_len(const pkv_alloc* a, int64_t seq) {
  if (!a) return pkv::fail(PKV_ERR_INVALID, "null allocator");
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return no_seq(seq);
  return it->second.len;
}

int pkv_alloc_len(const pkv_alloc* a, int64_t seq) {
  const int64_t n = pkv_alloc_seq_len(a, seq);
  return (int)n;   // an error code, or a length <= num_blocks * block_size <= INT32_MAX
}

int pkv_alloc_refcount(const pkv_alloc* a, int32_t block) {
  if (!a || block < 0 || block >= a->num_blocks)
    return pkv::fail(PKV_ERR_INVALID, "block id out of range");
  return a->ref[block];
}

int pkv_alloc_num_free(const pkv_alloc* a) {
  if (!a) return pkv::fail(PKV_ERR_INVALID, "null allocator");
  return (int)a->free_q.size();
}

int pkv_alloc_free_list(const pkv_alloc* a, int32_t* out, int cap) {
  if (!a) return pkv::fail(PKV_ERR_INVALID, "null allocator");
  int n = 0;
  for (int32_t b : a->free_q) {
    if (n >= cap) break;
    out[n++] = b;
  }
  return n;
}

}  // extern "C"
