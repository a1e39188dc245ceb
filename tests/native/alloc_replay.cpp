// Test aid: replays allocator and host-planning calls of libpkv's host code,
// read one command per line from stdin, and prints one result line each.
// Built by tests/test_sanitized_host.py with g++ -fsanitize=address,undefined
// against allocator.cpp and host.cpp only (no HIP), so every call the CPU
// tests make against the specification model also runs under the
// sanitizers.
//
// Commands (integers separated by spaces):
//   new NB BS K o_0 .. o_{K-1}   create (K = 0: default free order)
//   add S | fork P C | free S | touch S | pool N
//   append S N                    -> rc, slots, copy-on-write pairs
//   out S | in S                  -> rc, swap pairs
//   lru | lfu                     -> rc, sequence
//   state K s_0 .. s_{K-1}        -> free list, refcounts, host free count,
//                                    then len / swapped / table of each s_i
//   poff P N L_0 ..               -> rc, partition offsets
//   toff BS N L_0 ..              -> rc, tile offsets
//   plan BS P HQ HKV N L_0 .. NG GO_0 .. GO_NG GB_0 .. GB_{NG-1}
//                                 -> rc, rows, suffixes, token starts,
//                                    prefix items, totals

#include <cstdint>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "pkv.h"

namespace {

template <class T>
void put(std::ostream& o, const std::vector<T>& v) {
  o << ' ' << v.size();
  for (const T& x : v) o << ' ' << (long long)x;
}

std::vector<int32_t> read_ints(std::istringstream& in, long long n) {
  std::vector<int32_t> v;
  for (long long i = 0; i < n; ++i) {
    long long x = 0;
    in >> x;
    v.push_back((int32_t)x);
  }
  return v;
}

}  // namespace

int main() {
  std::ios::sync_with_stdio(false);
  pkv_alloc* a = nullptr;
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string cmd;
    in >> cmd;
    std::ostringstream out;
    if (cmd == "new") {
      long long nb = 0, bs = 0, k = 0;
      in >> nb >> bs >> k;
      const std::vector<int32_t> order = read_ints(in, k);
      if (a) pkv_alloc_destroy(a);
      a = pkv_alloc_create((int)nb, (int)bs, k ? order.data() : nullptr);
      out << "rc " << (a ? 0 : -1);
    } else if (cmd == "add" || cmd == "free" || cmd == "touch" || cmd == "pool") {
      long long s = 0;
      in >> s;
      const int rc = cmd == "add"    ? pkv_alloc_add_seq(a, s)
                     : cmd == "free" ? pkv_alloc_free_seq(a, s)
                     : cmd == "touch" ? pkv_alloc_touch(a, s)
                                      : pkv_alloc_set_host_pool(a, (int)s);
      out << "rc " << rc;
    } else if (cmd == "fork") {
      long long p = 0, c = 0;
      in >> p >> c;
      out << "rc " << pkv_alloc_fork(a, p, c);
    } else if (cmd == "append") {
      long long s = 0, n = 0;
      in >> s >> n;
      std::vector<int32_t> slots(n > 0 ? (size_t)n : 0), cow(2);
      int ncow = 0;
      const int rc = pkv_alloc_append(a, s, (int)n, slots.empty() ? nullptr : slots.data(),
                                      cow.data(), 1, &ncow);
      out << "rc " << rc;
      if (rc == PKV_OK) {
        put(out, slots);
        cow.resize(2 * (size_t)ncow);
        put(out, cow);
      }
    } else if (cmd == "out" || cmd == "in") {
      long long s = 0;
      in >> s;
      const int64_t len = pkv_alloc_seq_len(a, s);
      const int cap = len > 0 ? (int)(len / 1 + 1) : 1;   // >= table length for any block size
      std::vector<int32_t> pairs(2 * (size_t)cap);
      int n = 0;
      const int rc = cmd == "out" ? pkv_alloc_swap_out(a, s, pairs.data(), cap, &n)
                                  : pkv_alloc_swap_in(a, s, pairs.data(), cap, &n);
      out << "rc " << rc;
      if (rc == PKV_OK) {
        pairs.resize(2 * (size_t)n);
        put(out, pairs);
      }
    } else if (cmd == "lru" || cmd == "lfu") {
      int64_t s = -1;
      const int rc = cmd == "lru" ? pkv_alloc_lru(a, &s) : pkv_alloc_lfu(a, &s);
      out << "rc " << rc;
      if (rc == PKV_OK) out << ' ' << (long long)s;
    } else if (cmd == "state") {
      long long k = 0;
      in >> k;
      const int nfree = pkv_alloc_num_free(a);
      std::vector<int32_t> fl(nfree > 0 ? (size_t)nfree : 0);
      const int got = pkv_alloc_free_list(a, fl.data(), nfree);
      fl.resize(got > 0 ? (size_t)got : 0);
      out << "free";
      put(out, fl);
      std::vector<int32_t> ref;
      for (int32_t b = 0; pkv_alloc_refcount(a, b) >= 0; ++b) ref.push_back(pkv_alloc_refcount(a, b));
      out << " ref";
      put(out, ref);
      out << " host " << pkv_alloc_num_host_free(a);
      for (long long i = 0; i < k; ++i) {
        long long s = 0;
        in >> s;
        const int len = pkv_alloc_len(a, s);
        const int64_t len64 = pkv_alloc_seq_len(a, s);
        const int sw = pkv_alloc_is_swapped(a, s);
        std::vector<int32_t> tab((size_t)(len64 > 0 ? len64 : 0) + 1);
        int n = 0;
        const int rc = pkv_alloc_block_table(a, s, tab.data(), (int)tab.size(), &n);
        tab.resize(rc == PKV_OK ? (size_t)n : 0);
        out << " seq " << s << ' ' << len << ' ' << (long long)len64 << ' ' << sw;
        put(out, tab);
      }
    } else if (cmd == "poff" || cmd == "toff") {
      long long p = 0, n = 0;
      in >> p >> n;
      const std::vector<int32_t> lens = read_ints(in, n);
      std::vector<int32_t> off((size_t)n + 1);
      int tot = -1;
      const int rc = cmd == "poff"
                         ? paged_attention_partition_offsets(lens.data(), (int)n, (int)p,
                                                             off.data(), &tot)
                         : paged_attention_tile_offsets(lens.data(), (int)n, (int)p, off.data(),
                                                        &tot);
      out << "rc " << rc;
      if (rc == PKV_OK) {
        put(out, off);
        out << ' ' << tot;
      }
    } else if (cmd == "plan") {
      long long bs = 0, p = 0, hq = 0, hkv = 0, n = 0, ng = 0;
      in >> bs >> p >> hq >> hkv >> n;
      const std::vector<int32_t> lens = read_ints(in, n);
      in >> ng;
      const std::vector<int32_t> go = read_ints(in, ng + 1);
      const std::vector<int32_t> gb = read_ints(in, ng);
      std::vector<int32_t> rows((size_t)n + 1), suf((size_t)n + 1), ts((size_t)n + 1),
          pre((size_t)ng + 1), tot(3);
      const int rc = paged_attention_prefix_plan(lens.data(), (int)n, go.data(), gb.data(),
                                                 (int)ng, (int)bs, (int)p, (int)hq, (int)hkv,
                                                 rows.data(), suf.data(), ts.data(), pre.data(),
                                                 tot.data());
      out << "rc " << rc;
      if (rc == PKV_OK) {
        ts.resize((size_t)n);
        put(out, rows);
        put(out, suf);
        put(out, ts);
        put(out, pre);
        put(out, tot);
      }
    } else {
      out << "unknown";
    }
    std::cout << out.str() << '\n' << std::flush;
  }
  if (a) pkv_alloc_destroy(a);
  return 0;
}
