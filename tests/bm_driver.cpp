// Host-only driver for the C++ block manager, built by the tests with g++
// (optionally under AddressSanitizer/UBSan). Reads an op stream on stdin and
// prints every result, so the tests can compare it with the Python model.
//
// Input:  nb bs k order[0..k)   (k = 0: ascending order)
//         then lines: a <seq> <n> | b <n_tokens> <n> <ids...> | f <src> <dst> | x <seq> |
//                     t <mb> <n> <ids...> | k <seq> <n> <token ids...> | s
// Output: one line per op.
#include <cstdio>
#include <string>
#include <vector>

#include "block_manager.h"

int main() {
  int nb, bs, k;
  if (std::scanf("%d %d %d", &nb, &bs, &k) != 3) return 2;
  std::vector<int32_t> order(static_cast<size_t>(k));
  for (int i = 0; i < k; ++i) std::scanf("%d", &order[static_cast<size_t>(i)]);
  std::string err;
  if (pa::BlockManager::Validate(nb, bs, k ? order.data() : nullptr, &err) != pa::kOk) {
    std::printf("invalid\n");
    return 0;
  }
  pa::BlockManager bm(nb, bs, k ? order.data() : nullptr);
  char op[4];
  while (std::scanf("%3s", op) == 1) {
    if (op[0] == 'a') {
      long long seq;
      int n;
      std::scanf("%lld %d", &seq, &n);
      std::vector<int64_t> slots(static_cast<size_t>(n > 0 ? n : 0));
      int st = bm.Append(seq, n, slots.data(), &err);
      std::printf("%d", st);
      if (st == 0)
        for (int64_t s : slots) std::printf(" %lld", static_cast<long long>(s));
      std::printf("\n");
    } else if (op[0] == 'b') {
      int nt, n;
      std::scanf("%d %d", &nt, &n);
      std::vector<int64_t> ids(static_cast<size_t>(n));
      for (int i = 0; i < n; ++i) {
        long long v;
        std::scanf("%lld", &v);
        ids[static_cast<size_t>(i)] = v;
      }
      std::vector<int64_t> slots(static_cast<size_t>(n) * (nt > 0 ? nt : 0) + 1);
      int st = bm.AppendBatch(ids.data(), n, nt, slots.data(), &err);
      std::printf("%d", st);
      if (st == 0)
        for (int i = 0; i < n * nt; ++i) std::printf(" %lld", static_cast<long long>(slots[static_cast<size_t>(i)]));
      std::printf("\n");
    } else if (op[0] == 'k') {
      long long seq;
      int n;
      std::scanf("%lld %d", &seq, &n);
      std::vector<int32_t> toks(static_cast<size_t>(n) + 1);
      for (int i = 0; i < n; ++i) std::scanf("%d", &toks[static_cast<size_t>(i)]);
      std::vector<int64_t> slots(static_cast<size_t>(n) + 1);
      int32_t cached = 0;
      int st = bm.AppendTokens(seq, toks.data(), n, slots.data(), &cached, &err);
      std::printf("%d", st);
      if (st == 0) {
        std::printf(" %d", cached);
        for (int i = 0; i < n; ++i) std::printf(" %lld", static_cast<long long>(slots[static_cast<size_t>(i)]));
      }
      std::printf("\n");
    } else if (op[0] == 'f') {
      long long a, b;
      std::scanf("%lld %lld", &a, &b);
      std::printf("%d\n", bm.Fork(a, b, &err));
    } else if (op[0] == 'x') {
      long long a;
      std::scanf("%lld", &a);
      std::printf("%d\n", bm.Free(a, &err));
    } else if (op[0] == 't') {
      int mb, n;
      std::scanf("%d %d", &mb, &n);
      std::vector<int64_t> ids(static_cast<size_t>(n));
      for (int i = 0; i < n; ++i) {
        long long v;
        std::scanf("%lld", &v);
        ids[static_cast<size_t>(i)] = v;
      }
      std::vector<int32_t> tab(static_cast<size_t>(n) * mb + 1), lens(static_cast<size_t>(n) + 1);
      int st = bm.ExportTables(ids.data(), n, mb, tab.data(), lens.data(), &err);
      std::printf("%d", st);
      if (st == 0) {
        for (int i = 0; i < n; ++i) std::printf(" %d", lens[static_cast<size_t>(i)]);
        for (int i = 0; i < n * mb; ++i) std::printf(" %d", tab[static_cast<size_t>(i)]);
      }
      std::printf("\n");
    } else if (op[0] == 's') {
      pa::PoolStats s = bm.Stats();
      std::printf("%d %d %d %lld %lld", s.free_blocks, s.used_blocks, s.shared_blocks,
                  static_cast<long long>(s.filled_slots), static_cast<long long>(s.allocated_slots));
      const pa::BlockManager::PrefixStats ps = bm.prefix_stats();
      std::printf(" %d %lld %lld", ps.cached_blocks, static_cast<long long>(ps.lookups),
                  static_cast<long long>(ps.hits));
      for (const auto& c : bm.pending_copies()) std::printf(" %d %d", c.first, c.second);
      std::printf("\n");
    }
  }
  return 0;
}
