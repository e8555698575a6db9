// Host-side block manager for a paged KV pool: free list, per-sequence block
// tables, per-block reference counts.
//
// Paging model ("vLLM的'内存分页'到底多神奇 — PagedAttention原理图解", xxqk.cn):
//  §2  the pool is cut into fixed-size pages; a sequence's page table lists
//      the physical pages it uses, in logical order, and they need not be
//      contiguous; free pages sit on a free list; sequences with the same
//      prompt prefix may point at the same physical pages.
//  §3  phase 1: pages are taken on demand, one more each time the current
//      page fills; phase 3: a finished sequence's pages return to the free
//      list, a shared page only when its last user ends (reference count);
//      sharing is copy-on-write: a sequence about to write into a page it
//      shares gets its own copy first.
//  §4  admission control: refuse a request that cannot get its pages rather
//      than run out of memory; abort frees every page of a request.
//
// Policy choices where the page is silent: the free list is a LIFO stack
// seeded from a caller-given order; freed blocks are pushed in table order;
// append is all-or-nothing; fork shares every block, a partly filled last
// one included. Appending into a partly filled last block that is shared
// takes a fresh block first (before any new tail block), records a pending
// copy old -> new of that block, and drops one reference of the old block.
// The device copy is the caller's: pa_write_kv performs the pending copies,
// in the order they were recorded, before its scatter, so a copy sees the
// block as the device holds it then. Pending copies survive frees of
// their blocks (a later copy in the list may read one).
//
// Plain C++ (no HIP): it is built into the device library and, on its own,
// into host-only test drivers.
#pragma once

#include <cstdint>
#include <string>
#include <unordered_map>
#include <utility>
#include <vector>

namespace pa {

enum Status : int {
  kOk = 0,
  kErrInvalid = -1,
  kErrNoBlocks = -2,
  kErrUnsupported = -3,
  kErrHip = -4,
  kErrUnknownSeq = -5,
};

struct PoolStats {
  int32_t free_blocks = 0;
  int32_t used_blocks = 0;
  int32_t shared_blocks = 0;
  int64_t filled_slots = 0;
  int64_t allocated_slots = 0;
};

class BlockManager {
 public:
  // free_order: nullptr (ascending ids) or a permutation of [0, num_blocks);
  // free_order[0] is handed out first. Use Validate() first: the constructor
  // assumes valid arguments.
  BlockManager(int32_t num_blocks, int32_t block_size, const int32_t* free_order);

  static Status Validate(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                         std::string* err);

  Status Append(int64_t seq, int32_t n, int64_t* slots_out, std::string* err);
  // n_tokens more tokens for each of n distinct sequences, all-or-nothing over
  // the whole batch. slots_out: n × n_tokens, row i for seqs[i].
  Status AppendBatch(const int64_t* seqs, int32_t n, int32_t n_tokens, int64_t* slots_out,
                     std::string* err);
  Status Fork(int64_t src, int64_t dst, std::string* err);
  Status Free(int64_t seq, std::string* err);
  Status ExportTables(const int64_t* seqs, int32_t n, int32_t max_blocks, int32_t* tables,
                      int32_t* lens, std::string* err) const;
  PoolStats Stats() const;

  int32_t num_blocks() const { return num_blocks_; }
  int32_t block_size() const { return block_size_; }
  int32_t refcount(int32_t blk) const { return ref_[blk]; }
  // Blocks with more than one reference (shared prefixes, forks), kept up to
  // date by every reference change.
  int32_t shared_blocks() const { return shared_count_; }
  int32_t free_count() const { return static_cast<int32_t>(free_.size()); }

  // Block copies (src, dst) recorded by copy-on-write appends, in order.
  const std::vector<std::pair<int32_t, int32_t>>& pending_copies() const { return pending_; }
  void ClearPendingCopies() { pending_.clear(); }

  // Prefix caching: append tokens whose ids are known. A block that a
  // token-aware append fills completely is registered under a key that
  // stands for the ids of every token from position 0 to the block's end.
  // When such an append reaches a block boundary, the following full blocks
  // of new tokens are looked up in order, and while they are found they are
  // shared (refcount + 1; a cached block with refcount 0 is taken back off
  // the free list) instead of allocated; their slots are reported as -1 (the
  // K/V is already in the pool) and counted in *n_cached. Lookups stop at
  // the first miss. A registered block keeps its key after it is freed, until
  // it is handed out again. Physical order of a call: cached blocks taken,
  // then the copy-on-write block, then fresh blocks in logical order.
  // A sequence whose tokens did not all arrive through AppendTokens (created
  // or grown by Append) is not keyed, and AppendTokens on it is Append.
  Status AppendTokens(int64_t seq, const int32_t* tokens, int32_t n, int64_t* slots_out, int32_t* n_cached,
                      std::string* err);
  struct PrefixStats {
    int32_t cached_blocks = 0;  // blocks holding a registered key (in use or free)
    int64_t lookups = 0;        // full blocks looked up
    int64_t hits = 0;           // of which found
  };
  PrefixStats prefix_stats() const;

 private:
  struct Seq {
    std::vector<int32_t> table;
    int64_t len = 0;
    bool keyed = false;                // every token arrived through AppendTokens
    uint64_t key = 0;                  // key of the full blocks so far (kRootKey when none)
    std::vector<int32_t> tail_tokens;  // ids of the tokens in a partly filled last block
  };
  struct CacheEntry {
    int32_t block;
    uint64_t parent;
    std::vector<int32_t> tokens;
  };
  static constexpr uint64_t kRootKey = 14695981039346656037ull;  // FNV-1a 64-bit offset basis
  static uint64_t ChainKey(uint64_t parent, const int32_t* ids, int32_t n);
  // Pops the top of the free list and drops any key the block held.
  int32_t PopFree();
  // Grows s by n tokens (copy-on-write of a shared partly filled last block,
  // new blocks from the free list) and writes their slots. The caller has
  // checked that enough blocks are free and reserved s.table and pending_.
  void Grow(Seq& s, int32_t n, int64_t* slots_out);
  // Takes a given (cached) block off the free list.
  void TakeFree(int32_t blk);
  // One more / one fewer reference to blk; keeps shared_count_. DropRef
  // returns the new count.
  void AddRef(int32_t blk) {
    if (++ref_[static_cast<size_t>(blk)] == 2) ++shared_count_;
  }
  int32_t DropRef(int32_t blk) {
    const int32_t r = --ref_[static_cast<size_t>(blk)];
    if (r == 1) --shared_count_;
    return r;
  }
  int32_t shared_count_ = 0;
  int32_t num_blocks_;
  int32_t block_size_;
  std::vector<int32_t> free_;  // stack: back() is the next block handed out
  std::vector<int32_t> ref_;
  std::unordered_map<int64_t, Seq> seqs_;
  std::vector<std::pair<int32_t, int32_t>> pending_;
  std::unordered_map<uint64_t, CacheEntry> cache_;  // key -> registered block
  std::vector<uint64_t> block_key_;                 // key a block is registered under
  std::vector<char> block_keyed_;
  // Scratch reused by AppendBatch and ExportTables so that a steady serving
  // loop makes no heap allocation in them.
  std::vector<int64_t> scratch_ids_;
  std::vector<Seq*> scratch_grow_;
  std::vector<int64_t> scratch_created_;  // sequences a batch append created
  std::vector<int32_t> scratch_drop_;     // per block: copy-on-write references dropped so far in a batch
  std::vector<int32_t> scratch_dropped_;  // blocks with a non-zero scratch_drop_ entry
  mutable std::vector<const Seq*> scratch_seqs_;
  PrefixStats pstats_;
};

}  // namespace pa
