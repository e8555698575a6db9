// Host block manager: see block_manager.h for the paging model it follows.
#include "block_manager.h"

#include <algorithm>
#include <climits>
#include <cstddef>

namespace pa {

namespace {
int64_t CeilDiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
}  // namespace

Status BlockManager::Validate(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                              std::string* err) {
  if (num_blocks <= 0 || block_size <= 0) {
    *err = "num_blocks and block_size must be positive";
    return kErrInvalid;
  }
  if (free_order) {
    std::vector<char> seen(static_cast<size_t>(num_blocks), 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[static_cast<size_t>(b)]) {
        *err = "free_order is not a permutation of [0, num_blocks)";
        return kErrInvalid;
      }
      seen[static_cast<size_t>(b)] = 1;
    }
  }
  return kOk;
}

BlockManager::BlockManager(int32_t num_blocks, int32_t block_size, const int32_t* free_order)
    : num_blocks_(num_blocks), block_size_(block_size),
      ref_(static_cast<size_t>(num_blocks), 0), block_key_(static_cast<size_t>(num_blocks), 0),
      block_keyed_(static_cast<size_t>(num_blocks), 0) {
  free_.resize(static_cast<size_t>(num_blocks));
  // Stack top is the back: store the hand-out order reversed.
  for (int32_t i = 0; i < num_blocks; ++i)
    free_[static_cast<size_t>(num_blocks - 1 - i)] = free_order ? free_order[i] : i;
}

Status BlockManager::Append(int64_t seq, int32_t n, int64_t* slots_out, std::string* err) {
  if (n < 0) {
    *err = "n_tokens must be >= 0";
    return kErrInvalid;
  }
  if (n > 0 && !slots_out) {
    *err = "slots_out is null";
    return kErrInvalid;
  }
  auto it = seqs_.find(seq);
  const int64_t old_len = it == seqs_.end() ? 0 : it->second.len;
  const int64_t new_len = old_len + n;
  if (new_len > static_cast<int64_t>(INT32_MAX)) {
    *err = "sequence length would exceed INT32_MAX";
    return kErrInvalid;
  }
  const int64_t have = it == seqs_.end() ? 0 : static_cast<int64_t>(it->second.table.size());
  const bool cow = n > 0 && have > 0 && old_len % block_size_ != 0 &&
                   ref_[static_cast<size_t>(it->second.table.back())] > 1;
  const int64_t tail = CeilDiv(new_len, block_size_) - have;
  const int64_t need = tail + (cow ? 1 : 0);
  if (need > static_cast<int64_t>(free_.size())) {
    *err = "not enough free blocks: need " + std::to_string(need) + ", have " +
           std::to_string(free_.size());
    return kErrNoBlocks;
  }
  // Everything that can throw happens before the first mutation.
  if (cow) pending_.reserve(pending_.size() + 1);
  if (it == seqs_.end()) it = seqs_.try_emplace(seq).first;
  Seq& s = it->second;
  s.table.reserve(static_cast<size_t>(have + tail));
  Grow(s, n, slots_out);
  return kOk;
}

void BlockManager::Grow(Seq& s, int32_t n, int64_t* slots_out) {
  const int64_t old_len = s.len;
  const int64_t new_len = old_len + n;
  const int64_t have = static_cast<int64_t>(s.table.size());
  const bool cow = n > 0 && have > 0 && old_len % block_size_ != 0 &&
                   ref_[static_cast<size_t>(s.table.back())] > 1;
  const int64_t tail = CeilDiv(new_len, block_size_) - have;
  if (n > 0) {  // token ids unknown from here on: no prefix keys for this sequence
    s.keyed = false;
    s.tail_tokens.clear();
  }
  if (cow) {  // the shared, partly filled last block: this sequence writes into its own copy
    const int32_t old_blk = s.table.back();
    const int32_t blk = PopFree();
    AddRef(blk);
    DropRef(old_blk);
    s.table.back() = blk;
    pending_.emplace_back(old_blk, blk);
  }
  for (int64_t i = 0; i < tail; ++i) {
    const int32_t blk = PopFree();
    AddRef(blk);
    s.table.push_back(blk);
  }
  s.len = new_len;
  const int64_t bs = block_size_;
  for (int64_t p = old_len; p < new_len; ++p)
    slots_out[p - old_len] = static_cast<int64_t>(s.table[static_cast<size_t>(p / bs)]) * bs + p % bs;
}

Status BlockManager::AppendBatch(const int64_t* seqs, int32_t n, int32_t n_tokens,
                                 int64_t* slots_out, std::string* err) {
  if (n < 0 || n_tokens < 0) {
    *err = "n and n_tokens must be >= 0";
    return kErrInvalid;
  }
  if (n == 0) return kOk;
  if (!seqs || (n_tokens > 0 && !slots_out)) {
    *err = "null pointer argument";
    return kErrInvalid;
  }
  // Validate the whole batch and count its new blocks before any mutation.
  scratch_ids_.assign(seqs, seqs + n);
  std::sort(scratch_ids_.begin(), scratch_ids_.end());
  const auto dup = std::adjacent_find(scratch_ids_.begin(), scratch_ids_.end());
  if (dup != scratch_ids_.end()) {
    *err = "sequence " + std::to_string(*dup) + " appears twice in the batch";
    return kErrInvalid;
  }
  // References dropped by copies earlier in the batch, per block (a member
  // array of num_blocks counters, reset below for the blocks touched).
  scratch_drop_.resize(ref_.size(), 0);
  scratch_dropped_.clear();
  int64_t need = 0;
  scratch_grow_.resize(static_cast<size_t>(n));
  for (int32_t i = 0; i < n; ++i) {
    auto it = seqs_.find(seqs[i]);
    scratch_grow_[static_cast<size_t>(i)] = it == seqs_.end() ? nullptr : &it->second;
    const int64_t old_len = it == seqs_.end() ? 0 : it->second.len;
    const int64_t have = it == seqs_.end() ? 0 : static_cast<int64_t>(it->second.table.size());
    if (old_len + n_tokens > static_cast<int64_t>(INT32_MAX)) {
      for (int32_t blk : scratch_dropped_) scratch_drop_[static_cast<size_t>(blk)] = 0;
      *err = "sequence length would exceed INT32_MAX";
      return kErrInvalid;
    }
    need += CeilDiv(old_len + n_tokens, block_size_) - have;
    // A copy-on-write of a shared partial last block needs one more block;
    // an earlier copy in the same batch may have left it with one user.
    if (n_tokens > 0 && have > 0 && old_len % block_size_ != 0 &&
        ref_[static_cast<size_t>(it->second.table.back())] > 1) {
      const int32_t last = it->second.table.back();
      int32_t& dropped = scratch_drop_[static_cast<size_t>(last)];
      if (ref_[static_cast<size_t>(last)] - dropped > 1) {
        if (dropped == 0) scratch_dropped_.push_back(last);
        ++need;
        ++dropped;
      }
    }
  }
  for (int32_t blk : scratch_dropped_) scratch_drop_[static_cast<size_t>(blk)] = 0;
  if (need > static_cast<int64_t>(free_.size())) {
    *err = "not enough free blocks for the batch: need " + std::to_string(need) + ", have " +
           std::to_string(free_.size());
    return kErrNoBlocks;
  }
  // New sequences are created before any block moves, so an allocation
  // failure here leaves the pool unchanged apart from empty entries, which
  // are removed again.
  // (Pointers to map entries stay valid while other entries are inserted.)
  std::vector<int64_t>& created = scratch_created_;
  created.clear();
  created.reserve(static_cast<size_t>(n));  // so recording a new entry cannot throw
  try {
    for (int32_t i = 0; i < n; ++i) {
      Seq*& ps = scratch_grow_[static_cast<size_t>(i)];
      if (!ps) {
        ps = &seqs_.try_emplace(seqs[i]).first->second;
        created.push_back(seqs[i]);
      }
    }
    for (int32_t i = 0; i < n; ++i) {
      Seq& s = *scratch_grow_[static_cast<size_t>(i)];
      s.table.reserve(static_cast<size_t>(CeilDiv(s.len + n_tokens, block_size_)));
    }
    pending_.reserve(pending_.size() + static_cast<size_t>(n));
  } catch (...) {
    for (int64_t id : created) seqs_.erase(id);
    throw;
  }
  for (int32_t i = 0; i < n; ++i)  // cannot fail: validated and reserved above
    Grow(*scratch_grow_[static_cast<size_t>(i)], n_tokens,
         slots_out ? slots_out + static_cast<int64_t>(i) * n_tokens : nullptr);
  return kOk;
}

Status BlockManager::Fork(int64_t src, int64_t dst, std::string* err) {
  auto it = seqs_.find(src);
  if (it == seqs_.end()) {
    *err = "unknown source sequence " + std::to_string(src);
    return kErrUnknownSeq;
  }
  if (dst == src || seqs_.count(dst)) {
    *err = "destination sequence " + std::to_string(dst) + " already exists";
    return kErrInvalid;
  }
  Seq copy = it->second;  // may throw before any mutation
  for (int32_t blk : copy.table) AddRef(blk);
  seqs_.emplace(dst, std::move(copy));
  return kOk;
}

Status BlockManager::Free(int64_t seq, std::string* err) {
  auto it = seqs_.find(seq);
  if (it == seqs_.end()) {
    *err = "unknown sequence " + std::to_string(seq);
    return kErrUnknownSeq;
  }
  // free_ never exceeds num_blocks_ entries: reserve once so push_back cannot throw.
  free_.reserve(static_cast<size_t>(num_blocks_));
  for (int32_t blk : it->second.table) {
    if (DropRef(blk) == 0) {
      // A pending copy into this block stays: a later copy may read the
      // block, and the scatter that follows the copies overwrites whatever
      // rows a new owner gets.
      free_.push_back(blk);
    }
  }
  seqs_.erase(it);
  return kOk;
}

Status BlockManager::ExportTables(const int64_t* seqs, int32_t n, int32_t max_blocks,
                                  int32_t* tables, int32_t* lens, std::string* err) const {
  if (n < 0 || max_blocks < 0) {
    *err = "n and max_blocks must be >= 0";
    return kErrInvalid;
  }
  if (n > 0 && (!seqs || !lens || (max_blocks > 0 && !tables))) {
    *err = "null pointer argument";
    return kErrInvalid;
  }
  scratch_seqs_.resize(static_cast<size_t>(n));
  for (int32_t i = 0; i < n; ++i) {  // validate all before writing anything
    auto it = seqs_.find(seqs[i]);
    if (it == seqs_.end()) {
      *err = "unknown sequence " + std::to_string(seqs[i]);
      return kErrUnknownSeq;
    }
    if (static_cast<int64_t>(it->second.table.size()) > max_blocks) {
      *err = "sequence " + std::to_string(seqs[i]) + " needs more than max_blocks table entries";
      return kErrInvalid;
    }
    scratch_seqs_[static_cast<size_t>(i)] = &it->second;
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = *scratch_seqs_[static_cast<size_t>(i)];
    int32_t* row = tables + static_cast<int64_t>(i) * max_blocks;
    std::copy(s.table.begin(), s.table.end(), row);
    std::fill(row + s.table.size(), row + max_blocks, -1);
    lens[i] = static_cast<int32_t>(s.len);
  }
  return kOk;
}

PoolStats BlockManager::Stats() const {
  PoolStats st;
  std::vector<int32_t> fill(static_cast<size_t>(num_blocks_), 0);
  const int64_t bs = block_size_;
  for (const auto& kv : seqs_) {
    const Seq& s = kv.second;
    for (size_t i = 0; i < s.table.size(); ++i) {
      int64_t f = std::min<int64_t>(bs, s.len - static_cast<int64_t>(i) * bs);
      int32_t& cur = fill[static_cast<size_t>(s.table[i])];
      cur = std::max<int32_t>(cur, static_cast<int32_t>(f));
    }
  }
  for (int32_t b = 0; b < num_blocks_; ++b) {
    int32_t r = ref_[static_cast<size_t>(b)];
    if (r > 0) ++st.used_blocks;
    st.filled_slots += fill[static_cast<size_t>(b)];
  }
  st.shared_blocks = shared_count_;
  st.free_blocks = static_cast<int32_t>(free_.size());
  st.allocated_slots = static_cast<int64_t>(st.used_blocks) * bs;
  return st;
}

int32_t BlockManager::PopFree() {
  const int32_t blk = free_.back();
  free_.pop_back();
  const size_t b = static_cast<size_t>(blk);
  if (block_keyed_[b]) {  // new contents: its key no longer describes it
    cache_.erase(block_key_[b]);
    block_keyed_[b] = 0;
  }
  return blk;
}

void BlockManager::TakeFree(int32_t blk) {
  free_.erase(std::find(free_.begin(), free_.end(), blk));
}

// 64-bit FNV-1a (Fowler, Noll, Vo) over the parent key's 8 bytes and the
// block's token ids, 4 bytes each, least significant byte first.
uint64_t BlockManager::ChainKey(uint64_t parent, const int32_t* ids, int32_t n) {
  constexpr uint64_t kPrime = 1099511628211ull;
  uint64_t h = kRootKey;
  for (int i = 0; i < 8; ++i) {
    h ^= (parent >> (8 * i)) & 0xFFu;
    h *= kPrime;
  }
  for (int32_t t = 0; t < n; ++t) {
    const uint32_t v = static_cast<uint32_t>(ids[t]);
    for (int i = 0; i < 4; ++i) {
      h ^= (v >> (8 * i)) & 0xFFu;
      h *= kPrime;
    }
  }
  return h;
}

Status BlockManager::AppendTokens(int64_t seq, const int32_t* tokens, int32_t n, int64_t* slots_out,
                                  int32_t* n_cached, std::string* err) {
  if (n < 0) {
    *err = "n_tokens must be >= 0";
    return kErrInvalid;
  }
  if (!n_cached || (n > 0 && (!tokens || !slots_out))) {
    *err = "null pointer argument";
    return kErrInvalid;
  }
  auto it = seqs_.find(seq);
  if (it != seqs_.end() && !it->second.keyed) {
    *n_cached = 0;
    return Append(seq, n, slots_out, err);
  }
  const int64_t bs = block_size_;
  const int64_t old_len = it == seqs_.end() ? 0 : it->second.len;
  const int64_t new_len = old_len + n;
  if (new_len > static_cast<int64_t>(INT32_MAX)) {
    *err = "sequence length would exceed INT32_MAX";
    return kErrInvalid;
  }
  const int64_t have = it == seqs_.end() ? 0 : static_cast<int64_t>(it->second.table.size());
  const int64_t r = old_len % bs;
  const int64_t fill = r ? std::min<int64_t>(n, bs - r) : 0;  // into the partly filled last block
  const bool cow = fill > 0 && ref_[static_cast<size_t>(it->second.table.back())] > 1;

  // Keys of the blocks this call completes, and lookups of the full blocks
  // that start at a block boundary (until the first miss).
  uint64_t key = it == seqs_.end() ? kRootKey : it->second.key;
  bool completes_tail = false;
  uint64_t tail_key = 0;
  std::vector<int32_t> ids;
  if (r && r + fill == bs) {
    ids = it->second.tail_tokens;
    ids.insert(ids.end(), tokens, tokens + fill);
    tail_key = ChainKey(key, ids.data(), static_cast<int32_t>(bs));
    key = tail_key;
    completes_tail = true;
  }
  struct Planned {
    uint64_t key;
    uint64_t parent;
    int32_t hit;  // cached block, or -1
  };
  std::vector<Planned> full;
  int64_t pos = fill;
  bool searching = true;
  int64_t lookups = 0, free_hits = 0, hits = 0;
  while (n - pos >= bs) {
    const int32_t* blk_ids = tokens + pos;
    const uint64_t k = ChainKey(key, blk_ids, static_cast<int32_t>(bs));
    int32_t hit = -1;
    if (searching) {
      ++lookups;
      auto c = cache_.find(k);
      if (c != cache_.end() && c->second.parent == key &&
          std::equal(c->second.tokens.begin(), c->second.tokens.end(), blk_ids)) {
        hit = c->second.block;
        ++hits;
        if (ref_[static_cast<size_t>(hit)] == 0) ++free_hits;
      } else {
        searching = false;
      }
    }
    full.push_back({k, key, hit});
    key = k;
    pos += bs;
  }
  const int64_t rem = n - pos;
  const int64_t fresh = static_cast<int64_t>(full.size()) - hits + (rem > 0 ? 1 : 0);
  const int64_t need = free_hits + (cow ? 1 : 0) + fresh;
  if (need > static_cast<int64_t>(free_.size())) {
    *err = "not enough free blocks: need " + std::to_string(need) + ", have " + std::to_string(free_.size());
    return kErrNoBlocks;
  }
  // Everything that can throw happens before the first mutation.
  if (cow) pending_.reserve(pending_.size() + 1);
  cache_.reserve(cache_.size() + full.size() + 1);
  if (it == seqs_.end()) {
    it = seqs_.emplace(seq, Seq{}).first;
    it->second.keyed = true;
    it->second.key = kRootKey;
  }
  Seq& s = it->second;
  s.table.reserve(static_cast<size_t>(CeilDiv(new_len, bs)));
  // ids of the tokens in the partly filled last block after the call
  std::vector<int32_t> new_tail;
  const int64_t t_len = new_len % bs;
  if (t_len > 0 && t_len <= n) {
    new_tail.assign(tokens + (n - t_len), tokens + n);
  } else if (t_len > n) {  // the call stays inside the old partial block
    new_tail = s.tail_tokens;
    new_tail.insert(new_tail.end(), tokens, tokens + n);
  }

  // (1) cached blocks taken
  for (const Planned& f : full)
    if (f.hit >= 0) {
      if (ref_[static_cast<size_t>(f.hit)] == 0) TakeFree(f.hit);
      AddRef(f.hit);
    }
  // (2) the copy-on-write block
  if (cow) {
    const int32_t old_blk = s.table.back();
    const int32_t blk = PopFree();
    AddRef(blk);
    DropRef(old_blk);
    s.table.back() = blk;
    pending_.emplace_back(old_blk, blk);
  }
  // (3) fresh blocks in logical order
  auto reg = [&](uint64_t k, uint64_t parent, int32_t blk, const int32_t* blk_ids) {
    if (cache_.count(k)) return;  // an equal block is already registered (or a key collision)
    cache_.emplace(k, CacheEntry{blk, parent, std::vector<int32_t>(blk_ids, blk_ids + bs)});
    block_key_[static_cast<size_t>(blk)] = k;
    block_keyed_[static_cast<size_t>(blk)] = 1;
  };
  for (const Planned& f : full) {
    if (f.hit >= 0) {
      s.table.push_back(f.hit);
      continue;
    }
    const int32_t blk = PopFree();
    AddRef(blk);
    s.table.push_back(blk);
  }
  if (rem > 0) {
    const int32_t blk = PopFree();
    AddRef(blk);
    s.table.push_back(blk);
  }
  // registration of the blocks this call filled
  if (completes_tail) reg(tail_key, s.key, s.table[static_cast<size_t>(have - 1)], ids.data());
  for (size_t i = 0; i < full.size(); ++i)
    if (full[i].hit < 0)
      reg(full[i].key, full[i].parent, s.table[static_cast<size_t>(have) + i],
          tokens + fill + static_cast<int64_t>(i) * bs);

  // slots: -1 where the K/V is already in a cached block
  int32_t cached = 0;
  for (int64_t p = old_len; p < new_len; ++p) {
    const int64_t lb = p / bs;
    const int64_t i = lb - have;  // index into `full` when p sits in a planned full block
    const bool in_full = p - old_len >= fill && i >= 0 && i < static_cast<int64_t>(full.size());
    if (in_full && full[static_cast<size_t>(i)].hit >= 0) {
      slots_out[p - old_len] = -1;
      ++cached;
    } else {
      slots_out[p - old_len] = static_cast<int64_t>(s.table[static_cast<size_t>(lb)]) * bs + p % bs;
    }
  }
  *n_cached = cached;
  s.len = new_len;
  s.key = key;
  s.tail_tokens = std::move(new_tail);
  pstats_.lookups += lookups;
  pstats_.hits += hits;
  return kOk;
}

BlockManager::PrefixStats BlockManager::prefix_stats() const {
  PrefixStats p = pstats_;
  p.cached_blocks = static_cast<int32_t>(cache_.size());
  return p;
}

}  // namespace pa
