// C ABI of the paged-attention library: argument validation, error state,
// pool handles, and dispatch to the HIP kernels. Declarations and their
// contracts are in include/pa.h.
#include "pa.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <exception>
#include <new>
#include <string>

#include "block_manager.h"
#include "launch.h"

struct pa_pool {
  pa_kv_layout layout;
  void* k_cache;
  void* v_cache;
  pa::BlockManager bm;
  float k_scale = 1.f;  // FP8 pools: a code c stands for value(c) * scale
  float v_scale = 1.f;
  pa_pool(const pa_kv_layout& l, void* k, void* v, const int32_t* order)
      : layout(l), k_cache(k), v_cache(v), bm(l.num_blocks, l.block_size, order) {}
};

namespace {

thread_local std::string g_error;

pa_status Fail(pa_status s, const std::string& msg) {
  g_error = msg;
  return s;
}

pa_status FromHip(hipError_t e, const char* what) {
  if (e == hipSuccess) return PA_OK;
  return Fail(PA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int ElemBytes(int32_t dtype) { return dtype == PA_F32 ? 4 : dtype == PA_BF16 ? 2 : 1; }

bool Aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

pa_status CheckLayout(const pa_kv_layout& l) {
  if (l.num_blocks <= 0 || l.block_size <= 0 || l.num_kv_heads <= 0 || l.head_dim <= 0)
    return Fail(PA_ERR_INVALID, "layout sizes must be positive");
  if (l.dtype != PA_F32 && l.dtype != PA_BF16 && l.dtype != PA_FP8_E4M3)
    return Fail(PA_ERR_UNSUPPORTED, "dtype must be PA_F32, PA_BF16 or PA_FP8_E4M3");
  if (l.head_dim != 64 && l.head_dim != 128) return Fail(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (l.dtype == PA_FP8_E4M3 && l.head_dim != 128)
    return Fail(PA_ERR_UNSUPPORTED, "PA_FP8_E4M3 pools need head_dim 128");
  if (l.block_size != 8 && l.block_size != 16 && l.block_size != 32)
    return Fail(PA_ERR_UNSUPPORTED, "block_size must be 8, 16 or 32");
  const int64_t slots = static_cast<int64_t>(l.num_blocks) * l.block_size;
  if (slots * l.num_kv_heads * l.head_dim > (int64_t{1} << 40))
    return Fail(PA_ERR_UNSUPPORTED, "pool too large");
  return PA_OK;
}

template <typename F>
pa_status Guard(F&& f) {
  try {
    return f();
  } catch (const std::bad_alloc&) {
    return Fail(PA_ERR_INVALID, "host allocation failed");
  } catch (const std::exception& e) {
    return Fail(PA_ERR_INVALID, e.what());
  } catch (...) {
    return Fail(PA_ERR_INVALID, "unknown exception");
  }
}

pa_status FromBm(pa::Status s, const std::string& err) {
  return s == pa::kOk ? PA_OK : Fail(static_cast<pa_status>(s), err);
}

pa_status CheckHeads(const pa_pool* pool, int32_t Hq, int32_t* G) {
  const int32_t Hkv = pool->layout.num_kv_heads;
  if (Hq <= 0) return Fail(PA_ERR_INVALID, "num_q_heads must be positive");
  if (Hq % Hkv) return Fail(PA_ERR_INVALID, "num_q_heads must be a multiple of num_kv_heads");
  *G = Hq / Hkv;
  if (*G != 1 && *G != 2 && *G != 4 && *G != 8)
    return Fail(PA_ERR_UNSUPPORTED, "num_q_heads / num_kv_heads must be 1, 2, 4 or 8");
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_last_error(void) { return g_error.c_str(); }

pa_status pa_alloc_pool(const pa_kv_layout* layout, void* k_cache, void* v_cache,
                        const int32_t* free_order, pa_pool** out) {
  return Guard([&]() -> pa_status {
    if (!layout || !k_cache || !v_cache || !out) return Fail(PA_ERR_INVALID, "null argument");
    pa_status s = CheckLayout(*layout);
    if (s != PA_OK) return s;
    if (!Aligned16(k_cache) || !Aligned16(v_cache))
      return Fail(PA_ERR_INVALID, "k_cache and v_cache must be 16-byte aligned");
    std::string err;
    if (pa::BlockManager::Validate(layout->num_blocks, layout->block_size, free_order, &err) != pa::kOk)
      return Fail(PA_ERR_INVALID, err);
    *out = new pa_pool(*layout, k_cache, v_cache, free_order);
    return PA_OK;
  });
}

void pa_free_pool(pa_pool* pool) { delete pool; }

pa_status pa_seq_append(pa_pool* pool, int64_t seq_id, int32_t n_tokens, int64_t* slots_out) {
  return Guard([&]() -> pa_status {
    if (!pool) return Fail(PA_ERR_INVALID, "null pool");
    std::string err;
    return FromBm(pool->bm.Append(seq_id, n_tokens, slots_out, &err), err);
  });
}

pa_status pa_seq_append_batch(pa_pool* pool, const int64_t* seq_ids, int32_t n, int32_t n_tokens,
                              int64_t* slots_out) {
  return Guard([&]() -> pa_status {
    if (!pool) return Fail(PA_ERR_INVALID, "null pool");
    std::string err;
    return FromBm(pool->bm.AppendBatch(seq_ids, n, n_tokens, slots_out, &err), err);
  });
}

pa_status pa_seq_fork(pa_pool* pool, int64_t src_seq_id, int64_t dst_seq_id) {
  return Guard([&]() -> pa_status {
    if (!pool) return Fail(PA_ERR_INVALID, "null pool");
    std::string err;
    return FromBm(pool->bm.Fork(src_seq_id, dst_seq_id, &err), err);
  });
}

pa_status pa_seq_free(pa_pool* pool, int64_t seq_id) {
  return Guard([&]() -> pa_status {
    if (!pool) return Fail(PA_ERR_INVALID, "null pool");
    std::string err;
    return FromBm(pool->bm.Free(seq_id, &err), err);
  });
}

pa_status pa_block_tables(const pa_pool* pool, const int64_t* seq_ids, int32_t n, int32_t max_blocks,
                          int32_t* tables_out, int32_t* seq_lens_out) {
  return Guard([&]() -> pa_status {
    if (!pool) return Fail(PA_ERR_INVALID, "null pool");
    std::string err;
    return FromBm(pool->bm.ExportTables(seq_ids, n, max_blocks, tables_out, seq_lens_out, &err), err);
  });
}

pa_status pa_pool_stats(const pa_pool* pool, pa_pool_stats_t* out) {
  return Guard([&]() -> pa_status {
    if (!pool || !out) return Fail(PA_ERR_INVALID, "null argument");
    pa::PoolStats s = pool->bm.Stats();
    out->free_blocks = s.free_blocks;
    out->used_blocks = s.used_blocks;
    out->shared_blocks = s.shared_blocks;
    out->pending_copies = static_cast<int32_t>(pool->bm.pending_copies().size());
    out->filled_slots = s.filled_slots;
    out->allocated_slots = s.allocated_slots;
    return PA_OK;
  });
}

pa_status pa_pool_pending_copies(const pa_pool* pool, int32_t* src_out, int32_t* dst_out, int32_t capacity,
                                 int32_t* n_out) {
  return Guard([&]() -> pa_status {
    if (!pool || !n_out) return Fail(PA_ERR_INVALID, "null argument");
    const auto& pend = pool->bm.pending_copies();
    const int32_t n = static_cast<int32_t>(pend.size());
    if (capacity < n) return Fail(PA_ERR_INVALID, "capacity smaller than the pending copy count");
    if (n > 0 && (!src_out || !dst_out)) return Fail(PA_ERR_INVALID, "null argument");
    for (int32_t i = 0; i < n; ++i) {
      src_out[i] = pend[static_cast<size_t>(i)].first;
      dst_out[i] = pend[static_cast<size_t>(i)].second;
    }
    *n_out = n;
    return PA_OK;
  });
}

pa_status pa_pool_set_kv_scales(pa_pool* pool, float k_scale, float v_scale) {
  return Guard([&]() -> pa_status {
    if (!pool) return Fail(PA_ERR_INVALID, "null pool");
    if (pool->layout.dtype != PA_FP8_E4M3) return Fail(PA_ERR_UNSUPPORTED, "kv scales apply to FP8 pools only");
    if (!(k_scale > 0.f) || !(v_scale > 0.f) || k_scale > 3.0e38f || v_scale > 3.0e38f)
      return Fail(PA_ERR_INVALID, "scales must be finite and > 0");
    pool->k_scale = k_scale;
    pool->v_scale = v_scale;
    return PA_OK;
  });
}

pa_status pa_write_kv(pa_pool* pool, const void* key, const void* value, const int64_t* slot_mapping,
                      int32_t T, void* stream) {
  return Guard([&]() -> pa_status {
    if (!pool) return Fail(PA_ERR_INVALID, "null pool");
    if (T < 0) return Fail(PA_ERR_INVALID, "T must be >= 0");
    if (T > 0 && (!key || !value || !slot_mapping)) return Fail(PA_ERR_INVALID, "null argument");
    if (T > 0 && (!Aligned16(key) || !Aligned16(value)))
      return Fail(PA_ERR_INVALID, "key and value must be 16-byte aligned");
    // Copy-on-write copies recorded by earlier appends run first, in order.
    // Consecutive copies share a launch until one touches a block that an
    // earlier copy of the launch writes, or writes a block it reads.
    const pa_kv_layout& l = pool->layout;
    const int64_t block_bytes =
        static_cast<int64_t>(l.block_size) * l.num_kv_heads * l.head_dim * ElemBytes(l.dtype);
    pa::BlockCopyList list{};
    auto flush = [&]() -> pa_status {
      const pa_status st = FromHip(pa::LaunchCopyBlocks(pool->k_cache, pool->v_cache, list, block_bytes,
                                                        static_cast<hipStream_t>(stream)),
                                   "copy-on-write block copy launch");
      list.n = 0;
      return st;
    };
    for (const auto& cp : pool->bm.pending_copies()) {
      bool depends = list.n == pa::kMaxCopiesPerLaunch;
      for (int32_t i = 0; i < list.n && !depends; ++i)
        depends = cp.first == list.dst[i] || cp.second == list.dst[i] || cp.second == list.src[i];
      if (depends) {
        const pa_status st = flush();
        if (st != PA_OK) return st;
      }
      list.src[list.n] = cp.first;
      list.dst[list.n] = cp.second;
      ++list.n;
    }
    const pa_status st = flush();
    if (st != PA_OK) return st;
    pool->bm.ClearPendingCopies();
    if (T == 0) return PA_OK;
    const int64_t row_elems = static_cast<int64_t>(l.num_kv_heads) * l.head_dim;
    const int64_t num_slots = static_cast<int64_t>(l.num_blocks) * l.block_size;
    const hipStream_t st_ = static_cast<hipStream_t>(stream);
    if (l.dtype == PA_FP8_E4M3) {
      const int64_t chunks = static_cast<int64_t>(T) * (row_elems / 16);
      if ((chunks + 255) / 256 >= (int64_t{1} << 31)) return Fail(PA_ERR_UNSUPPORTED, "T too large");
      return FromHip(pa::LaunchWriteKvFp8(key, value, slot_mapping, pool->k_cache, pool->v_cache, T, row_elems,
                                          num_slots, pool->k_scale, pool->v_scale, st_),
                     "write_kv launch");
    }
    const int64_t row_bytes = row_elems * ElemBytes(l.dtype);
    const int64_t chunks = static_cast<int64_t>(T) * (row_bytes / 16);
    if ((chunks + 255) / 256 >= (int64_t{1} << 31)) return Fail(PA_ERR_UNSUPPORTED, "T too large");
    return FromHip(pa::LaunchWriteKv(key, value, slot_mapping, pool->k_cache, pool->v_cache, T,
                                     row_bytes, num_slots, st_),
                   "write_kv launch");
  });
}

size_t pa_decode_workspace_bytes(int32_t B, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_seq_len, int32_t partition_tokens) {
  if (B < 0 || num_q_heads <= 0 || head_dim <= 0 || max_seq_len < 0 || partition_tokens < 0) return 0;
  const int32_t pt = partition_tokens == 0 ? 512 : partition_tokens;
  return pa::DecodeWorkspaceBytes(B, num_q_heads, head_dim, pa::DecodePartitions(max_seq_len, pt));
}

pa_status pa_decode(pa_pool* pool, void* out, const void* q, const int32_t* block_tables,
                    int32_t max_blocks, const int32_t* seq_lens, int32_t B, int32_t num_q_heads,
                    float scale, int32_t max_seq_len, int32_t partition_tokens, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return Guard([&]() -> pa_status {
    if (!pool) return Fail(PA_ERR_INVALID, "null pool");
    if (B < 0 || max_blocks < 0 || max_seq_len < 0 || partition_tokens < 0)
      return Fail(PA_ERR_INVALID, "negative size argument");
    int32_t G = 0;
    pa_status s = CheckHeads(pool, num_q_heads, &G);
    if (s != PA_OK) return s;
    if (B == 0) return PA_OK;
    if (!out || !q || !block_tables || !seq_lens) return Fail(PA_ERR_INVALID, "null argument");
    if (!Aligned16(out) || !Aligned16(q)) return Fail(PA_ERR_INVALID, "q and out must be 16-byte aligned");
    const pa_kv_layout& l = pool->layout;
    if (static_cast<int64_t>(max_seq_len) > static_cast<int64_t>(max_blocks) * l.block_size)
      return Fail(PA_ERR_INVALID, "max_seq_len exceeds max_blocks * block_size");
    const int32_t pt = partition_tokens == 0 ? 512 : partition_tokens;
    if (pt % 64 || pt > 2048)
      return Fail(PA_ERR_UNSUPPORTED, "partition_tokens must be a multiple of 64, at most 2048");
    const int32_t P = pa::DecodePartitions(max_seq_len, pt);
    if (static_cast<int64_t>(P) * B * l.num_kv_heads >= (int64_t{1} << 31) - 8)
      return Fail(PA_ERR_UNSUPPORTED, "grid too large");
    const size_t need = pa::DecodeWorkspaceBytes(B, num_q_heads, l.head_dim, P);
    if (need && (!workspace || workspace_bytes < need))
      return Fail(PA_ERR_INVALID, "workspace too small: need " + std::to_string(need) + " bytes");
    if (need && !Aligned16(workspace)) return Fail(PA_ERR_INVALID, "workspace must be 16-byte aligned");
    pa::DecodeArgs a{};
    a.out = out;
    a.q = q;
    a.k_cache = pool->k_cache;
    a.v_cache = pool->v_cache;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.ws = workspace;
    a.B = B;
    a.Hq = num_q_heads;
    a.Hkv = l.num_kv_heads;
    a.D = l.head_dim;
    a.G = G;
    a.block_size = l.block_size;
    a.num_blocks = l.num_blocks;
    a.max_blocks = max_blocks;
    a.max_seq_len = max_seq_len;
    a.partition_tokens = pt;
    a.num_partitions = P;
    a.scale = scale;
    a.k_scale = pool->k_scale;
    a.v_scale = pool->v_scale;
    a.dtype = l.dtype;
    return FromHip(pa::LaunchDecode(a, static_cast<hipStream_t>(stream)), "decode launch");
  });
}

pa_status pa_prefill(pa_pool* pool, void* out, const void* q, const int32_t* cu_q_lens,
                     const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
                     int32_t B, int32_t num_q_heads, int32_t max_q_len, float scale, void* stream) {
  return Guard([&]() -> pa_status {
    if (!pool) return Fail(PA_ERR_INVALID, "null pool");
    if (B < 0 || max_blocks < 0 || max_q_len < 0) return Fail(PA_ERR_INVALID, "negative size argument");
    int32_t G = 0;
    pa_status s = CheckHeads(pool, num_q_heads, &G);
    if (s != PA_OK) return s;
    const pa_kv_layout& l = pool->layout;
    if (l.dtype != PA_BF16) return Fail(PA_ERR_UNSUPPORTED, "prefill supports bf16 pools only");
    if (B == 0 || max_q_len == 0) return PA_OK;
    if (!out || !q || !cu_q_lens || !block_tables || !seq_lens)
      return Fail(PA_ERR_INVALID, "null argument");
    if (!Aligned16(out) || !Aligned16(q)) return Fail(PA_ERR_INVALID, "q and out must be 16-byte aligned");
    pa::PrefillArgs a{};
    a.out = out;
    a.q = q;
    a.k_cache = pool->k_cache;
    a.v_cache = pool->v_cache;
    a.cu_q_lens = cu_q_lens;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.B = B;
    a.Hq = num_q_heads;
    a.Hkv = l.num_kv_heads;
    a.D = l.head_dim;
    a.G = G;
    a.block_size = l.block_size;
    a.num_blocks = l.num_blocks;
    a.max_blocks = max_blocks;
    a.max_q_len = max_q_len;
    a.scale = scale;
    hipError_t e = pa::LaunchPrefill(a, static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported) return Fail(PA_ERR_UNSUPPORTED, "prefill shape not supported");
    return FromHip(e, "prefill launch");
  });
}

}  // extern "C"
