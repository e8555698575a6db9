// C ABI of the paged-attention library: argument validation, error state,
// pool handles, and dispatch to the HIP kernels. Declarations and their
// contracts are in include/pa.h.
#include "pa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <exception>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "block_manager.h"
#include "launch.h"

// Device memory of pa_decode_static: the split-KV partial states of one
// decode call, for callers that cannot allocate. Each GPU the library runs on
// holds its own copy of this array until the process ends. Host code never
// uses the array's name as an address (on the host it is only a stand-in):
// it takes each device's address once with hipGetSymbolAddress, with that
// device current, and passes that pointer on.
static __device__ __align__(256) unsigned char scratch[PA_DECODE_STATIC_SCRATCH_BYTES];

struct pa_pool {
  pa_kv_layout layout;
  void* k_cache;
  void* v_cache;
  pa::BlockManager bm;
  float k_scale = 1.f;  // FP8 pools: a code c stands for value(c) * scale
  float v_scale = 1.f;
  // Mixed steps run the prefill on a second stream beside the decode: the
  // stream (default priority) and its fork/join events are made on the first
  // pa_step / pa_step_graph_create, on the device current then, and released
  // with the pool.
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr;
  hipEvent_t join = nullptr;
  pa_pool(const pa_kv_layout& l, void* k, void* v, const int32_t* order)
      : layout(l), k_cache(k), v_cache(v), bm(l.num_blocks, l.block_size, order) {}
  ~pa_pool() {
    if (join) (void)hipEventDestroy(join);
    if (fork) (void)hipEventDestroy(fork);
    if (side) (void)hipStreamDestroy(side);
  }
  pa_pool(const pa_pool&) = delete;
  pa_pool& operator=(const pa_pool&) = delete;
};

struct pa_step_graph {
  pa_pool* pool;
  hipGraph_t graph;
  hipGraphExec_t exec;
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

// ------------------------------------------------------ static scratch
// Per-device address of `scratch`, resolved once per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The address of `scratch` on the current device, resolving it on the first
// call there (hipGetSymbolAddress; no allocation by this library).
pa_status StaticScratch(void** out) {
  int dev = -1;
  pa_status s = FromHip(hipGetDevice(&dev), "hipGetDevice");
  if (s != PA_OK) return s;
  if (dev < 0 || dev >= kMaxDevices) return Fail(PA_ERR_UNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    s = FromHip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (s != PA_OK) return s;
    if (!p) return Fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) returned null");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

// ------------------------------------------------------------ debug checks
// Duplicate slots in one scatter and block ids outside the pool are undefined
// behaviour for the kernels (they race, or read a clamped block). With debug
// checks on (pa_set_debug_checks, or PA_DEBUG_CHECKS=1 in the environment when
// the library first looks), device calls copy the slots, tables and lengths
// they are given to the host, wait for the copy, and reject such input with
// PA_ERR_INVALID before anything is launched.
std::atomic<int> g_debug{-1};  // -1: not read from the environment yet

bool DebugChecks() {
  int v = g_debug.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = std::getenv("PA_DEBUG_CHECKS");
    v = (e && *e && std::strcmp(e, "0") != 0) ? 1 : 0;
    int expected = -1;
    if (!g_debug.compare_exchange_strong(expected, v)) v = expected;
  }
  return v != 0;
}

// n elements of device memory into *h, ordered after the work on `st`.
template <typename T>
pa_status DebugToHost(std::vector<T>* h, const T* d, size_t n, hipStream_t st) {
  h->resize(n);
  if (n == 0) return PA_OK;
  pa_status s = FromHip(hipMemcpyAsync(h->data(), d, n * sizeof(T), hipMemcpyDeviceToHost, st), "debug check copy");
  if (s == PA_OK) s = FromHip(hipStreamSynchronize(st), "debug check copy");
  return s;
}

// Slots (host values) in the pool: no slot may appear twice.
pa_status DebugCheckSlotsUnique(const pa_pool& pool, const std::vector<int64_t>& slots) {
  const int64_t num_slots = static_cast<int64_t>(pool.layout.num_blocks) * pool.layout.block_size;
  std::vector<int64_t> live;
  live.reserve(slots.size());
  for (int64_t x : slots)
    if (x >= 0 && x < num_slots) live.push_back(x);
  std::sort(live.begin(), live.end());
  const auto dup = std::adjacent_find(live.begin(), live.end());
  if (dup != live.end())
    return Fail(PA_ERR_INVALID, "debug check: slot " + std::to_string(*dup) + " is written twice in one call");
  return PA_OK;
}

// Table entries a call reads: for row b, logical blocks [0, ceil(L_b / bs))
// with L_b clamped into [0, len_cap] as the kernels clamp it, must name a
// block of the pool. new_slots (host, may be empty): a fused append fills in
// the entry of row b's newest token itself when new_slots[b] is in the pool,
// so that entry is not checked.
pa_status DebugCheckTables(const pa_pool& pool, const int32_t* tables_dev, int32_t max_blocks,
                           const std::vector<int32_t>& lens, int64_t len_cap,
                           const std::vector<int64_t>& new_slots, hipStream_t st) {
  const int32_t B = static_cast<int32_t>(lens.size());
  if (B == 0) return PA_OK;
  std::vector<int32_t> tab;
  pa_status s = DebugToHost(&tab, tables_dev, static_cast<size_t>(B) * max_blocks, st);
  if (s != PA_OK) return s;
  const int64_t bs = pool.layout.block_size;
  const int64_t num_slots = static_cast<int64_t>(pool.layout.num_blocks) * bs;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t L = std::min<int64_t>(std::max<int64_t>(lens[static_cast<size_t>(b)], 0), len_cap);
    const int64_t nblk = std::min<int64_t>((L + bs - 1) / bs, max_blocks);
    const bool fills = b < static_cast<int32_t>(new_slots.size()) && L > 0 &&
                       new_slots[static_cast<size_t>(b)] >= 0 && new_slots[static_cast<size_t>(b)] < num_slots;
    for (int64_t i = 0; i < nblk; ++i) {
      if (fills && i == (L - 1) / bs) continue;
      const int32_t id = tab[static_cast<size_t>(b) * max_blocks + static_cast<size_t>(i)];
      if (id < 0 || id >= pool.layout.num_blocks)
        return Fail(PA_ERR_INVALID, "debug check: block_tables[" + std::to_string(b) + "][" + std::to_string(i) +
                                        "] = " + std::to_string(id) + " is not a block of the pool");
    }
  }
  return PA_OK;
}

pa_status DebugCheckWrite(const pa_pool& pool, const int64_t* slots_dev, int32_t T, hipStream_t st) {
  std::vector<int64_t> slots;
  pa_status s = DebugToHost(&slots, slots_dev, static_cast<size_t>(std::max(T, 0)), st);
  return s != PA_OK ? s : DebugCheckSlotsUnique(pool, slots);
}

// A decode call's tables. lens_dev or lens_host gives the lengths;
// slots_dev or slots_host the fused append's slots (both null: plain decode).
pa_status DebugCheckDecode(const pa_pool& pool, const pa::DecodeArgs& a, const int32_t* lens_host,
                           const int64_t* slots_dev, const int64_t* slots_host, hipStream_t st) {
  std::vector<int32_t> lens;
  pa_status s = PA_OK;
  if (lens_host) lens.assign(lens_host, lens_host + a.B);
  else s = DebugToHost(&lens, a.seq_lens, static_cast<size_t>(a.B), st);
  if (s != PA_OK) return s;
  std::vector<int64_t> slots;
  if (slots_host) slots.assign(slots_host, slots_host + a.B);
  else if (slots_dev) s = DebugToHost(&slots, slots_dev, static_cast<size_t>(a.B), st);
  if (s != PA_OK) return s;
  if (!slots.empty()) {
    s = DebugCheckSlotsUnique(pool, slots);
    if (s != PA_OK) return s;
  }
  return DebugCheckTables(pool, a.block_tables, a.max_blocks, lens, a.max_seq_len, slots, st);
}

pa_status DebugCheckPrefill(const pa_pool& pool, const pa::PrefillArgs& a, hipStream_t st) {
  std::vector<int32_t> lens;
  pa_status s = DebugToHost(&lens, a.seq_lens, static_cast<size_t>(a.B), st);
  if (s != PA_OK) return s;
  return DebugCheckTables(pool, a.block_tables, a.max_blocks, lens,
                          static_cast<int64_t>(a.max_blocks) * a.block_size, {}, st);
}

// ---------------------------------------------------------------- device ops
// Validation is kept apart from enqueueing, so that a composite call
// (pa_step) checks every part before it launches anything.

// Copy-on-write copies recorded by earlier appends, in recorded order.
// Consecutive copies share a launch until one touches a block that an
// earlier copy of the launch writes, or writes a block it reads.
pa_status FlushCopies(pa_pool* pool, hipStream_t stream) {
  const pa_kv_layout& l = pool->layout;
  const int64_t block_bytes =
      static_cast<int64_t>(l.block_size) * l.num_kv_heads * l.head_dim * ElemBytes(l.dtype);
  pa::BlockCopyList list{};
  auto flush = [&]() -> pa_status {
    const pa_status st = FromHip(pa::LaunchCopyBlocks(pool->k_cache, pool->v_cache, list, block_bytes, stream),
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
  return PA_OK;
}

struct WriteCall {
  const void* key;
  const void* value;
  const int64_t* slots;
  int32_t T;
};

pa_status CheckWrite(const pa_pool& pool, const WriteCall& w) {
  if (w.T < 0) return Fail(PA_ERR_INVALID, "T must be >= 0");
  if (w.T > 0 && (!w.key || !w.value || !w.slots)) return Fail(PA_ERR_INVALID, "null argument");
  if (w.T > 0 && (!Aligned16(w.key) || !Aligned16(w.value)))
    return Fail(PA_ERR_INVALID, "key and value must be 16-byte aligned");
  const pa_kv_layout& l = pool.layout;
  const int64_t row_elems = static_cast<int64_t>(l.num_kv_heads) * l.head_dim;
  const int64_t chunks = static_cast<int64_t>(w.T) * (row_elems * ElemBytes(l.dtype) / 16);
  if ((chunks + 255) / 256 >= (int64_t{1} << 31)) return Fail(PA_ERR_UNSUPPORTED, "T too large");
  return PA_OK;
}

// The scatter itself (copies are flushed separately); arguments checked.
pa_status EnqueueWrite(const pa_pool& pool, const WriteCall& w, hipStream_t st) {
  if (w.T == 0) return PA_OK;
  const pa_kv_layout& l = pool.layout;
  const int64_t row_elems = static_cast<int64_t>(l.num_kv_heads) * l.head_dim;
  const int64_t num_slots = static_cast<int64_t>(l.num_blocks) * l.block_size;
  if (l.dtype == PA_FP8_E4M3)
    return FromHip(pa::LaunchWriteKvFp8(w.key, w.value, w.slots, pool.k_cache, pool.v_cache, w.T, row_elems,
                                        num_slots, pool.k_scale, pool.v_scale, st),
                   "write_kv launch");
  return FromHip(pa::LaunchWriteKv(w.key, w.value, w.slots, pool.k_cache, pool.v_cache, w.T,
                                   row_elems * ElemBytes(l.dtype), num_slots, st),
                 "write_kv launch");
}

// Checks a decode call and fills its launch arguments; *run stays false for
// an empty batch (nothing to launch).
pa_status PrepareDecode(const pa_pool& pool, void* out, const void* q, const int32_t* block_tables,
                        int32_t max_blocks, const int32_t* seq_lens, int32_t B, int32_t num_q_heads, float scale,
                        int32_t max_seq_len, int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                        pa::DecodeArgs* a, bool* run, bool seq_lens_on_device = true) {
  *run = false;
  if (B < 0 || max_blocks < 0 || max_seq_len < 0 || partition_tokens < 0)
    return Fail(PA_ERR_INVALID, "negative size argument");
  int32_t G = 0;
  pa_status s = CheckHeads(&pool, num_q_heads, &G);
  if (s != PA_OK) return s;
  if (B == 0) return PA_OK;
  if (!out || !q || !block_tables || !seq_lens) return Fail(PA_ERR_INVALID, "null argument");
  if (!Aligned16(out) || !Aligned16(q)) return Fail(PA_ERR_INVALID, "q and out must be 16-byte aligned");
  const pa_kv_layout& l = pool.layout;
  if (static_cast<int64_t>(max_seq_len) > static_cast<int64_t>(max_blocks) * l.block_size)
    return Fail(PA_ERR_INVALID, "max_seq_len exceeds max_blocks * block_size");
  const int32_t pt =
      partition_tokens == 0 ? pa::DecodeDefaultPartition(B, l.num_kv_heads, max_seq_len, l.dtype == PA_FP8_E4M3)
                             : partition_tokens;
  if (pt % 64 || pt > pa::kDecodeMaxPartition)
    return Fail(PA_ERR_UNSUPPORTED, "partition_tokens must be a multiple of 64, at most " +
                                        std::to_string(pa::kDecodeMaxPartition));
  int32_t P = pa::DecodePartitions(max_seq_len, pt);
  if (static_cast<int64_t>(P) * B * l.num_kv_heads >= (int64_t{1} << 31) - 8)
    return Fail(PA_ERR_UNSUPPORTED, "grid too large");
  // The library's choice for long contexts is made on the device, from the
  // lengths (the shape rule above cannot see a batch where one long
  // sequence sits among short ones). That needs the workspace of 512-token
  // partitions, the shortest the device can choose; without room for it
  // (pa_decode_static's fixed scratch), the shape rule stays.
  int32_t auto_items = 0;
  if (partition_tokens == 0 && seq_lens_on_device && B <= pa::kDecodeCompactBatch &&
      max_seq_len >= pa::kDecodeLongContext) {
    const int32_t P512 = pa::DecodePartitions(max_seq_len, 512);
    if (static_cast<int64_t>(P512) * B * l.num_kv_heads < (int64_t{1} << 31) - 8 && workspace &&
        workspace_bytes >= pa::DecodeWorkspaceBytes(B, num_q_heads, l.head_dim, P512)) {
      P = P512;
      auto_items = static_cast<int32_t>(l.dtype == PA_FP8_E4M3 ? pa::kDecodeShortItemsFp8 : pa::kDecodeShortItems);
    }
  }
  const size_t need = pa::DecodeWorkspaceBytes(B, num_q_heads, l.head_dim, P);
  if (need && (!workspace || workspace_bytes < need))
    return Fail(PA_ERR_INVALID, "workspace too small: need " + std::to_string(need) + " bytes");
  if (need && !Aligned16(workspace)) return Fail(PA_ERR_INVALID, "workspace must be 16-byte aligned");
  a->out = out;
  a->q = q;
  a->k_cache = pool.k_cache;
  a->v_cache = pool.v_cache;
  a->block_tables = block_tables;
  a->seq_lens = seq_lens;
  a->ws = workspace;
  a->B = B;
  a->Hq = num_q_heads;
  a->Hkv = l.num_kv_heads;
  a->D = l.head_dim;
  a->G = G;
  a->block_size = l.block_size;
  a->num_blocks = l.num_blocks;
  a->max_blocks = max_blocks;
  a->max_seq_len = max_seq_len;
  a->partition_tokens = pt;
  a->num_partitions = P;
  a->auto_items = auto_items;
  a->scale = scale;
  a->k_scale = pool.k_scale;
  a->v_scale = pool.v_scale;
  a->dtype = l.dtype;
  // Streamed (non-temporal) K/V loads unless some block is shared: a shared
  // prefix is read by many sequences and should stay in the caches.
  a->stream_loads = pool.bm.shared_blocks() == 0;
  *run = true;
  return PA_OK;
}

pa_status PreparePrefill(const pa_pool& pool, void* out, const void* q, const int32_t* cu_q_lens,
                         const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens, int32_t B,
                         int32_t num_q_heads, int32_t max_q_len, float scale, pa::PrefillArgs* a, bool* run) {
  *run = false;
  if (B < 0 || max_blocks < 0 || max_q_len < 0) return Fail(PA_ERR_INVALID, "negative size argument");
  int32_t G = 0;
  pa_status s = CheckHeads(&pool, num_q_heads, &G);
  if (s != PA_OK) return s;
  const pa_kv_layout& l = pool.layout;
  if (l.dtype != PA_BF16) return Fail(PA_ERR_UNSUPPORTED, "prefill supports bf16 pools only");
  if (B == 0 || max_q_len == 0) return PA_OK;
  if (!out || !q || !cu_q_lens || !block_tables || !seq_lens) return Fail(PA_ERR_INVALID, "null argument");
  if (!Aligned16(out) || !Aligned16(q)) return Fail(PA_ERR_INVALID, "q and out must be 16-byte aligned");
  if (pa::PrefillWorkItems(l.num_kv_heads, G, B, max_q_len) >= (int64_t{1} << 31) - 8)
    return Fail(PA_ERR_UNSUPPORTED, "grid too large");
  a->out = out;
  a->q = q;
  a->k_cache = pool.k_cache;
  a->v_cache = pool.v_cache;
  a->cu_q_lens = cu_q_lens;
  a->block_tables = block_tables;
  a->seq_lens = seq_lens;
  a->B = B;
  a->Hq = num_q_heads;
  a->Hkv = l.num_kv_heads;
  a->D = l.head_dim;
  a->G = G;
  a->block_size = l.block_size;
  a->num_blocks = l.num_blocks;
  a->max_blocks = max_blocks;
  a->max_q_len = max_q_len;
  a->scale = scale;
  *run = true;
  return PA_OK;
}

// A mixed step: the scatter of every new row, then decode, then prefill.
struct StepPlan {
  WriteCall write{};
  pa::DecodeArgs dec{};
  pa::PrefillArgs pre{};
  bool run_dec = false;
  bool run_pre = false;
};

pa_status PrepareStep(const pa_pool& pool, const pa_step_desc& d, StepPlan* plan) {
  plan->write = WriteCall{d.key, d.value, d.slot_mapping, d.num_new_tokens};
  pa_status s = CheckWrite(pool, plan->write);
  if (s != PA_OK) return s;
  s = PrepareDecode(pool, d.dec_out, d.dec_q, d.dec_block_tables, d.max_blocks, d.dec_seq_lens, d.dec_batch,
                    d.num_q_heads, d.scale, d.dec_max_seq_len, d.partition_tokens, d.workspace,
                    d.workspace_bytes, &plan->dec, &plan->run_dec);
  if (s != PA_OK) return s;
  return PreparePrefill(pool, d.pre_out, d.pre_q, d.pre_cu_q_lens, d.pre_block_tables, d.max_blocks,
                        d.pre_seq_lens, d.pre_batch, d.num_q_heads, d.pre_max_q_len, d.scale, &plan->pre,
                        &plan->run_pre);
}

// Debug checks of every part of a step (slots of the scatter, tables of the
// decode and of the prefill).
pa_status DebugCheckStep(const pa_pool& pool, const StepPlan& plan, hipStream_t st) {
  pa_status s = PA_OK;
  if (plan.write.T > 0) s = DebugCheckWrite(pool, plan.write.slots, plan.write.T, st);
  if (s == PA_OK && plan.run_dec) s = DebugCheckDecode(pool, plan.dec, nullptr, nullptr, nullptr, st);
  if (s == PA_OK && plan.run_pre) s = DebugCheckPrefill(pool, plan.pre, st);
  return s;
}

// The pool's side stream and fork/join events, made on first use.
pa_status EnsureSideStream(pa_pool* pool) {
  if (pool->side) return PA_OK;
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  pa_status s = FromHip(hipStreamCreateWithFlags(&side, hipStreamNonBlocking), "side stream");
  if (s == PA_OK) s = FromHip(hipEventCreateWithFlags(&fork, hipEventDisableTiming), "fork event");
  if (s == PA_OK) s = FromHip(hipEventCreateWithFlags(&join, hipEventDisableTiming), "join event");
  if (s != PA_OK) {
    if (join) (void)hipEventDestroy(join);
    if (fork) (void)hipEventDestroy(fork);
    if (side) (void)hipStreamDestroy(side);
    return s;
  }
  pool->side = side;
  pool->fork = fork;
  pool->join = join;
  return PA_OK;
}

// The step's device work on stream st: the scatter, then decode and prefill.
// When both run, the prefill goes to the pool's side stream after the
// scatter (fork) and st waits for it at the end (join), so the HBM-bound
// decode and the MFMA-bound prefill share the GPU (measured on MI355X: 341
// -> 307 us per step for 56 decode sequences beside 8 x 256-row chunks), and
// the prefill leaves the CUs it can spare to the decode (262 -> 232 us per
// replayed step on the same batch). The join is made on every path, so a
// capture of st always ends joined.
pa_status EnqueueStep(const pa_pool& pool, const StepPlan& plan, hipStream_t st) {
  pa_status s = EnqueueWrite(pool, plan.write, st);
  if (s != PA_OK) return s;
  if (plan.run_dec && plan.run_pre && pool.side) {
    s = FromHip(hipEventRecord(pool.fork, st), "fork record");
    if (s != PA_OK) return s;
    s = FromHip(hipStreamWaitEvent(pool.side, pool.fork, 0), "fork wait");
    if (s != PA_OK) return s;
    // A decode with at least one (sequence, kv-head group) item for every
    // second CU can use the CUs the prefill leaves it.
    pa::PrefillArgs pre_args = plan.pre;
    const int64_t dec_pairs = static_cast<int64_t>(plan.dec.B) * (plan.dec.Hkv >> pa::DecodeHeadShift(plan.dec.Hkv));
    pre_args.beside_decode = 2 * dec_pairs >= pa::DeviceCuCount();
    const pa_status pre = FromHip(pa::LaunchPrefill(pre_args, pool.side), "prefill launch");
    const pa_status rec = FromHip(hipEventRecord(pool.join, pool.side), "join record");
    pa::DecodeArgs beside = plan.dec;
    beside.place_by_rank = false;  // the prefill holds some of the CUs
    const pa_status dec = pre == PA_OK && rec == PA_OK
                              ? FromHip(pa::LaunchDecode(beside, st), "decode launch") : PA_OK;
    const pa_status wait = rec == PA_OK ? FromHip(hipStreamWaitEvent(st, pool.join, 0), "join wait") : rec;
    return pre != PA_OK ? pre : dec != PA_OK ? dec : wait;
  }
  if (plan.run_dec) {
    s = FromHip(pa::LaunchDecode(plan.dec, st), "decode launch");
    if (s != PA_OK) return s;
  }
  if (plan.run_pre) return FromHip(pa::LaunchPrefill(plan.pre, st), "prefill launch");
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_last_error(void) { return g_error.c_str(); }

int32_t pa_set_debug_checks(int32_t enable) {
  const bool was = DebugChecks();
  g_debug.store(enable ? 1 : 0, std::memory_order_relaxed);
  return was ? 1 : 0;
}

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
    // Set-up of pa_decode_static's scratch on the current device. Best
    // effort: without a usable device (host-only use of the block manager)
    // the address is resolved on that entry point's first call instead.
    void* ignored = nullptr;
    const std::string keep = g_error;
    if (StaticScratch(&ignored) != PA_OK) g_error = keep;
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

pa_status pa_seq_append_tokens(pa_pool* pool, int64_t seq_id, const int32_t* token_ids, int32_t n_tokens,
                               int64_t* slots_out, int32_t* n_cached_out) {
  return Guard([&]() -> pa_status {
    if (!pool) return Fail(PA_ERR_INVALID, "null pool");
    std::string err;
    return FromBm(pool->bm.AppendTokens(seq_id, token_ids, n_tokens, slots_out, n_cached_out, &err), err);
  });
}

pa_status pa_pool_prefix_stats(const pa_pool* pool, pa_prefix_stats_t* out) {
  return Guard([&]() -> pa_status {
    if (!pool || !out) return Fail(PA_ERR_INVALID, "null argument");
    const pa::BlockManager::PrefixStats p = pool->bm.prefix_stats();
    out->cached_blocks = p.cached_blocks;
    out->lookups = p.lookups;
    out->hits = p.hits;
    return PA_OK;
  });
}

int32_t pa_tier_block_size(int64_t expected_len) {
  if (expected_len < 1024) return 32;
  if (expected_len < 8192) return 16;
  return 8;
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

pa_status pa_pool_layout(const pa_pool* pool, pa_kv_layout* out) {
  if (!pool || !out) return Fail(PA_ERR_INVALID, "null argument");
  *out = pool->layout;
  return PA_OK;
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
    const WriteCall w{key, value, slot_mapping, T};
    pa_status s = CheckWrite(*pool, w);
    if (s != PA_OK) return s;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (DebugChecks() && T > 0) {
      s = DebugCheckWrite(*pool, slot_mapping, T, st);
      if (s != PA_OK) return s;
    }
    s = FlushCopies(pool, st);
    if (s != PA_OK) return s;
    return EnqueueWrite(*pool, w, st);
  });
}

size_t pa_decode_workspace_bytes(int32_t B, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_seq_len, int32_t partition_tokens) {
  if (B < 0 || num_q_heads <= 0 || head_dim <= 0 || max_seq_len < 0 || partition_tokens < 0) return 0;
  // 0: the library's choice, which is never shorter than 512 tokens (or it
  // covers max_seq_len in one partition), so 512 bounds its workspace.
  const int32_t pt = partition_tokens == 0 ? 512 : partition_tokens;
  return pa::DecodeWorkspaceBytes(B, num_q_heads, head_dim, pa::DecodePartitions(max_seq_len, pt));
}

int32_t pa_decode_partition_tokens_for_lengths(const pa_pool* pool, const int32_t* seq_lens_host, int32_t B,
                                               int32_t max_seq_len) {
  if (!pool || B < 0 || max_seq_len < 0 || (B > 0 && !seq_lens_host)) return 0;
  if (B == 0) return pa::DecodeDefaultPartition(0, pool->layout.num_kv_heads, max_seq_len, false);
  return pa::DecodePartitionForLengths(seq_lens_host, B, pool->layout.num_kv_heads, max_seq_len);
}

int32_t pa_decode_partition_tokens(const pa_pool* pool, int32_t B, int32_t max_seq_len) {
  if (!pool || B < 0 || max_seq_len < 0) return 0;
  const pa_kv_layout& l = pool->layout;
  return pa::DecodeDefaultPartition(B, l.num_kv_heads, max_seq_len, l.dtype == PA_FP8_E4M3);
}

pa_status pa_decode(pa_pool* pool, void* out, const void* q, const int32_t* block_tables,
                    int32_t max_blocks, const int32_t* seq_lens, int32_t B, int32_t num_q_heads,
                    float scale, int32_t max_seq_len, int32_t partition_tokens, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return Guard([&]() -> pa_status {
    if (!pool) return Fail(PA_ERR_INVALID, "null pool");
    pa::DecodeArgs a{};
    bool run = false;
    pa_status s = PrepareDecode(*pool, out, q, block_tables, max_blocks, seq_lens, B, num_q_heads, scale,
                                max_seq_len, partition_tokens, workspace, workspace_bytes, &a, &run);
    if (s != PA_OK || !run) return s;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (DebugChecks()) {
      s = DebugCheckDecode(*pool, a, nullptr, nullptr, nullptr, st);
      if (s != PA_OK) return s;
    }
    return FromHip(pa::LaunchDecode(a, st), "decode launch");
  });
}

pa_status pa_decode_static(pa_pool* pool, void* out, const void* q, const int32_t* block_tables,
                           int32_t max_blocks, const int32_t* seq_lens, int32_t B, int32_t num_q_heads,
                           float scale, int32_t max_seq_len, int32_t partition_tokens, void* stream) {
  return Guard([&]() -> pa_status {
    if (!pool) return Fail(PA_ERR_INVALID, "null pool");
    if (B < 0 || num_q_heads <= 0 || max_seq_len < 0 || partition_tokens < 0)
      return Fail(PA_ERR_INVALID, "negative size argument");
    const pa_kv_layout& l = pool->layout;
    const int32_t pt = partition_tokens == 0 ? pa::DecodeDefaultPartition(B, l.num_kv_heads, max_seq_len,
                                                                            l.dtype == PA_FP8_E4M3)
                                             : partition_tokens;
    if (pt > 0) {
      const size_t need = pa::DecodeWorkspaceBytes(B, num_q_heads, l.head_dim, pa::DecodePartitions(max_seq_len, pt));
      if (need > PA_DECODE_STATIC_SCRATCH_BYTES)
        return Fail(PA_ERR_UNSUPPORTED, "pa_decode_static: the partial states need " + std::to_string(need) +
                                            " bytes, more than its " +
                                            std::to_string(PA_DECODE_STATIC_SCRATCH_BYTES) +
                                            "-byte scratch (use longer partitions or pa_decode)");
    }
    void* ws = nullptr;
    pa_status s = B > 0 ? StaticScratch(&ws) : PA_OK;
    if (s != PA_OK) return s;
    pa::DecodeArgs a{};
    bool run = false;
    s = PrepareDecode(*pool, out, q, block_tables, max_blocks, seq_lens, B, num_q_heads, scale, max_seq_len,
                      partition_tokens, ws, PA_DECODE_STATIC_SCRATCH_BYTES, &a, &run);
    if (s != PA_OK || !run) return s;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (DebugChecks()) {
      s = DebugCheckDecode(*pool, a, nullptr, nullptr, nullptr, st);
      if (s != PA_OK) return s;
    }
    return FromHip(pa::LaunchDecode(a, st), "decode launch");
  });
}

pa_status pa_append_decode(pa_pool* pool, void* out, const void* q, const void* key, const void* value,
                           const int64_t* slot_mapping, int32_t* block_tables, int32_t max_blocks,
                           const int32_t* seq_lens, int32_t B, int32_t num_q_heads, float scale,
                           int32_t max_seq_len, int32_t partition_tokens, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return Guard([&]() -> pa_status {
    if (!pool) return Fail(PA_ERR_INVALID, "null pool");
    if (pool->layout.dtype == PA_FP8_E4M3)
      return Fail(PA_ERR_UNSUPPORTED, "pa_append_decode needs a bf16 or fp32 pool (use pa_write_kv + pa_decode)");
    pa::DecodeArgs a{};
    bool run = false;
    pa_status s = PrepareDecode(*pool, out, q, block_tables, max_blocks, seq_lens, B, num_q_heads, scale,
                                max_seq_len, partition_tokens, workspace, workspace_bytes, &a, &run);
    if (s != PA_OK) return s;
    if (run) {
      if (!key || !value || !slot_mapping) return Fail(PA_ERR_INVALID, "null argument");
      if (!Aligned16(key) || !Aligned16(value)) return Fail(PA_ERR_INVALID, "key and value must be 16-byte aligned");
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (run && DebugChecks()) {
      s = DebugCheckDecode(*pool, a, nullptr, slot_mapping, nullptr, st);
      if (s != PA_OK) return s;
    }
    s = FlushCopies(pool, st);
    if (s != PA_OK || !run) return s;
    a.new_k = key;
    a.new_v = value;
    a.new_slots = slot_mapping;
    a.tables_out = block_tables;
    return FromHip(pa::LaunchDecode(a, st), "append-decode launch");
  });
}

pa_status pa_append_decode_args(pa_pool* pool, void* out, const void* q, const void* key, const void* value,
                                const int64_t* slot_mapping_host, int32_t* block_tables, int32_t max_blocks,
                                const int32_t* seq_lens_host, int32_t B, int32_t num_q_heads, float scale,
                                int32_t max_seq_len, int32_t partition_tokens, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return Guard([&]() -> pa_status {
    if (!pool) return Fail(PA_ERR_INVALID, "null pool");
    if (pool->layout.dtype == PA_FP8_E4M3)
      return Fail(PA_ERR_UNSUPPORTED, "pa_append_decode_args needs a bf16 or fp32 pool");
    if (B > pa::kStepArgBatch)
      return Fail(PA_ERR_UNSUPPORTED, "pa_append_decode_args takes at most " + std::to_string(pa::kStepArgBatch) +
                                          " sequences (use pa_append_decode)");
    pa::DecodeArgs a{};
    bool run = false;
    const int32_t pt = partition_tokens == 0 && B > 0 && seq_lens_host && max_seq_len >= 0
                           ? pa::DecodePartitionForLengths(seq_lens_host, B, pool->layout.num_kv_heads, max_seq_len)
                           : partition_tokens;
    pa_status s = PrepareDecode(*pool, out, q, block_tables, max_blocks, seq_lens_host, B, num_q_heads, scale,
                                max_seq_len, pt, workspace, workspace_bytes, &a, &run, false);
    if (s != PA_OK) return s;
    if (run) {
      if (!key || !value || !slot_mapping_host) return Fail(PA_ERR_INVALID, "null argument");
      if (!Aligned16(key) || !Aligned16(value)) return Fail(PA_ERR_INVALID, "key and value must be 16-byte aligned");
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (run && DebugChecks()) {
      s = DebugCheckDecode(*pool, a, seq_lens_host, nullptr, slot_mapping_host, st);
      if (s != PA_OK) return s;
    }
    s = FlushCopies(pool, st);
    if (s != PA_OK || !run) return s;
    pa::StepArgs args{};
    for (int32_t b = 0; b < B; ++b) {
      args.slots[b] = slot_mapping_host[b];
      args.lens[b] = seq_lens_host[b];
    }
    a.seq_lens = nullptr;
    a.new_k = key;
    a.new_v = value;
    a.new_slots = nullptr;
    a.tables_out = block_tables;
    a.step_args = &args;
    return FromHip(pa::LaunchDecode(a, st), "append-decode launch");
  });
}

pa_status pa_prefill(pa_pool* pool, void* out, const void* q, const int32_t* cu_q_lens,
                     const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
                     int32_t B, int32_t num_q_heads, int32_t max_q_len, float scale, void* stream) {
  return Guard([&]() -> pa_status {
    if (!pool) return Fail(PA_ERR_INVALID, "null pool");
    pa::PrefillArgs a{};
    bool run = false;
    pa_status s = PreparePrefill(*pool, out, q, cu_q_lens, block_tables, max_blocks, seq_lens, B,
                                 num_q_heads, max_q_len, scale, &a, &run);
    if (s != PA_OK || !run) return s;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (DebugChecks()) {
      s = DebugCheckPrefill(*pool, a, st);
      if (s != PA_OK) return s;
    }
    return FromHip(pa::LaunchPrefill(a, st), "prefill launch");
  });
}

pa_status pa_step(pa_pool* pool, const pa_step_desc* desc, void* stream) {
  return Guard([&]() -> pa_status {
    if (!pool || !desc) return Fail(PA_ERR_INVALID, "null argument");
    StepPlan plan;
    pa_status s = PrepareStep(*pool, *desc, &plan);
    if (s != PA_OK) return s;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (DebugChecks()) {
      s = DebugCheckStep(*pool, plan, st);
      if (s != PA_OK) return s;
    }
    if (plan.run_dec && plan.run_pre) {
      s = EnsureSideStream(pool);
      if (s != PA_OK) return s;
    }
    s = FlushCopies(pool, st);
    if (s != PA_OK) return s;
    return EnqueueStep(*pool, plan, st);
  });
}

pa_status pa_step_graph_create(pa_pool* pool, const pa_step_desc* desc, pa_step_graph** out) {
  return Guard([&]() -> pa_status {
    if (!pool || !desc || !out) return Fail(PA_ERR_INVALID, "null argument");
    if (!pool->bm.pending_copies().empty())
      return Fail(PA_ERR_INVALID, "copy-on-write copies are pending: run them first (pa_write_kv with T = 0)");
    StepPlan plan;
    pa_status s = PrepareStep(*pool, *desc, &plan);
    if (s != PA_OK) return s;
    if (DebugChecks()) {   // the buffers' contents at capture time
      s = DebugCheckStep(*pool, plan, nullptr);
      if (s != PA_OK) return s;
    }
    if (plan.run_dec && plan.run_pre) {
      s = EnsureSideStream(pool);
      if (s != PA_OK) return s;
    }
    // Captured on a private stream of default priority, so that no caller
    // stream (the legacy default stream included) enters capture mode.
    hipStream_t cap = nullptr;
    s = FromHip(hipStreamCreateWithFlags(&cap, hipStreamNonBlocking), "capture stream");
    if (s != PA_OK) return s;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    s = FromHip(hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal), "begin capture");
    if (s == PA_OK) {
      const pa_status launched = EnqueueStep(*pool, plan, cap);
      const pa_status ended = FromHip(hipStreamEndCapture(cap, &graph), "end capture");
      s = launched != PA_OK ? launched : ended;
    }
    if (s == PA_OK) s = FromHip(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0), "graph instantiate");
    (void)hipStreamDestroy(cap);
    if (s != PA_OK) {
      if (exec) (void)hipGraphExecDestroy(exec);
      if (graph) (void)hipGraphDestroy(graph);
      return s;
    }
    *out = new pa_step_graph{pool, graph, exec};
    return PA_OK;
  });
}

pa_status pa_step_graph_launch(pa_step_graph* g, void* stream) {
  return Guard([&]() -> pa_status {
    if (!g) return Fail(PA_ERR_INVALID, "null graph");
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const pa_status s = FlushCopies(g->pool, st);   // copies vary per step: enqueued outside the graph
    if (s != PA_OK) return s;
    return FromHip(hipGraphLaunch(g->exec, st), "graph launch");
  });
}

void pa_step_graph_destroy(pa_step_graph* g) {
  if (!g) return;
  (void)hipGraphExecDestroy(g->exec);
  (void)hipGraphDestroy(g->graph);
  delete g;
}

}  // extern "C"
