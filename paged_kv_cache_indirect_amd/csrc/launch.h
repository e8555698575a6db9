// Kernel launchers called by the C-ABI layer (pa_api.cpp). Arguments are
// validated by the caller; these only enqueue work on `stream`.
#pragma once
#include <climits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// KV append scatter: rows of `row_bytes` bytes (a multiple of 16).
hipError_t LaunchWriteKv(const void* key, const void* value, const int64_t* slots, void* k_cache,
                         void* v_cache, int32_t T, int64_t row_bytes, int64_t num_slots,
                         hipStream_t stream);

// KV append scatter into FP8 (E4M3) pools: bf16 rows of `row_elems` elements
// (a multiple of 16) are quantised with the pool's per-tensor scales.
hipError_t LaunchWriteKvFp8(const void* key, const void* value, const int64_t* slots, void* k_cache,
                            void* v_cache, int32_t T, int64_t row_elems, int64_t num_slots, float k_scale,
                            float v_scale, hipStream_t stream);

// Up to kMaxCopiesPerLaunch independent block copies (no pair reads or
// writes a block another pair of the list writes), passed by value.
constexpr int kMaxCopiesPerLaunch = 64;
struct BlockCopyList {
  int32_t src[kMaxCopiesPerLaunch];
  int32_t dst[kMaxCopiesPerLaunch];
  int32_t n;
};

// Copy block src[p] to block dst[p] in both pools for every pair of the list
// (copy-on-write of shared blocks).
hipError_t LaunchCopyBlocks(void* k_cache, void* v_cache, const BlockCopyList& list, int64_t block_bytes,
                            hipStream_t stream);

// A decode step's per-sequence slots and lengths passed by value in the
// launch (pa_append_decode_args), for batches up to kStepArgBatch.
constexpr int kStepArgBatch = 128;
struct StepArgs {
  int64_t slots[kStepArgBatch];
  int32_t lens[kStepArgBatch];
  // ordered != 0: order lists the sequences by decreasing partition length
  // (the host sorts them); the decode kernel builds its work list in that
  // order and places the items on the CUs by rank.
  uint8_t order[kStepArgBatch];
  int32_t ordered;
};

struct DecodeArgs {
  void* out;
  const void* q;
  void* k_cache;      // written only by the fused append (new rows)
  void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  void* ws;           // workspace (DecodeWorkspaceLayout); null when num_partitions == 1
  int32_t B, Hq, Hkv, D, G;
  int32_t block_size, num_blocks, max_blocks;
  int32_t max_seq_len, partition_tokens, num_partitions;
  float scale;
  float k_scale, v_scale;  // FP8 pools: code value multipliers (1 otherwise)
  int dtype;          // pa_dtype
  // Fused append (all null for a plain decode): new K/V rows [B, Hkv, D],
  // their slots [B], and the table buffer that receives their blocks.
  const void* new_k = nullptr;
  const void* new_v = nullptr;
  const int64_t* new_slots = nullptr;
  int32_t* tables_out = nullptr;
  // Slots and lengths in the launch arguments (seq_lens and new_slots null).
  const StepArgs* step_args = nullptr;
  // K/V rows loaded non-temporally (pools without shared blocks).
  bool stream_loads = true;
  // Items placed on the CUs by length rank, which assumes the decode has the
  // whole GPU (off when it shares the GPU with a concurrent prefill).
  bool place_by_rank = true;
  // > 0: the decode kernel chooses the partition from the device lengths
  // (at most this many items; partition_tokens then holds the shape rule's
  // choice, used when every sequence is a long context) and records it in
  // the workspace for the merge. num_partitions is sized for 512 tokens.
  int32_t auto_items = 0;
};
hipError_t LaunchDecode(const DecodeArgs& a, hipStream_t stream);

// Compute units of the current device (0 if the query fails), cached per
// device; sizes the launches that place work by CU.
int DeviceCuCount();

struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* cu_q_lens;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  int32_t B, Hq, Hkv, D, G;
  int32_t block_size, num_blocks, max_blocks;
  int32_t max_q_len;
  float scale;
  // Running beside a concurrent decode on other CUs: the kernel serves its
  // items with the fewest CUs that keep its span near its longest item.
  bool beside_decode = false;
};
hipError_t LaunchPrefill(const PrefillArgs& a, hipStream_t stream);

// Prefill work items: (kv head, tile of kPrefillRows query rows = positions x
// G heads, sequence), for the grid-size check made before any launch.
constexpr int kPrefillRows = 256;
inline int64_t PrefillWorkItems(int32_t Hkv, int32_t G, int32_t B, int32_t max_q_len) {
  const int32_t rows_per_tile = kPrefillRows / G;
  return static_cast<int64_t>(Hkv) * ((max_q_len + rows_per_tile - 1) / rows_per_tile) * B;
}

// Grid / workspace geometry shared by the API layer and the launchers.
//
// Decode workgroups cover (1 << DecodeHeadShift(Hkv)) kv heads of one
// partition of one sequence: two neighbouring heads (512 contiguous bytes
// of every bf16 slot at D = 128) when Hkv is even, measured faster on MI355X
// than one head (256-byte rows) or four (fewer, longer streams per wave).
inline int32_t DecodeHeadShift(int32_t Hkv) { return Hkv % 2 == 0 ? 1 : 0; }
//
// The library's decode partition when the caller passes 0, from the launch
// shape alone (the host does not see the lengths). Measured on MI355X:
//  * Contexts of kDecodeLongContext tokens and more: every wave should
//    stream a long run of blocks, so the fewest partitions that still give
//    kDecodeLongItems (sequence, kv-head group, partition) work items,
//    counted as if every sequence had max_seq_len tokens.
//  * Shorter contexts: the lengths of a batch differ, and shorter partitions
//    even out the waves' work, as long as every item still finds a
//    workgroup slot in the first round (about 512 on 256 CUs; an item left
//    for a second round costs a whole partition's time). Counting lengths
//    as uniform in [0, max_seq_len], a sequence has max_seq_len / (2 pt) +
//    1/2 partitions on average; the partition is the smallest whose
//    expected item count stays within kDecodeShortItems
//    (kDecodeShortItemsFp8 for E4M3 pools). Both stay below two items per
//    CU (512), where the decode kernel places the items on the CUs by
//    length rank; the E4M3 count keeps more margin, measured on the
//    8B-shaped FP8 batch: 72.1 us at 960 tokens (748 items, no placement),
//    67.4 us at 1664 (500 items).
// The partition is kept within [kDecodeMinPartition, kDecodeDefaultMaxPartition]
// and rounded up to a multiple of 64.
constexpr int32_t kDecodeCompactBatch = 1024;  // batches up to this size get the compact work list
constexpr int32_t kDecodeLongContext = 8192;
constexpr int64_t kDecodeLongItems = 256;
constexpr int64_t kDecodeShortItems = 480;
constexpr int64_t kDecodeShortItemsFp8 = 448;
constexpr int32_t kDecodeMinPartition = 640;
constexpr int32_t kDecodeDefaultMaxPartition = 8192;
constexpr int32_t kDecodeMaxPartition = 1 << 24;
inline int32_t DecodeDefaultPartition(int32_t B, int32_t Hkv, int32_t max_seq_len, bool fp8) {
  const int64_t len = max_seq_len > 1 ? max_seq_len : 1;
  const int64_t groups = Hkv > 1 ? (Hkv >> DecodeHeadShift(Hkv)) : 1;
  const int64_t pairs = static_cast<int64_t>(B > 1 ? B : 1) * groups;
  int64_t pt;
  if (len >= kDecodeLongContext) {
    const int64_t parts = (kDecodeLongItems + pairs - 1) / pairs;
    pt = (len + parts - 1) / parts;
  } else {
    // smallest pt with pairs * (len / (2 pt) + 1/2) <= target
    const int64_t target = fp8 ? kDecodeShortItemsFp8 : kDecodeShortItems;
    const int64_t room = 2 * target - pairs;  // = 2 pairs (target / pairs - 1/2)
    pt = room > 0 ? (pairs * len + room - 1) / room : len;
  }
  pt = (pt + 63) / 64 * 64;
  if (pt > kDecodeDefaultMaxPartition) pt = kDecodeDefaultMaxPartition;
  if (pt < kDecodeMinPartition) pt = kDecodeMinPartition;
  return static_cast<int32_t>(pt);
}
// The default partition when the caller's lengths are on the host
// (pa_append_decode_args): batches whose every sequence is a long context
// keep the shape rule above; otherwise the smallest partition (a multiple of
// 64, at least 512 tokens) whose actual item count, head groups x
// sum_b max(1, ceil(L_b / pt)), is at most kDecodeShortItems, so that every
// item starts in the first round while long sequences in a batch of short
// ones are split finely. One partition per sequence when even that exceeds
// the count.
inline int32_t DecodePartitionForLengths(const int32_t* lens, int32_t B, int32_t Hkv, int32_t max_seq_len) {
  int64_t lo = INT64_MAX, hi = 1;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t L = lens[b] < 0 ? 0 : (lens[b] > max_seq_len ? max_seq_len : lens[b]);
    lo = L < lo ? L : lo;
    hi = L > hi ? L : hi;
  }
  if (B > 0 && lo >= kDecodeLongContext) return DecodeDefaultPartition(B, Hkv, max_seq_len, false);
  const int64_t groups = Hkv > 1 ? (Hkv >> DecodeHeadShift(Hkv)) : 1;
  const int64_t top = (hi + 63) / 64 * 64;
  auto items = [&](int64_t pt) {
    int64_t n = 0;
    for (int32_t b = 0; b < B; ++b) {
      const int64_t L = lens[b] < 0 ? 0 : (lens[b] > max_seq_len ? max_seq_len : lens[b]);
      n += L > pt ? (L + pt - 1) / pt : 1;
    }
    return n * groups;
  };
  int64_t a = 512, z = top < 512 ? 512 : top;  // smallest pt in [a, z] with items(pt) <= target
  if (items(z) > kDecodeShortItems) return static_cast<int32_t>(z);
  while (a < z) {
    const int64_t mid = (a + z) / 2 / 64 * 64;
    if (mid < a) break;
    if (items(mid) <= kDecodeShortItems) z = mid; else a = mid + 64;
  }
  return static_cast<int32_t>(z);
}
inline int32_t DecodePartitions(int32_t max_seq_len, int32_t partition_tokens) {
  int32_t p = (max_seq_len + partition_tokens - 1) / partition_tokens;
  return p < 1 ? 1 : p;
}
// Workspace of a decode call with more than one partition: the fp32 partial
// state of every (sequence, q head, partition), then the partition the
// kernel chose from the lengths (when it chooses):
//   [acc: B*Hq*P*D f32][max, sum: B*Hq*P*2 f32][partition: int32, 16 bytes]
inline size_t DecodeWorkspaceBytes(int32_t B, int32_t Hq, int32_t D, int32_t P) {
  if (P <= 1) return 0;
  return static_cast<size_t>(B) * Hq * P * (static_cast<size_t>(D) + 2) * sizeof(float) + 16;
}
struct DecodeWorkspace {
  float* acc;
  float* ml;
  int32_t* pt;
};
inline DecodeWorkspace DecodeWorkspaceLayout(void* ws, int32_t B, int32_t Hq, int32_t D, int32_t P) {
  DecodeWorkspace w{nullptr, nullptr, nullptr};
  if (!ws || P <= 1) return w;
  w.acc = static_cast<float*>(ws);
  w.ml = w.acc + static_cast<size_t>(B) * Hq * P * D;
  w.pt = reinterpret_cast<int32_t*>(w.ml + static_cast<size_t>(B) * Hq * P * 2);
  return w;
}

}  // namespace pa
