// Paged decode attention for gfx950.
//
// What it computes ("vLLM的'内存分页'到底多神奇 — PagedAttention原理图解",
// xxqk.cn, §3 phase 2): for each sequence b and q head h, walk b's block
// table, read the K/V pages in logical order as one contiguous sequence of
// L_b tokens, and return softmax(scale · q·Kᵀ)·V. Pool layout
// [num_blocks, block_size, Hkv, D] ("LLM推理优化：技术原理解析总览", dpshk.com,
// §3.3). Grouped-query heads: q head h reads kv head h / G.
//
// How (MI355X-first; the pages' own kernel design is CUDA prior art):
//  * Decode is a GEMV per head group: each K/V byte feeds G multiply-adds. It
//    is bandwidth-shaped, so it runs on VALU (no MFMA). Measured on MI355X, a
//    read-only gather of this access pattern reaches ~5.3 TB/s while the math
//    of a straightforward kernel costs more than the loads: the design is
//    about VALU instructions per byte as much as about bytes in flight.
//  * A workgroup of 4 waves owns one KV partition of one sequence for a
//    group of kv heads: two neighbouring heads when Hkv is even (so the
//    workgroup reads 512 contiguous bytes of every bf16 slot at D = 128, in
//    lockstep), else one. Each wave streams its head's share of the
//    partition (a half, or a quarter for one head), K and V together in a
//    single pass. A sequence's partitions are equal in length (at most
//    partition_tokens, rounded up to 64 tokens), so no wave of a short
//    partition idles beside a full one. Eight lanes cover one D-element row
//    with 16-byte loads (one load instruction fetches 8 whole rows); the
//    loads of a batch of steps are issued together, and where registers
//    allow the next batch is issued before the current one is consumed.
//  * The block ids of the wave's range are loaded 64 at a time, one per
//    lane (the next 64 while the current ones stream), and broadcast per
//    step with v_readlane (an SGPR), so the table lookup is off the per-row
//    dependency chain — the extra indirection paging adds ("LLM推理优化",
//    §2.2) costs one readlane per 8 rows.
//  * Each 8-lane row group keeps its own online-softmax state (running max,
//    sum, Σ w·V for the G heads). q·k: v_dot2_f32_bf16 plus a 3-step DPP sum.
//    Weights: one exp2 per (token, head) on scores pre-scaled to log2 units;
//    the running max is raised lazily (only when exceeded by more than 8),
//    so rescaling the accumulators is rare and weights stay ≤ 2^8.
//  * w·V for bf16 caches: two consecutive rows of a lane are interleaved per
//    element with v_perm and contracted with v_dot2_f32_bf16 against the two
//    weights rounded to bf16 (fp32 accumulate) — half the instructions of
//    unpack + FMA. fp32 caches use plain FMAs.
//  * At the end the 8 row groups of a wave merge by DPP and row swaps and the
//    waves of one head through LDS, by log-sum-exp. A sequence that fits in
//    one partition writes its output directly; otherwise every partition
//    writes its partial state (max, sum, Σ w·V) and a second, small kernel
//    merges them by log-sum-exp, one wave per (sequence, q head), four per
//    workgroup. (Merging inside the first
//    kernel through an arrival counter needs an agent-scope release/acquire
//    per partition — an L2 writeback and invalidate per workgroup on this
//    chip — which measured far slower than one extra launch.)
//  * Work items are the (kv-head group, sequence, partition) triples that exist:
//    each workgroup prefix-sums the sequences' partition counts (batches up
//    to 1024) and takes its item from that compact list, so partitions past a
//    sequence's end do not occupy workgroup slots between real ones (the
//    grid is sized for every sequence at max_seq_len; its surplus comes last
//    and exits). Measured on MI355X, interleaved empty workgroups slowed a
//    launch by up to 2.4x. Items are mapped XCD-major with the head group
//    outermost: consecutive hardware workgroup ids go to different XCDs, so
//    each XCD owns a contiguous range (half a head group when Hkv = 8) and a
//    shared prefix block of those heads is re-read from few XCDs' L2.
//    Plain decodes whose items would need more than two workgroups per CU
//    (long contexts at short partitions) take one partition per wave
//    instead: an item holds the consecutive partitions of a head's waves,
//    each wave streams a whole partition and writes its own partial state,
//    so there are half (a quarter at odd Hkv) as many workgroups to start
//    and no merge of a head's waves (measured on 8 x 32768 tokens at
//    512-token partitions: 191 -> 183 us).
//    Pools without shared blocks, where the items number more than one but
//    at most two per CU, place them by length rank instead: the sequences
//    are ranked by partition length (by the host when the lengths come in
//    the launch arguments, by each workgroup for device lengths of up to 256
//    sequences), workgroups c and c + (CU count) share a CU, and the CUs
//    left with one workgroup take the longest items while every other CU
//    pairs a longer item (in its first workgroup, whose waves the SIMDs
//    serve first) with a shorter one. Measured on the 8B-shaped batch:
//    98.8 -> 94.8 us per fused step, 98.3 -> 95.3 us per plain decode.
//    Without that placement a CU's second workgroup raises its waves'
//    priority instead.
//  * Fused append (a decode step in one call): each sequence's new token is
//    the last of its sequence, so it ends the range of exactly one wave per
//    kv head. That wave streams the rest of its range as usual, then adds
//    the token from the step's input row in one extra step and stores the
//    row into the pool; its block's table entry is taken from the token's
//    slot and written back for later calls. The step's lengths and slots
//    come from device memory or, for batches up to 128, from the launch
//    arguments (no host-to-device copy per step).
#include "device_common.h"
#include "launch.h"

#include <algorithm>
#include <atomic>
#include <climits>
#include <type_traits>

namespace pa {

namespace {

constexpr int kWaves = 4;                 // waves per workgroup (one partition of 1, 2 or 4 kv heads)
constexpr int kThreads = 64 * kWaves;
constexpr int kCompactBatch = kDecodeCompactBatch;
constexpr int kLanesPerRow = 8;
constexpr int kRowsPerStep = 64 / kLanesPerRow;
constexpr float kLazyMax = 8.f;
// Running-max start value: finite, so exp2(x - m) needs no -inf guard, and
// far below any score, so the first real score always raises it.
constexpr float kMaxInit = -1.0e30f;

// 8-bit OCP E4M3 cache element (a code; its value is decoded on load).
struct Fp8E4M3 {
  uint8_t bits;
};

template <typename KV, int D>
struct RowGeom {
  static constexpr int kElemPerChunk = 16 / static_cast<int>(sizeof(KV));
  static constexpr int kChunks = D * static_cast<int>(sizeof(KV)) / 16;    // 16-byte chunks per row
  static constexpr int kChunksPerLane = kChunks / kLanesPerRow;            // 1, 2 or 4
  static constexpr int kElemPerLane = kChunksPerLane * kElemPerChunk;
  // Steps (8 rows each) whose loads are issued together: 8 KiB of K+V per
  // wave at 256-byte rows. The kernel is bound by VALU issue rather than by
  // bytes in flight, so 3 waves per SIMD beat deeper batches at 2 waves.
  static constexpr int kStepsInFlight = kChunksPerLane == 1 ? 4 : 2;
  static_assert(kChunks % kLanesPerRow == 0, "row must split into 8 lanes of 16-byte chunks");
};

// Whether the main loop double-buffers its loads (batch n + 1 in flight while
// batch n is consumed). It costs one more batch of registers, so it is used
// where accumulators, q fragments and two load buffers fit in 192 VGPRs and
// the kernel still runs 2 waves per SIMD without spilling.
template <typename T, typename KV, int D, int G>
struct Pipelined {
  using RG = RowGeom<KV, D>;
  static constexpr int kQOut = sizeof(KV) == 1 ? 2 : 1;
  static constexpr int kAcc = G * RG::kElemPerLane;
  static constexpr int kQ = G * RG::kChunksPerLane * kQOut * 4;
  static constexpr int kBuf = RG::kStepsInFlight * RG::kChunksPerLane * 2 * 4;
  static constexpr bool value = kAcc + kQ + 2 * kBuf <= 192;
  // Waves per SIMD the register budget is set for: 3 (168 VGPRs) where one
  // buffer set fits comfortably, else 2 (256 VGPRs).
  static constexpr int kMinWaves = !value && kAcc + kQ + kBuf <= 128 ? 3 : 2;
};

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) { return f32_to_bf16(x); }

// Dot product of one 16-byte chunk of K with the same chunk of q (fp32 accumulate).
__device__ __forceinline__ float chunk_dot(const uint4& k, const uint4& q, float acc, uint16_t) {
  acc = dot2_bf16(k.x, q.x, acc);
  acc = dot2_bf16(k.y, q.y, acc);
  acc = dot2_bf16(k.z, q.z, acc);
  acc = dot2_bf16(k.w, q.w, acc);
  return acc;
}
__device__ __forceinline__ float chunk_dot(const uint4& k, const uint4& q, float acc, float) {
  acc = fmaf(__uint_as_float(k.x), __uint_as_float(q.x), acc);
  acc = fmaf(__uint_as_float(k.y), __uint_as_float(q.y), acc);
  acc = fmaf(__uint_as_float(k.z), __uint_as_float(q.z), acc);
  acc = fmaf(__uint_as_float(k.w), __uint_as_float(q.w), acc);
  return acc;
}

// Element e of a 16-byte chunk as fp32 (8 bf16 or 4 fp32 elements).
__device__ __forceinline__ float chunk_elem(const uint4& c, int e, uint16_t) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  const uint32_t x = w[e >> 1];
  return __uint_as_float((e & 1) ? (x & 0xFFFF0000u) : (x << 16));
}
__device__ __forceinline__ float chunk_elem(const uint4& c, int e, float) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  return __uint_as_float(w[e]);
}

__device__ __forceinline__ uint32_t perm_lo(uint32_t x, uint32_t y) {  // (x.lo, y.lo)
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t x, uint32_t y) {  // (x.hi, y.hi)
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2_t r;
  r.x = static_cast<__bf16>(lo);
  r.y = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, r);
}

// acc[e] += w0 * V0[e] + w1 * V1[e] over one 16-byte chunk of two V rows.
// bf16: the two rows are interleaved per element with v_perm and contracted
// with v_dot2_f32_bf16 against (w0, w1) rounded to bf16; fp32: two FMAs.
__device__ __forceinline__ void pv_pair(const uint4& v0, const uint4& v1, uint32_t wpk, float, float,
                                        float* acc, uint16_t) {
  const uint32_t a[4] = {v0.x, v0.y, v0.z, v0.w};
  const uint32_t b[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    acc[2 * k] = dot2_bf16(perm_lo(a[k], b[k]), wpk, acc[2 * k]);
    acc[2 * k + 1] = dot2_bf16(perm_hi(a[k], b[k]), wpk, acc[2 * k + 1]);
  }
}
__device__ __forceinline__ void pv_pair(const uint4& v0, const uint4& v1, uint32_t, float w0, float w1,
                                        float* acc, float) {
  const uint32_t a[4] = {v0.x, v0.y, v0.z, v0.w};
  const uint32_t b[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = fmaf(w1, __uint_as_float(b[k]), fmaf(w0, __uint_as_float(a[k]), acc[k]));
}

// A 16-byte chunk of cache elements as 16-byte chunks of the compute type:
// the same chunk for fp32 / bf16 caches; for E4M3 codes, 16 codes become 16
// bf16 values (exact: every E4M3 value is a bf16 value) in two chunks.
template <typename KV>
struct Widen {
  static constexpr int kOut = 1;
  __device__ __forceinline__ static void run(const uint4& c, uint4* o) { o[0] = c; }
};
template <>
struct Widen<Fp8E4M3> {
  static constexpr int kOut = 2;
  // Codes 0, 1 (lo) or 2, 3 (hi) of a 32-bit word -> two bf16 in one word.
  __device__ __forceinline__ static uint32_t lo(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  }
  __device__ __forceinline__ static uint32_t hi(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  }
  __device__ __forceinline__ static void run(const uint4& c, uint4* o) {
    o[0] = make_uint4(lo(c.x), hi(c.x), lo(c.y), hi(c.y));
    o[1] = make_uint4(lo(c.z), hi(c.z), lo(c.w), hi(c.w));
  }
};

// One 16-byte chunk of a cached K/V row. kStream: loaded non-temporally.
// Decode reads each K/V byte once, so streamed rows should not displace what
// stays useful in the caches (block ids, queries, partial states); measured
// on MI355X on the 8B-shaped batch, 112.3 -> 99.7 us per launch. A pool with
// shared blocks (a prefix that many sequences read) uses ordinary loads, so
// the shared rows stay in L2 for the sequences that read them next (the
// shared-prefix batch: 116.7 us streamed, 112.5 us with ordinary loads).
template <bool kStream>
__device__ __forceinline__ uint4 load_kv(const void* p) {
  if constexpr (kStream) {
    typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
    const u32x4v v = __builtin_nontemporal_load(static_cast<const u32x4v*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *static_cast<const uint4*>(p);
  }
}

__device__ __forceinline__ int clamp_block(int blk, int num_blocks) {
  return (static_cast<unsigned>(blk) < static_cast<unsigned>(num_blocks)) ? blk : 0;
}

// T: q / out / arithmetic type (float or bf16 bits); KV: cache element type
// (T itself, or Fp8E4M3 with bf16 T). v_scale multiplies the output (the
// FP8 value scale; 1 otherwise); the key scale is folded into scale_log2.
// Launch-argument block of the fused variants; the plain decode takes an
// empty one (a 1.5 KB argument block and the reads of it cost the plain
// kernel about 13 VGPRs and 2-3% of its time).
struct NoStepArgs {};
template <bool kFused>
using StepArgsOf = typename std::conditional<kFused, StepArgs, NoStepArgs>::type;

// The pools: read-only for the plain decode; the fused variant also stores
// each new row into them (through the same pointers: every access to a pool
// in the kernel goes through its parameter).
template <bool kFused, typename KV>
using PoolPtr = typename std::conditional<kFused, KV*, const KV*>::type;

// The decode work list over positions of the batch: the thread holding
// positions tid * kPer .. + kPer - 1 (lengths Lv, -1 past the batch) writes
// s_pref[i] = the first item of the sequence at position i, and thread
// kThreads - 1 writes s_pref[kCompactBatch] = the items per kv-head group
// (a sequence of length L has max(1, ceil(L / PT)) items). Ends with a
// workgroup barrier.
template <int kPer>
__device__ __forceinline__ void build_work_list(const int (&Lv)[kPer], int PT, int tid, int lane, int w,
                                                int* s_wsum, int* s_pref) {
  int cnt[kPer];
  int tsum = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    cnt[i] = Lv[i] >= 0 ? max(1, (Lv[i] + PT - 1) / PT) : 0;
    tsum += cnt[i];
  }
  // inclusive scan of tsum over the workgroup
  int incl = tsum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) s_wsum[w] = incl;
  __syncthreads();
  int wbase = 0;
  for (int ww = 0; ww < w; ++ww) wbase += s_wsum[ww];
  int run = wbase + incl - tsum;  // exclusive prefix of this thread
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    s_pref[tid * kPer + i] = run;
    run += cnt[i];
  }
  if (tid == kThreads - 1) s_pref[kCompactBatch] = run;
  __syncthreads();
}

// kFused: the fused-append variant (pa_append_decode*); the plain decode is
// compiled without that code. kArgs (with kFused): lengths and slots come
// from the launch arguments (pa_append_decode_args), not device memory.
// kStream: K/V rows are loaded non-temporally (see load_kv).
template <typename T, typename KV, int D, int G, bool kFused, bool kArgs, bool kStream>
__global__ __launch_bounds__(kThreads, (Pipelined<T, KV, D, G>::kMinWaves)) void DecodeKernel(
    T* __restrict__ out, const T* __restrict__ q, PoolPtr<kFused, KV> __restrict__ kc,
    PoolPtr<kFused, KV> __restrict__ vc, const int32_t* tables,
    const int32_t* seq_lens_in, float* __restrict__ ws_acc,
    float* __restrict__ ws_ml, int32_t B, int32_t Hkv,
    int32_t max_blocks, int32_t bs_shift, int32_t num_blocks, int32_t max_seq_len, int32_t PT,
    int32_t P, int32_t per_xcd, float scale_log2, float v_scale, int32_t hsh,
    const T* __restrict__ knew, const T* __restrict__ vnew, const int64_t* new_slots_in,
    int32_t* tables_out, int32_t auto_items, int32_t* ws_pt, int32_t place_cus, int32_t pair_cus,
    const StepArgsOf<kArgs> meta) {
  using RG = RowGeom<KV, D>;
  using WD = Widen<KV>;
  constexpr int CPL = RG::kChunksPerLane;
  constexpr int EPC = RG::kElemPerChunk;
  constexpr int EPL = RG::kElemPerLane;
  constexpr int QPC = WD::kOut;        // compute-type chunks per cache chunk
  constexpr int EPQ = EPC / QPC;       // elements per compute-type chunk
  static_assert(EPQ * static_cast<int>(sizeof(T)) == 16, "compute chunks are 16 bytes");
  constexpr int U = RG::kStepsInFlight;  // even: steps are consumed in pairs
  static_assert(U % 2 == 0, "steps are consumed in pairs");
  __shared__ float s_acc[kWaves][G][D];
  __shared__ float s_ml[kWaves][G][2];

  // Lengths (and the fused append's slots) come from device memory, or from
  // the launch arguments in the kArgs variant. (The arguments are read in
  // place: no pointer into them is formed, which would make the compiler
  // copy them to private memory.)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int r = lane >> 3;  // row within a step
  const int j = lane & 7;   // lane within the row

  // ---- work item (XCD-major; kv-head group, then sequence, then partition)
  const int wg = blockIdx.x;
  int p, b, gq;  // gq: group of (1 << hsh) kv heads
  // ordered: the work list runs through the sequences by decreasing
  // partition length (sorted by the host, or below), and the items are
  // placed on the place_cus CUs by rank.
  bool ordered = false;
  bool pair = false;  // one partition per wave (workgroup-uniform)
  int L;          // the sequence's length, clamped to [0, max_seq_len]
  const int NG = Hkv >> hsh;
  if (B <= kCompactBatch) {
    // Compact work list: only the (head group, sequence, partition) items
    // that exist, head group outermost, XCD-major over the real count; the grid's
    // surplus workgroups (sized for B x P) come last and exit.
    __shared__ int s_pref[kCompactBatch + 1];
    __shared__ int s_len[kCompactBatch];  // clamped lengths
    __shared__ int s_wsum[kWaves];
    constexpr int kPer = kCompactBatch / kThreads;  // sequences per thread
    // Position bb of the list holds sequence bb, or the host's order[bb].
    if constexpr (kArgs) ordered = meta.ordered != 0 && place_cus > 0;
    int Lv[kPer];  // this thread's clamped lengths (-1: no such sequence)
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int bb = tid * kPer + i;
      int Lb = 0;
      if (bb < B) {
        if constexpr (kArgs) Lb = meta.lens[ordered ? meta.order[bb] : bb];
        else Lb = seq_lens_in[bb];
      }
      Lb = min(max(Lb, 0), max_seq_len);
      s_len[bb] = Lb;
      Lv[i] = bb < B ? Lb : -1;
    }
    if (auto_items > 0) {
      // The partition from the lengths themselves (the launch passed the
      // shape rule's choice in PT): unless every sequence is a long context,
      // the smallest multiple of 64 tokens, at least 512, whose item count
      // (head groups x sum of max(1, ceil(L / pt))) is at most auto_items;
      // one partition per sequence when even the longest length gives more.
      // Every workgroup computes the same value; workgroup 0 records it for
      // the merge.
      __shared__ int s_red[2][kWaves];
      int parity = 0;
      auto reduce = [&](int v, auto op) {
        v = wave_reduce(v, op);
        if (lane == 0) s_red[parity][w] = v;
        __syncthreads();
        int r = s_red[parity][0];
#pragma unroll
        for (int ww = 1; ww < kWaves; ++ww) r = op(r, s_red[parity][ww]);
        parity ^= 1;  // the next reduction writes the other buffer
        return r;
      };
      int mn = INT_MAX, mx = 0;
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (Lv[i] >= 0) {
          mn = min(mn, Lv[i]);
          mx = max(mx, Lv[i]);
        }
      mn = reduce(mn, [](int a, int c) { return min(a, c); });
      mx = reduce(mx, [](int a, int c) { return max(a, c); });
      if (mn < kDecodeLongContext) {
        auto items = [&](int pt) {
          int n = 0;
#pragma unroll
          for (int i = 0; i < kPer; ++i)
            if (Lv[i] >= 0) n += max(1, (Lv[i] + pt - 1) / pt);
          return reduce(n, [](int a, int c) { return a + c; }) * NG;
        };
        int lo = 512, hi = max(512, (mx + 63) / 64 * 64);
        if (items(hi) <= auto_items) {
          while (lo < hi) {
            const int mid = (lo + hi) / 2 / 64 * 64;
            if (mid < lo) break;
            if (items(mid) <= auto_items) hi = mid; else lo = mid + 64;
          }
        }
        PT = hi;
      }
      if (wg == 0 && tid == 0 && ws_pt != nullptr) *ws_pt = PT;
    }
    build_work_list<kPer>(Lv, PT, tid, lane, w, s_wsum, s_pref);
    // One partition per wave, when the items would take more than two
    // workgroups per CU (pair_cus, the CU count, when allowed): an item is
    // then the 2^(2 - hsh) consecutive partitions of a head's waves, so a
    // sequence of Pb partitions has ceil(Pb / 2^(2 - hsh)) items. Fewer
    // workgroups mean less start-up, and no merge of a head's waves.
    if (pair_cus > 0 && NG * s_pref[kCompactBatch] > 2 * pair_cus) {
      pair = true;
      build_work_list<kPer>(Lv, PT << (2 - hsh), tid, lane, w, s_wsum, s_pref);
    }
    // Device lengths, up to kSortBatch sequences, whose items fill more than
    // one workgroup per CU but at most two (where the placement by rank
    // pays; measured worse with more): the sequences are ranked by
    // decreasing partition length (ties by index) and the list is rebuilt in
    // that order; position i then holds sequence s_ord[i]. (Pipelined
    // variants only: the launch places items only for them.)
    constexpr int kSortBatch = 256;
    bool dev_sort = false;
    __shared__ int s_ord[kSortBatch];
    if constexpr (!kArgs && Pipelined<T, KV, D, G>::value) {
      static_assert(kSortBatch <= kCompactBatch, "sorted batches use the compact list");
      __shared__ __align__(16) int s_key[kSortBatch];
      const int n_items = NG * s_pref[kCompactBatch];
      dev_sort = !pair && place_cus > 0 && B <= kSortBatch && n_items > place_cus && n_items <= 2 * place_cus;
      // Workgroup ids from n_items on hold no item when placed by rank: the
      // grid's surplus (sized for every sequence at max_seq_len) leaves now.
      if (dev_sort && wg >= n_items) return;
      if (dev_sort) {
        static_assert(kSortBatch <= kThreads && kSortBatch % 4 == 0, "one sequence per thread");
        // Thread t ranks sequence t (keys past the batch are -1, below every
        // sequence): rank = sequences with a longer partition, or as long
        // and earlier. The keys are read four at a time.
        int key = -1;
        if (tid < B) {
          const int Lt = s_len[tid];
          const int Pb = max(1, (Lt + PT - 1) / PT);
          key = ((Lt + Pb - 1) / Pb + 63) & ~63;
        }
        if (tid < kSortBatch) s_key[tid] = key;
        __syncthreads();
        int rank = 0;
        for (int x = 0; x < B; x += 4) {
          const int4 k4 = *reinterpret_cast<const int4*>(&s_key[x]);
          rank += (k4.x > key) | ((k4.x == key) & (x < tid));
          rank += (k4.y > key) | ((k4.y == key) & (x + 1 < tid));
          rank += (k4.z > key) | ((k4.z == key) & (x + 2 < tid));
          rank += (k4.w > key) | ((k4.w == key) & (x + 3 < tid));
        }
        if (tid < B) s_ord[rank] = tid;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          const int bb = tid * kPer + i;
          Lv[i] = bb < B ? s_len[s_ord[bb]] : -1;
        }
        build_work_list<kPer>(Lv, PT, tid, lane, w, s_wsum, s_pref);
        ordered = true;
      }
    }
    const int S = s_pref[kCompactBatch];  // items per kv head
    int k;
    if (ordered) {
      // Items ranked by decreasing length, head groups innermost. Workgroups
      // c and c + C (C = place_cus, the CU count) run on the same CU,
      // two per CU: when the items fill more than one workgroup per CU but
      // at most two, the CUs left with one workgroup take the longest items,
      // and each other CU pairs a longer item in its first workgroup (whose
      // waves the SIMDs serve first) with a shorter one in its second, so
      // that the CUs' totals even out. Otherwise workgroup i takes rank i.
      const int C = place_cus;
      const int n = NG * S;
      if (wg >= n) return;
      int rank = wg;
      if (n > C && n <= 2 * C) {
        const int pairs = n - C;  // CUs that hold two workgroups
        if (wg >= C) rank = n - 1 - (wg - C);
        else if (wg >= pairs) rank = wg - pairs;
        else rank = (C - pairs) + wg;
      }
      gq = rank % NG;
      k = rank / NG;
    } else {
      const int per_xcd_real = (NG * S + 7) / 8;
      if ((wg >> 3) >= per_xcd_real) return;
      const int item = (wg & 7) * per_xcd_real + (wg >> 3);
      if (item >= NG * S) return;
      gq = item / S;
      k = item - gq * S;
    }
    int lo = 0, hi = B - 1;  // largest b with s_pref[b] <= k
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= k) lo = mid; else hi = mid - 1;
    }
    p = k - s_pref[lo];
    b = lo;
    if (dev_sort) b = s_ord[lo];
    if constexpr (kArgs) b = ordered ? meta.order[lo] : lo;
    L = s_len[dev_sort ? b : lo];  // s_len: by sequence, or by position (host order)
  } else {
    const int item = (wg & 7) * per_xcd + (wg >> 3);
    if (item >= NG * B * P) return;
    p = item % P;
    const int bg = item / P;
    b = bg % B;
    gq = bg / B;
    int Lr;
    if constexpr (kArgs) Lr = meta.lens[b];
    else Lr = seq_lens_in[b];
    L = min(max(Lr, 0), max_seq_len);
  }
  const int WS = 2 - hsh;  // log2(waves per kv head)
  const int hh = w >> WS;  // kv head within the workgroup
  const int g = (gq << hsh) + hh;
  const int wq = w & ((1 << WS) - 1);
  const int Hq = Hkv * G;

  const int Pb = max(1, (L + PT - 1) / PT);  // partitions of this sequence
  if ((pair ? p << (2 - hsh) : p) >= Pb) return;

  // Fused append (new_slots given): row b of knew / vnew is sequence b's
  // newest token, at position L - 1, bound for slot new_slots[b] (< 0, or
  // outside the pool: no new token). The slot also names the block that
  // holds it, so that block's table entry is taken from the slot rather than
  // from the table (a new block, or a copy-on-write block, is not in the
  // table yet). The token is the last of the sequence, so it ends the range
  // of one wave per kv head: that wave streams the rest of its range as
  // usual, then takes the token from knew / vnew in one extra step after the
  // loop and stores its head's part of the row into the pool; head group 0's
  // workgroup of the last partition fills in the table entry for later calls.
  constexpr bool kFusable = kFused && sizeof(KV) == sizeof(T);  // not for E4M3 pools
  int64_t nslot = -1;
  if constexpr (kFusable) {
    if (knew != nullptr && L > 0) {
      if constexpr (kArgs) nslot = meta.slots[b];
      else nslot = new_slots_in != nullptr ? new_slots_in[b] : -1;
    }
  }
  // A slot outside the pool is skipped, as pa_write_kv skips it.
  const bool has_new = nslot >= 0 && nslot < (static_cast<int64_t>(num_blocks) << bs_shift);  // wave-uniform
  const int new_tok = has_new ? L - 1 : -1;
  const int new_lb = has_new ? (L - 1) >> bs_shift : -1;
  const int new_blk = static_cast<int>(nslot >> bs_shift);
  const int64_t row_stride = static_cast<int64_t>(Hkv) * D;  // elements between slots
  if (has_new && p == Pb - 1 && gq == 0 && tid == 0)
    tables_out[static_cast<int64_t>(b) * max_blocks + new_lb] = new_blk;

  const int PTb = ((L + Pb - 1) / Pb + 63) & ~63;  // equal split, multiple of 64 (<= PT)
  // A wave streams its share of the item's partition, or with one partition
  // per wave the whole partition (p << WS) + wq (empty past the sequence's
  // end).
  const int TPW = pair ? PTb : PTb >> WS;
  const int w0 = pair ? ((p << WS) + wq) * PTb : p * PTb + wq * TPW;
  // holds_new: this wave's range ends with the fused append's token, which
  // the loop leaves for the step after it.
  const bool holds_new = has_new && w0 <= new_tok && new_tok < w0 + TPW;  // wave-uniform
  const int ntok = max(0, min(w0 + TPW, L) - w0) - (holds_new ? 1 : 0);
  const int nsteps = (ntok + kRowsPerStep - 1) / kRowsPerStep;

  // The new token's K/V row (this wave's head), loaded now so that its
  // latency overlaps the streaming loop rather than following it.
  uint4 kxn[CPL], vxn[CPL];
  if constexpr (kFusable) {
    if (holds_new) {
      const int64_t nrow = (static_cast<int64_t>(b) * Hkv + g) * D;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        kxn[i] = *reinterpret_cast<const uint4*>(knew + nrow + (j + kLanesPerRow * i) * EPC);
        vxn[i] = *reinterpret_cast<const uint4*>(vnew + nrow + (j + kLanesPerRow * i) * EPC);
      }
    }
  }

  // q fragments: this lane's chunks (j, j + 8, ...) of the G heads.
  uint4 qf[G][CPL][QPC];
  {
    const T* qb = q + (static_cast<int64_t>(b) * Hq + g * G) * D;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < CPL; ++i)
#pragma unroll
        for (int qq = 0; qq < QPC; ++qq)
          qf[h][i][qq] = *reinterpret_cast<const uint4*>(qb + h * D + (j + kLanesPerRow * i) * EPC + qq * EPQ);
  }

  // Block ids of the wave's range, 64 at a time (a window): lane x holds
  // logical block lbw + x of the current window, and the next window's ids
  // are loaded while this one streams. Steps start on multiples of 8 tokens
  // and block sizes are multiples of 8, so the 8 rows of one step always sit
  // in one block; wave ranges start on multiples of 16 tokens, so every
  // window but the last covers an even number of steps.
  constexpr int kWinBlocks = 64;
  const int bs = 1 << bs_shift;
  const int32_t* trow = tables + static_cast<int64_t>(b) * max_blocks;
  const int lb0 = w0 >> bs_shift;
  // A wave with no tokens has no blocks (its start may lie past the table's
  // last entry when it falls inside a block).
  const int lb_end = ntok > 0 ? (w0 + ntok + bs - 1) >> bs_shift : lb0;
  // Table entry idx, or the fused append's block for the new token's entry.
  auto table_at = [&](int idx) {
    if constexpr (kFusable) return idx == new_lb ? new_blk : trow[idx];
    else return trow[idx];
  };
  int cur_blk = 0, nxt_blk = 0;  // ids of the current window and of the next one
  if (lb0 + lane < lb_end) cur_blk = clamp_block(table_at(lb0 + lane), num_blocks);
  if (lb_end > lb0) nxt_blk = table_at(min(lb0 + kWinBlocks + lane, lb_end - 1));
  int lbw = lb0;  // first block of the current window

  const KV* kbase = kc + static_cast<int64_t>(g) * D + static_cast<int64_t>(r) * row_stride;
  const KV* vbase = vc + static_cast<int64_t>(g) * D + static_cast<int64_t>(r) * row_stride;

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kMaxInit;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  // Loads of one step (8 rows) into one buffer slot. Steps are issued in
  // increasing order, so the window of block ids only ever moves forward, by
  // at most one window per step.
  auto issue = [&](int st, uint4 (&kx)[CPL], uint4 (&vx)[CPL]) {
    const int tok = w0 + st * kRowsPerStep;
    const int lb = tok >> bs_shift;
    if (lb - lbw >= kWinBlocks) {
      lbw += kWinBlocks;
      cur_blk = clamp_block(nxt_blk, num_blocks);
      nxt_blk = table_at(min(lbw + kWinBlocks + lane, lb_end - 1));
    }
    const int blk = __builtin_amdgcn_readlane(cur_blk, lb - lbw);
    const int64_t slot0 = (static_cast<int64_t>(blk) << bs_shift) + (tok & (bs - 1));
    const KV* krow = kbase + slot0 * row_stride;
    const KV* vrow = vbase + slot0 * row_stride;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      kx[i] = load_kv<kStream>(krow + (j + kLanesPerRow * i) * EPC);
      vx[i] = load_kv<kStream>(vrow + (j + kLanesPerRow * i) * EPC);
    }
  };

  // Two consecutive steps (rows t and t + 8 for this lane) at a time.
  auto consume_pair = [&](int st, uint4 (&kb)[U][CPL], uint4 (&vb)[U][CPL], int u) {
    float x0[G], x1[G];  // scores in log2 units
    uint4 k0[CPL][QPC], k1[CPL][QPC];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      WD::run(kb[u][i], k0[i]);
      WD::run(kb[u + 1][i], k1[i]);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int i = 0; i < CPL; ++i)
#pragma unroll
        for (int qq = 0; qq < QPC; ++qq) {
          a0 = chunk_dot(k0[i][qq], qf[h][i][qq], a0, T{});
          a1 = chunk_dot(k1[i][qq], qf[h][i][qq], a1, T{});
        }
      x0[h] = sum8(a0) * scale_log2;
      x1[h] = sum8(a1) * scale_log2;
    }
    if ((st + 2) * kRowsPerStep > ntok) {  // rows past the end hold stale data (maybe NaN)
      const bool bad0 = st * kRowsPerStep + r >= ntok;
      const bool bad1 = (st + 1) * kRowsPerStep + r >= ntok;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        x0[h] = bad0 ? -INFINITY : x0[h];
        x1[h] = bad1 ? -INFINITY : x1[h];
      }
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        if (bad0) vb[u][i] = make_uint4(0, 0, 0, 0);
        if (bad1) vb[u + 1][i] = make_uint4(0, 0, 0, 0);
      }
    }
    // Lazy running max: raise it only when a score exceeds it by > kLazyMax.
    float over = -INFINITY;
#pragma unroll
    for (int h = 0; h < G; ++h) over = fmaxf(over, fmaxf(x0[h], x1[h]) - m[h]);
    if (__builtin_amdgcn_ballot_w64(over > kLazyMax)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float top = fmaxf(x0[h], x1[h]);
        const float mn = top > m[h] + kLazyMax ? top : m[h];
        const float f = fast_exp2(m[h] - mn);
        l[h] *= f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= f;
        m[h] = mn;
      }
    }
    uint4 v0[CPL][QPC], v1[CPL][QPC];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      WD::run(vb[u][i], v0[i]);
      WD::run(vb[u + 1][i], v1[i]);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float w0v = fast_exp2(x0[h] - m[h]);
      const float w1v = fast_exp2(x1[h] - m[h]);
      l[h] += w0v + w1v;
      const uint32_t wpk = sizeof(T) == 2 ? pack_bf16(w0v, w1v) : 0u;
#pragma unroll
      for (int i = 0; i < CPL; ++i)
#pragma unroll
        for (int qq = 0; qq < QPC; ++qq)
          pv_pair(v0[i][qq], v1[i][qq], wpk, w0v, w1v, &acc[h][i * EPC + qq * EPQ], T{});
    }
  };

  // Batches of U steps. A step past the wave's end re-reads its last step (a
  // cache hit), so every path issues the same number of loads and the
  // compiler's wait counts stay exact. Pipelined: the loads of batch n + 1
  // are issued before batch n is consumed, so the wave keeps a batch in
  // flight while it computes; otherwise each batch is loaded, then consumed.
  if (nsteps > 0) {
    auto issue_batch = [&](int st0, uint4 (&kx)[U][CPL], uint4 (&vx)[U][CPL]) {
#pragma unroll
      for (int u = 0; u < U; ++u) issue(min(st0 + u, nsteps - 1), kx[u], vx[u]);
    };
    auto consume_batch = [&](int st0, uint4 (&kx)[U][CPL], uint4 (&vx)[U][CPL]) {
#pragma unroll
      for (int u = 0; u < U; u += 2)
        if (st0 + u < nsteps) consume_pair(st0 + u, kx, vx, u);
    };
    uint4 kA[U][CPL], vA[U][CPL];
    if constexpr (Pipelined<T, KV, D, G>::value) {
      uint4 kB[U][CPL], vB[U][CPL];
      const int nbat = (nsteps + U - 1) / U;
      issue_batch(0, kA, vA);
      // A CU holds two of these workgroups; the SIMDs issue for the older
      // wave first, so the second workgroup's waves (wave slot 1) stream
      // about 1.4x slower than the first's (measured on the 8B-shaped batch:
      // 7.2 against 10.1 tokens per us per wave) and finish last. Unless the
      // items were placed for that (ordered), raising their priority evens
      // the two out.
      if (!ordered && (__builtin_amdgcn_s_getreg((3 << 11) | 4) & 0xF) != 0)  // HW_ID.WAVE_ID
        __builtin_amdgcn_s_setprio(1);
      for (int n = 0; n < nbat; n += 2) {
        issue_batch((n + 1) * U, kB, vB);
        __builtin_amdgcn_sched_barrier(0);
        consume_batch(n * U, kA, vA);
        issue_batch((n + 2) * U, kA, vA);
        __builtin_amdgcn_sched_barrier(0);
        if (n + 1 < nbat) consume_batch((n + 1) * U, kB, vB);
      }
    } else {
      for (int st0 = 0; st0 < nsteps; st0 += U) {
        issue_batch(st0, kA, vA);
        // Keep all U steps' loads ahead of the math (the scheduler would
        // sink each load next to its first use, exposing memory latency).
        __builtin_amdgcn_sched_barrier(0);
        consume_batch(st0, kA, vA);
      }
    }
  }

  // ---- the fused append's token (the last of the sequence): row group 0
  // adds it to its state with an exact rescale, and stores the row into the
  // pool.
  if constexpr (kFusable) {
    if (holds_new) {
      const uint4 (&kx)[CPL] = kxn;
      const uint4 (&vx)[CPL] = vxn;
      float x[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) a = chunk_dot(kx[i], qf[h][i][0], a, T{});
        x[h] = sum8(a) * scale_log2;
      }
      if (r == 0) {
        KV* kd = kc + nslot * row_stride + static_cast<int64_t>(g) * D;
        KV* vd = vc + nslot * row_stride + static_cast<int64_t>(g) * D;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          *reinterpret_cast<uint4*>(kd + (j + kLanesPerRow * i) * EPC) = kx[i];
          *reinterpret_cast<uint4*>(vd + (j + kLanesPerRow * i) * EPC) = vx[i];
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float mn = fmaxf(m[h], x[h]);
          const float f = fast_exp2(m[h] - mn);
          const float wn = fast_exp2(x[h] - mn);
          l[h] = fmaf(l[h], f, wn);
#pragma unroll
          for (int i = 0; i < CPL; ++i)
#pragma unroll
            for (int e = 0; e < EPC; ++e)
              acc[h][i * EPC + e] = fmaf(acc[h][i * EPC + e], f, wn * chunk_elem(vx[i], e, T{}));
          m[h] = mn;
        }
      }
    }
  }

  // ---- merge the 8 row groups of the wave (lanes that differ in bits 3..5)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float M = max_over_groups8(m[h]);
    const float f = fast_exp2(m[h] - M);
    l[h] = sum_over_groups8(l[h] * f);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = sum_over_groups8(acc[h][e] * f);
    m[h] = M;
  }
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < CPL; ++i)
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          s_acc[w][h][(j + kLanesPerRow * i) * EPC + e] = acc[h][i * EPC + e];
  }
  if (lane < G) {
    float mm = m[0], ll = l[0];
#pragma unroll
    for (int h = 1; h < G; ++h) {
      mm = lane == h ? m[h] : mm;
      ll = lane == h ? l[h] : ll;
    }
    s_ml[w][lane][0] = mm;
    s_ml[w][lane][1] = ll;
  }
  __syncthreads();

  // ---- one partition per wave: each wave's state is its partition's
  if (pair && Pb > 1) {
    for (int idx = tid; idx < (G * D << hsh << WS); idx += kThreads) {
      const int ww = idx / (G * D);  // wave
      const int h = (idx / D) % G;
      const int d = idx % D;
      const int pw = (p << WS) + (ww & ((1 << WS) - 1));
      if (pw >= Pb) continue;
      const int qh = ((gq << hsh) + (ww >> WS)) * G + h;  // q head
      const int64_t row = (static_cast<int64_t>(b) * Hq + qh) * P + pw;
      ws_acc[row * D + d] = s_acc[ww][h][d] * v_scale;
      if (d == 0) {
        ws_ml[row * 2 + 0] = s_ml[ww][h][0];
        ws_ml[row * 2 + 1] = s_ml[ww][h][1];
      }
    }
    return;
  }

  // ---- merge the 4 waves; write the output, or this partition's partial state
  for (int idx = tid; idx < (G * D << hsh); idx += kThreads) {
    const int hw = idx / (G * D);       // kv head within the workgroup
    const int h = (idx / D) % G;
    const int d = idx % D;
    const int wlo = hw << WS, whi = (hw + 1) << WS;
    const int qh = ((gq << hsh) + hw) * G + h;  // q head
    float M = kMaxInit;
    for (int ww = wlo; ww < whi; ++ww) M = fmaxf(M, s_ml[ww][h][0]);
    float a = 0.f, lsum = 0.f;
    for (int ww = wlo; ww < whi; ++ww) {
      const float f = fast_exp2(s_ml[ww][h][0] - M);
      a = fmaf(f, s_acc[ww][h][d], a);
      lsum = fmaf(f, s_ml[ww][h][1], lsum);
    }
    a *= v_scale;
    if (Pb == 1) {
      out[(static_cast<int64_t>(b) * Hq + qh) * D + d] = from_f32<T>(lsum > 0.f ? a / lsum : 0.f);
    } else {
      const int64_t row = (static_cast<int64_t>(b) * Hq + qh) * P + p;  // (b, q head, p)
      ws_acc[row * D + d] = a;
      if (d == 0) {
        ws_ml[row * 2 + 0] = M;
        ws_ml[row * 2 + 1] = lsum;
      }
    }
  }
}

// Pass 2: log-sum-exp merge of the partitions of each (sequence, q head),
// one wave each, four per workgroup. The partial states are read in chunks
// of 16 partitions: lane x holds partition x's (max, sum) and every lane
// its D/64 dims of each partition's Σ w·V, all loaded together once the
// length is known, so a merge costs two dependent loads. Chunks after the
// first (more than 16 partitions) rescale the running sums when the maximum
// grows. Partitions past the sequence's count hold stale data and are
// excluded by selection (a zero weight would not cancel a NaN).
template <typename T, int D, bool kArgs>
__global__ __launch_bounds__(256) void MergeKernel(T* __restrict__ out, const float* __restrict__ ws_acc,
                                                   const float* __restrict__ ws_ml,
                                                   const int32_t* seq_lens_in, int32_t BH,
                                                   int32_t Hq, int32_t max_seq_len, int32_t PT, int32_t P,
                                                   const int32_t* ws_pt, const StepArgsOf<kArgs> meta) {
  constexpr int EPL = D / 64;
  constexpr int kChunk = 16;
  const int lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + static_cast<int>(threadIdx.x >> 6);
  if (bh >= BH) return;
  const int b = bh / Hq;
  int L;
  if constexpr (kArgs) L = meta.lens[b];
  else L = seq_lens_in[b];
  L = min(max(L, 0), max_seq_len);
  if (ws_pt != nullptr) PT = *ws_pt;  // chosen from the lengths by pass 1
  const int Pb = (L + PT - 1) / PT;
  if (Pb <= 1) return;  // written by pass 1
  const float* ml = ws_ml + static_cast<int64_t>(bh) * P * 2;
  const float* acc = ws_acc + static_cast<int64_t>(bh) * P * D + lane * EPL;

  float M = kMaxInit, lsum = 0.f;
  float a[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) a[e] = 0.f;
  for (int x0 = 0; x0 < Pb; x0 += kChunk) {
    const int n = min(kChunk, Pb - x0);  // partitions of this chunk
    float mx = kMaxInit, lx = 0.f;
    if (lane < n) {
      mx = ml[2 * (x0 + lane)];
      lx = ml[2 * (x0 + lane) + 1];
    }
    float v[kChunk][EPL];
#pragma unroll
    for (int k = 0; k < kChunk; ++k)
#pragma unroll
      for (int e = 0; e < EPL; ++e) v[k][e] = k < n ? acc[static_cast<int64_t>(x0 + k) * D + e] : 0.f;
    const float Mc = wave_reduce(mx, OpMax{});
    const float Mn = fmaxf(M, Mc);
    const float f = fast_exp2(M - Mn);
    lsum *= f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) a[e] *= f;
    M = Mn;
    const float wgt = lane < n ? fast_exp2(mx - M) : 0.f;
    lsum = fmaf(wgt, lx, lsum);
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wgt), k));
#pragma unroll
      for (int e = 0; e < EPL; ++e) a[e] = k < n ? fmaf(wk, v[k][e], a[e]) : a[e];
    }
  }
  lsum = wave_reduce(lsum, OpAdd{});
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e)
    out[static_cast<int64_t>(bh) * D + lane * EPL + e] = from_f32<T>(a[e] * inv);
}

template <typename T, typename KV, int D, int G>
hipError_t LaunchTyped(const DecodeArgs& a, hipStream_t stream) {
  const int P = a.num_partitions;
  const int hsh = DecodeHeadShift(a.Hkv);
  const int64_t NG = a.Hkv >> hsh;
  int64_t items = static_cast<int64_t>(P) * a.B * NG;
  if (a.auto_items > 0) {
    // The kernel picks the partition: at most auto_items items, or one per
    // sequence, or what the shape rule (a.partition_tokens) gives.
    const int64_t shape = static_cast<int64_t>(DecodePartitions(a.max_seq_len, a.partition_tokens)) * a.B * NG;
    items = std::min(items, std::max(std::max<int64_t>(a.auto_items, a.B * NG), shape));
  } else if (a.step_args != nullptr && a.B <= kCompactBatch) {
    // Lengths on the host: the grid holds exactly the compact list's items
    // (the kernel builds the same list). Sized for every sequence at
    // max_seq_len instead, a batch with one long sequence among short ones
    // launches thousands of surplus workgroups that only run the prologue
    // and exit (measured: 63 x 512 + 1 x 32768 tokens, 91.7 us).
    int64_t S = 0;
    for (int32_t b = 0; b < a.B; ++b) {
      const int32_t L = std::min(std::max(a.step_args->lens[b], 0), a.max_seq_len);
      S += std::max(1, (L + a.partition_tokens - 1) / a.partition_tokens);
    }
    items = S * NG;
  }
  // Plain decodes with the compact list may take one partition per wave
  // (the kernel decides from the items); the grid stays sized for the items
  // of one partition per workgroup, an upper bound.
  const int32_t cus = DeviceCuCount();
  const int32_t pair_cus = a.new_k == nullptr && a.B <= kCompactBatch ? cus : 0;
  const int per_xcd = static_cast<int>((items + 7) / 8);
  const bool fp8 = sizeof(KV) == 1;
  const float scale_log2 = a.scale * (fp8 ? a.k_scale : 1.f) * 1.4426950408889634f;
  const float v_scale = fp8 ? a.v_scale : 1.f;
  DecodeWorkspace ws = DecodeWorkspaceLayout(a.ws, a.B, a.Hq, a.D, P);
  static const StepArgs kNoStepArgs{};
  StepArgs sorted;
  const StepArgs* meta_src = a.step_args != nullptr ? a.step_args : &kNoStepArgs;
  // Placement of the items by length rank (pools without shared blocks, whose
  // rows are streamed; pipelined variants, which run two workgroups per CU
  // as the placement assumes; more items than CUs but at most two per CU):
  // lengths in the launch arguments are sorted here, device lengths of up to
  // 256 sequences by the kernel.
  const int32_t place_cus =
      a.place_by_rank && a.stream_loads && Pipelined<T, KV, D, G>::value && a.B <= kCompactBatch ? cus : 0;
  if (a.step_args != nullptr && a.auto_items == 0 && place_cus > 0 && a.B <= kStepArgBatch &&
      items > place_cus && items <= 2 * static_cast<int64_t>(place_cus)) {
    // Sequences by decreasing partition length (the kernel's equal split,
    // stable).
    sorted = *a.step_args;
    int32_t part_len[kStepArgBatch];
    for (int32_t b = 0; b < a.B; ++b) {
      const int32_t L = std::min(std::max(sorted.lens[b], 0), a.max_seq_len);
      const int32_t Pb = std::max(1, (L + a.partition_tokens - 1) / a.partition_tokens);
      part_len[b] = ((L + Pb - 1) / Pb + 63) & ~63;
      sorted.order[b] = static_cast<uint8_t>(b);
    }
    std::stable_sort(sorted.order, sorted.order + a.B,
                     [&](uint8_t x, uint8_t y) { return part_len[x] > part_len[y]; });
    sorted.ordered = 1;
    meta_src = &sorted;
  }
  const StepArgs& meta = *meta_src;
  auto launch_kernel = [&](auto kernel, const auto& meta) {
    hipLaunchKernelGGL(kernel, dim3(per_xcd * 8), dim3(kThreads), 0, stream,
                       static_cast<T*>(a.out), static_cast<const T*>(a.q),
                       static_cast<KV*>(a.k_cache), static_cast<KV*>(a.v_cache),
                       a.block_tables, a.seq_lens, ws.acc, ws.ml, a.B, a.Hkv, a.max_blocks,
                       __builtin_ctz(a.block_size), a.num_blocks, a.max_seq_len, a.partition_tokens,
                       P, per_xcd, scale_log2, v_scale, hsh, static_cast<const T*>(a.new_k),
                       static_cast<const T*>(a.new_v), a.new_slots, a.tables_out, a.auto_items, ws.pt, place_cus,
                       pair_cus, meta);
  };
  auto launch = [&](auto stream_tag) {
    constexpr bool kStream = decltype(stream_tag)::value;
    if constexpr (sizeof(KV) == sizeof(T)) {
      if (a.new_k != nullptr && a.step_args != nullptr)
        launch_kernel(DecodeKernel<T, KV, D, G, true, true, kStream>, meta);
      else if (a.new_k != nullptr)
        launch_kernel(DecodeKernel<T, KV, D, G, true, false, kStream>, NoStepArgs{});
      else
        launch_kernel(DecodeKernel<T, KV, D, G, false, false, kStream>, NoStepArgs{});
    } else {
      launch_kernel(DecodeKernel<T, KV, D, G, false, false, kStream>, NoStepArgs{});
    }
  };
  if (a.stream_loads) launch(std::true_type{});
  else launch(std::false_type{});
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || P == 1) return e;
  const int BH = a.B * a.Hq;
  if (a.seq_lens == nullptr) {  // lengths in the launch arguments
    hipLaunchKernelGGL((MergeKernel<T, D, true>), dim3((BH + 3) / 4), dim3(256), 0, stream,
                       static_cast<T*>(a.out), ws.acc, ws.ml, a.seq_lens, BH, a.Hq, a.max_seq_len,
                       a.partition_tokens, P, a.auto_items > 0 ? ws.pt : nullptr, meta);
  } else {
    hipLaunchKernelGGL((MergeKernel<T, D, false>), dim3((BH + 3) / 4), dim3(256), 0, stream,
                       static_cast<T*>(a.out), ws.acc, ws.ml, a.seq_lens, BH, a.Hq, a.max_seq_len,
                       a.partition_tokens, P, a.auto_items > 0 ? ws.pt : nullptr, NoStepArgs{});
  }
  return hipGetLastError();
}

template <typename T, typename KV, int D>
hipError_t DispatchG(const DecodeArgs& a, hipStream_t s) {
  switch (a.G) {
    case 1: return LaunchTyped<T, KV, D, 1>(a, s);
    case 2: return LaunchTyped<T, KV, D, 2>(a, s);
    case 4: return LaunchTyped<T, KV, D, 4>(a, s);
    case 8: return LaunchTyped<T, KV, D, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t DispatchD(const DecodeArgs& a, hipStream_t s) {
  return a.D == 64 ? DispatchG<T, T, 64>(a, s) : DispatchG<T, T, 128>(a, s);
}

}  // namespace

int DeviceCuCount() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cus[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t LaunchDecode(const DecodeArgs& a, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  switch (a.dtype) {
    case 0: return DispatchD<float>(a, stream);
    case 1: return DispatchD<uint16_t>(a, stream);
    case 2: return a.D == 128 ? DispatchG<uint16_t, Fp8E4M3, 128>(a, stream) : hipErrorNotSupported;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
