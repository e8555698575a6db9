// Chunked causal prefill over the paged cache, bf16 MFMA (gfx950).
//
// What it computes: a long prompt is processed chunk by chunk ("LLM推理优化：
// 技术原理解析总览", dpshk.com, §2.3 chunked prefill); each chunk's K/V is first
// appended to the paged cache, then every query row of the chunk attends
// causally to the cached tokens up to and including its own position
// ("vLLM 生产级落地深剖", musen-ai.com, §2: prefill and decode share the paged
// cache). Sequence b's chunk has n_b rows; its cache holds L_b tokens (chunk
// included); row i sits at absolute position L_b - n_b + i. Keys and values
// are reached through the sequence's block table, as in decode
// ("vLLM的'内存分页'到底多神奇", xxqk.cn, §3 phase 2). Pool layout
// [num_blocks, block_size, Hkv, D] ("LLM推理优化", §3.3).
//
// How (MI355X-first; FlashAttention-2 on the pages is Ampere prior art):
//  * One workgroup = 8 waves = 256 query rows of one (sequence, kv head): the
//    G q heads that share the kv head are packed into the row dimension
//    (256 / G positions x G heads), so every K/V tile in LDS feeds all of
//    them. Each wave owns 32 rows.
//  * The contraction runs on v_mfma_f32_32x32x16_bf16 in transposed form:
//    S^T = K · Q^T and O^T = V^T · P^T. In the accumulator layout a lane then
//    owns one query row (lane % 32) and 16 keys (or 16 dims) of it, so the
//    online softmax is lane-local (the two half-waves exchange a max only
//    when the running max is raised), and P goes from the S^T accumulators
//    straight into the B operand of the second product with no data
//    movement: the V operand is read in the key order the accumulators hold.
//  * K/V tiles of kKT tokens go from the pool straight into LDS with direct
//    loads (global_load_lds_dwordx4: each lane's 16 bytes land at the
//    instruction's LDS base + 16 x lane), so staging costs no registers, no
//    LDS store instructions and no transpose. V keeps the pool's row-major
//    order in LDS and the PV product reads it transposed with
//    ds_read_b64_tr_b16 (gfx950): within each 16-lane group, lane i receives
//    element i % 4 of the 8-byte pieces addressed by lanes i / 4 + 4k,
//    k = 0..3, so four lanes pointing at four keys' 4-dim pieces give every
//    lane one dim of four keys.
//  * LDS tile layout (K and V alike): key groups of 1 KiB, one load
//    instruction each, of kKeysPerLoad keys (4 at head_dim 128, 8 at 64).
//    Group G's 16-byte unit kKeysPerLoad · pc + (key % kKeysPerLoad) holds
//    16-byte chunk pc ^ (G & kSwz) of that key (dims 8 chunk .. 8 chunk + 7,
//    kSwz = 16 / kKeysPerLoad - 1). The XOR spreads the 32 keys of a K
//    operand read over the banks; V's transposed reads touch 128 contiguous
//    bytes per 16 lanes either way. Each wave loads the key groups of keys
//    8w .. 8w + 7 of the tile (always inside one block) for K and V, with one
//    block id, fetched by one scalar load a tile ahead.
//  * A ring of four tile buffers and two wave groups, one wave of each per
//    SIMD: waves 0-3 run tile j as QK, softmax, PV; waves 4-7 run the softmax
//    and PV of tile j - 1 and then the QK of tile j. Both start a tile
//    together after its barrier. V of tile j - 1 is still read during tile
//    j, so the ring holds j - 1, j, j + 1 (landing) and j + 2 (in flight).
//    (Measured on MI355X with probes: exp, add, fma, max, select and bf16
//    packing of one wave issue while the other wave of the SIMD streams
//    MFMAs, but v_dot2_f32_bf16 and v_mov_b64 wait for them. The LDS serves
//    one read instruction per 4 cycles per CU, 256 B/cycle with
//    ds_read_b128 and 128 with ds_read_b64_tr_b16, so the 384 K and V reads
//    of a tile and the direct loads' writes keep it busy about 1800 cycles,
//    beside the SIMDs' 2048 MFMA cycles per tile.)
//  * MFMA operands are read from LDS four MFMAs ahead of their use.
//  * Online softmax in base 2 with no per-score max, subtraction or scaling
//    in the common case: q is scaled by scale·log2(e) once (rounded to
//    bf16), and each tile's score accumulators start from -m (the running
//    max), so the products are already x - m and the weights are exp2 of
//    them. The weights are packed to bf16 for the PV product and summed in
//    fp32 before the rounding (v_add_f32): a v_dot2_f32_bf16 sum of the
//    packed values, measured on MI355X, does not issue while another wave of
//    the SIMD runs MFMAs, and stalled the softmax behind them. The first tile, and a tile whose half-row
//    weight sum exceeds 2^15 (so no weight is larger), take the tile max,
//    raise m to the true running max, rescale O and l, and take the weights
//    again; every weight stays ≤ 2^15, and the result is exact up to
//    rounding.
//  * Causal mask only on tiles that reach past the smallest position of the
//    workgroup. V rows past the workgroup's last key are zeroed in LDS after
//    their loads land (a zero weight does not cancel a stale non-finite
//    value); K rows there need nothing, the mask replaces their scores.
//  * Work items are mapped XCD-major with the kv head outermost; within it
//    all query tiles of one sequence run together (they share each K/V tile
//    through L2; measured 18% faster than tile-major order), and sequences
//    are taken longest first.
//  * Persistent workgroups, one per CU: the dispatcher sends workgroup i to
//    XCD i % 8, so workgroup i serves XCD i % 8's range of items in bands of
//    as many items as the XCD has CUs, in serpentine order (slot s takes the
//    s-th item of even bands and the s-th from the end of odd ones, which
//    evens out the slots' totals). A grid of one workgroup per item left CUs
//    idle between a workgroup's end and the next one's start; this order
//    measured about 1.5% faster.
//  * Beside a concurrent decode (a mixed serving step) a prefill workgroup
//    still takes a whole CU, and the decode's workgroups wait for CUs. There
//    the kernel serves each XCD's items with the fewest slots whose span
//    stays within kBesideSpanAllowance x the XCD's longest item (costs in key
//    tiles, from the lengths on the device); the workgroups of the other
//    slots leave at once and their CUs go to the decode.
#include "device_common.h"
#include "launch.h"

#include <algorithm>

namespace pa {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = kPrefillRows;  // query rows (positions x heads) per workgroup
static_assert(kRows == 32 * kWaves, "one 32-row MFMA tile per wave");
constexpr int kKT = 64;             // KV tokens per tile
// Largest sum of one half-row's weights in a tile before the running max is
// raised (so every weight stays at most 2^15: finite in bf16 and fp32).
constexpr float kSumLimit = 32768.f;
constexpr int kRankedBatch = 256;   // batches up to this size are ordered by cache length
// Beside a concurrent decode, the prefill may stretch its span to this many
// times its longest item to leave CUs to the decode. Measured on MI355X, a
// step of 56 decode sequences beside 8 x 256-row chunks (graph replay) took
// 262 us with every CU open to the prefill, 242 / 232 / 236 us at 1.0 / 1.1 /
// 1.25, and 294 / 335 us at 1.5 / 2 (the prefill then outlasts the decode).
constexpr float kBesideSpanAllowance = 1.1f;

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef float f32x16v __attribute__((ext_vector_type(16)));
typedef short i16x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4v lds_i16x4v;

// Tile geometry for head_dim D.
template <int D>
struct PGeom {
  static constexpr int kRowBytes = D * 2;                  // one key's K (or V) row
  static constexpr int kKeysPerLoad = 1024 / kRowBytes;    // keys per load instruction (64 lanes x 16 B)
  static constexpr int kChunkBytes = 16 * kKeysPerLoad;    // between chunk slots of a key group
  static constexpr int kSwz = 16 / kKeysPerLoad - 1;       // chunk XOR mask of a key group
  static constexpr int kGroupsPerWave = 8 / kKeysPerLoad;  // key groups of keys 8w .. 8w + 7
  static constexpr int kTileBytes = kKT * kRowBytes;
  static constexpr int kBufBytes = 2 * kTileBytes;         // K tile, then V tile
  static constexpr int kBufs = 4;                          // tile t in buffer t % 4
  static constexpr int kLdsBytes = kBufs * kBufBytes;
  static constexpr int kLoadsPerTile = 2 * kGroupsPerWave; // per wave: K and V of its key groups
  static constexpr int kKSteps = D / 16;                   // MFMA k-steps of S^T = K Q^T
  static constexpr int kDBlocks = D / 32;                  // 32-dim output blocks
  static constexpr int kSBlocks = kKT / 32;                // 32-key S^T accumulator blocks per tile
  static constexpr int kPSteps = kKT / 16;                 // 16-key k-steps of O^T += V^T P^T
  static_assert(kKeysPerLoad * kGroupsPerWave == 8 && kKT / kKeysPerLoad == kGroupsPerWave * kWaves,
                "each wave loads the key groups of 8 keys");
  static_assert(kSwz == 1 || kSwz == 3, "the K read and V read address forms assume a 1- or 2-bit swizzle");
  static_assert(kLdsBytes + kRankedBatch * 4 <= 160 * 1024, "LDS per workgroup");
};

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]).
constexpr int WaitVm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int kWaitLgkm0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);

__device__ __forceinline__ int clamp_blk(int blk, int num_blocks) {
  return (static_cast<unsigned>(blk) < static_cast<unsigned>(num_blocks)) ? blk : 0;
}

template <int D, int G>
__global__ __launch_bounds__(kThreads, 1) void PrefillKernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const char* __restrict__ kc,
    const char* __restrict__ vc, const int32_t* __restrict__ cu_q_lens,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ seq_lens, int32_t B,
    int32_t Hkv, int32_t max_blocks, int32_t bs_shift, int32_t num_blocks, int32_t n_qtiles,
    int32_t per_xcd, float scale_log2, float span_allowance) {
  using PG = PGeom<D>;
  constexpr int QP = kRows / G;  // positions per workgroup
  constexpr int kKeysPerLoad = PG::kKeysPerLoad, kChunkBytes = PG::kChunkBytes, kSwz = PG::kSwz;
  constexpr int kGPW = PG::kGroupsPerWave;
  constexpr int kTileBytes = PG::kTileBytes, kBufBytes = PG::kBufBytes, kBufs = PG::kBufs;
  constexpr int kLoadsPerTile = PG::kLoadsPerTile;
  constexpr int kKSteps = PG::kKSteps, kDBlocks = PG::kDBlocks, kSBlocks = PG::kSBlocks, kPSteps = PG::kPSteps;
  // 16-byte aligned: the direct loads and the 128-bit reads address 16-byte units.
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;   // query row within the wave (accumulator column)
  const int h2 = lane >> 5;  // half-wave

  // ---- work items: kv head outermost (one XCD's range when Hkv = 8), then
  // sequence (longest cache first, ranked here for batches up to
  // kRankedBatch, so the short ones fill the tail), then query tile (last
  // first). All query tiles of a sequence run together, so each K/V tile they
  // all read comes from L2 after the first.
  const int wg = blockIdx.x;
  __shared__ int s_order[kRankedBatch];
  if (B <= kRankedBatch) {
    if (tid < B) {
      const int key = seq_lens[tid];
      int rank = 0;
      for (int u = 0; u < B; ++u) {
        const int ku = seq_lens[u];
        rank += (ku > key) || (ku == key && u < tid);
      }
      s_order[rank] = tid;
    }
    __syncthreads();
  }
  // Workgroup wg serves XCD wg % 8's range of items in bands of nslots
  // items, serpentine over the bands; every branch below that skips an item
  // is workgroup-uniform.
  const int xcd = wg & 7;
  const int slot = wg >> 3;
  int nslots = static_cast<int>(gridDim.x) >> 3;
  const int total = Hkv * n_qtiles * B;
  const int lo_item = xcd * per_xcd;
  const int count = max(0, min(per_xcd, total - lo_item));
  if (span_allowance > 0.f) {
    // Beside a concurrent decode: serve the XCD's items with the fewest slots
    // whose span stays within span_allowance x its longest item (in key
    // tiles, plus one per item for its start and end), so the other CUs go
    // to the decode from the start. The workgroups of the unused slots leave.
    float tsum = 0.f, tmax = 0.f;
    for (int i = tid; i < count; i += kThreads) {
      const int item = lo_item + i;
      const int rem = item % (n_qtiles * B);
      const int q0 = (n_qtiles - 1 - rem % n_qtiles) * QP;
      int b = rem / n_qtiles;
      if (B <= kRankedBatch) b = s_order[b];
      const int nq = cu_q_lens[b + 1] - cu_q_lens[b];
      if (q0 >= nq) continue;
      const int L = min(max(seq_lens[b], 0), max_blocks << bs_shift);
      const int keys = max(L - nq + min(q0 + QP, nq), 0);
      const float c = static_cast<float>((keys + kKT - 1) / kKT + 1);
      tsum += c;
      tmax = fmaxf(tmax, c);
    }
    __shared__ float s_red[2][kWaves];
    tsum = wave_reduce(tsum, OpAdd{});
    tmax = wave_reduce(tmax, OpMax{});
    if (lane == 0) {
      s_red[0][w] = tsum;
      s_red[1][w] = tmax;
    }
    __syncthreads();
    tsum = 0.f;
    tmax = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      tsum += s_red[0][v];
      tmax = fmaxf(tmax, s_red[1][v]);
    }
    if (tmax > 0.f) nslots = min(nslots, max(1, static_cast<int>(ceilf(tsum / (span_allowance * tmax)))));
    if (slot >= nslots) return;
  }
  for (int band = 0; band * nslots < count; ++band) {
    const int local = band * nslots + ((band & 1) ? nslots - 1 - slot : slot);
    if (local >= count) continue;  // workgroup-uniform
    const int item = lo_item + local;
    __syncthreads();  // every wave is done with the previous item's LDS
    const int g = item / (n_qtiles * B);
    const int rem = item - g * (n_qtiles * B);
    const int tile = n_qtiles - 1 - rem % n_qtiles;
    int b = rem / n_qtiles;
    if (B <= kRankedBatch) b = __builtin_amdgcn_readfirstlane(s_order[b]);

    const int qbeg = cu_q_lens[b];
    const int nq = cu_q_lens[b + 1] - qbeg;
    const int q0 = tile * QP;
    if (q0 >= nq) continue;
    const int bs = 1 << bs_shift;
    int L = seq_lens[b];
    L = min(max(L, 0), max_blocks * bs);
    const int ctx = L - nq;
    const int Hq = Hkv * G;

    const int mrow = w * 32 + n;
    const int hl = mrow / QP;
    const int qpos = q0 + (mrow - hl * QP);
    const bool row_valid = qpos < nq;
    const int apos = ctx + qpos;
    const int64_t row_off = (static_cast<int64_t>(qbeg + qpos) * Hq + g * G + hl) * D;

    // q fragment s of a half-wave: dims 16 s + 8 h2 .. + 7 (k-step s of the
    // K operand reads below takes the same dims of 32 keys).
    uint4 qraw[kKSteps];
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) {
      qraw[s] = make_uint4(0, 0, 0, 0);
      if (row_valid) qraw[s] = *reinterpret_cast<const uint4*>(q + row_off + 16 * s + 8 * h2);
    }
    bf16x8v qf[kKSteps];

    const int kv_end = max(0, ctx + min(q0 + QP, nq));
    const int n_tiles = (kv_end + kKT - 1) / kKT;
    const int min_apos = ctx + q0;

    // ---- direct loads. Lane l of a load moves 16-byte unit l of key group Gi:
    // key kKeysPerLoad Gi + l % kKeysPerLoad, chunk (l / kKeysPerLoad) ^
    // (Gi & kSwz). Its byte offset inside the key's block is fixed for the
    // kernel (tiles start on multiples of 64 tokens and blocks hold at most
    // 32).
    const int32_t* trow = tables + static_cast<int64_t>(b) * max_blocks;
    const uint32_t row_bytes = static_cast<uint32_t>(Hkv) * PG::kRowBytes;
    const uint32_t blk_bytes = static_cast<uint32_t>(bs) * row_bytes;  // < 4 GiB, checked at launch
    uint32_t ld_off[kGPW];
#pragma unroll
    for (int i = 0; i < kGPW; ++i) {
      const int Gi = kGPW * w + i;
      const int key = kKeysPerLoad * Gi + lane % kKeysPerLoad;
      ld_off[i] = static_cast<uint32_t>(key & (bs - 1)) * row_bytes + static_cast<uint32_t>(g) * PG::kRowBytes +
                  static_cast<uint32_t>(((lane / kKeysPerLoad) ^ (Gi & kSwz)) * 16);
    }
    const int last_blk = (kv_end - 1) >> bs_shift;  // used only when n_tiles > 0
    // The block id of this wave's keys in tile jt (clamped to the last block
    // the workgroup needs): one scalar load, wave-uniform.
    auto block_of = [&](int jt) {
      const int lb = min((jt * kKT + 8 * w) >> bs_shift, last_blk);
      return clamp_blk(trow[lb], num_blocks);
    };
    // The loads are written as inline assembly, not with the compiler's
    // builtin: the compiler then waits for every load in flight before any
    // transposed LDS read (it cannot tell which LDS bytes a load writes),
    // which would serialise the pipeline. Their completion is tracked here
    // instead, with explicit vmcnt waits; every other vector-memory load of
    // the kernel is issued before them or waited for at a point where all of
    // them have to be complete anyway. The LDS destination goes in M0 (an
    // input operand, so the compiler sets it).
    const uint32_t lds_base = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds));
    auto issue_tile = [&](int blk, int buf) {
      const uint64_t off = static_cast<uint64_t>(static_cast<uint32_t>(blk)) * blk_bytes;
      const uint64_t kbase = reinterpret_cast<uint64_t>(kc) + off;
      const uint64_t vbase = reinterpret_cast<uint64_t>(vc) + off;
      const uint32_t kd = lds_base + static_cast<uint32_t>(buf * kBufBytes + (kGPW * w) * 1024);
#pragma unroll
      for (int i = 0; i < kGPW; ++i) {
        asm volatile("global_load_lds_dwordx4 %0, %1"
                     :: "v"(ld_off[i]), "s"(kbase), "{m0}"(kd + i * 1024) : "memory");
        asm volatile("global_load_lds_dwordx4 %0, %1"
                     :: "v"(ld_off[i]), "s"(vbase), "{m0}"(kd + kTileBytes + i * 1024) : "memory");
      }
    };
    // V rows past the workgroup's last key may hold anything (stale slots,
    // NaN): after this wave's loads of tile t have landed, its rows there are
    // zeroed (their weights are 0, and 0 x NaN would not be). Only the last
    // tile has such rows. K rows there need nothing: the causal mask replaces
    // their scores.
    auto zero_tail = [&](int t, int buf) {
      if (t * kKT + 8 * w + 8 > kv_end) {  // wave-uniform
        char* vd = lds + buf * kBufBytes + kTileBytes + (kGPW * w) * 1024;
#pragma unroll
        for (int i = 0; i < kGPW; ++i)
          if (t * kKT + kKeysPerLoad * (kGPW * w + i) + lane % kKeysPerLoad >= kv_end)
            *reinterpret_cast<uint4*>(vd + i * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      }
    };

    // ---- per-lane LDS read addresses (added to a buffer's LDS address).
    // K operand (tb, st): key 32 tb + n, chunk 2 st + h2, in group
    // (32 tb + n) / kKeysPerLoad, whose swizzle s = (n / kKeysPerLoad) & kSwz
    // (32 tb / kKeysPerLoad is a multiple of kSwz + 1). For s < 4,
    // (2 st + h2) ^ s = 4 (st / 2) + ((2 (st % 2) + h2) ^ s), so two bases
    // (st even / odd) plus immediates cover all of them.
    uint32_t k_lane[2];
#pragma unroll
    for (int e = 0; e < 2; ++e)
      k_lane[e] = (n / kKeysPerLoad) * 1024 + (n % kKeysPerLoad) * 16 +
                  (((2 * e + h2) ^ ((n / kKeysPerLoad) & kSwz)) * kChunkBytes);
    // V^T operand (db, k4), read r (0, 1): lane a of 16-lane group gg points at
    // key 16 k4 + 8 r + 4 h2 + a / 4, dims 32 db + 16 (gg & 1) + 4 (a & 3) .. + 3;
    // the key order matches the S^T accumulator rows (element e of a half-wave:
    // key 8 (e / 4) + 4 h2 + e % 4 of the 16-key step). With kq = 8 r + 4 h2 +
    // a / 4 the key sits in group 16 k4 / kKeysPerLoad + kq / kKeysPerLoad,
    // whose swizzle is (kq / kKeysPerLoad) & kSwz, at slot kq % kKeysPerLoad;
    // its chunk is 4 db + x, x = 2 (gg & 1) + (a / 2) % 2 < 4, so the XOR only
    // touches x and k4, db add immediates.
    uint32_t v_lane[2];
    {
      const int gg = lane >> 4, a = lane & 15;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int kq = 8 * r + 4 * h2 + (a >> 2);
        const int gs = kq / kKeysPerLoad, sw = gs & kSwz;
        v_lane[r] = kTileBytes + gs * 1024 + (((2 * (gg & 1) + ((a >> 1) & 1)) ^ sw) * kChunkBytes) +
                    (kq % kKeysPerLoad) * 16 + 8 * (a & 1);
      }
    }
    auto lds_b128 = [](uint32_t addr) {
      return __builtin_bit_cast(bf16x8v, *reinterpret_cast<const __attribute__((address_space(3))) uint4*>(
                                             static_cast<uintptr_t>(addr)));
    };
    auto lds_tr = [](uint32_t addr) {
      return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                           reinterpret_cast<lds_i16x4v*>(static_cast<uintptr_t>(addr))));
    };

    f32x16v o[kDBlocks];
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[db][v] = 0.f;
    float m = -INFINITY;
    float l = 0.f;
    f32x16v negm;
#pragma unroll
    for (int v = 0; v < 16; ++v) negm[v] = 0.f;
    f32x16v s[kSBlocks];     // S^T of the tile between its product and its softmax
    bf16x8v p[kPSteps];

    // S^T = K · Q^T of tile j (from buffer buf), onto -m: s[] = x - m in log2 units.
    auto qk_tile = [&](int buf) {
      const uint32_t kb0 = lds_base + static_cast<uint32_t>(buf * kBufBytes) + k_lane[0];
      const uint32_t kb1 = lds_base + static_cast<uint32_t>(buf * kBufBytes) + k_lane[1];
      constexpr int kQK = kSBlocks * kKSteps;
      constexpr int kAhead = 4;
      auto k_operand = [&](int idx) {
        const int tb = idx / kKSteps, st = idx % kKSteps;
        return lds_b128(((st & 1) ? kb1 : kb0) +
                        static_cast<uint32_t>(tb * (32 / kKeysPerLoad) * 1024 + (st >> 1) * 4 * kChunkBytes));
      };
      bf16x8v kop[kAhead];
#pragma unroll
      for (int u = 0; u < kAhead; ++u) kop[u] = k_operand(u);
#pragma unroll
      for (int idx = 0; idx < kQK; ++idx) {
        const int tb = idx / kKSteps, st = idx % kKSteps;
        const bf16x8v a = kop[idx % kAhead];
        if (idx + kAhead < kQK) kop[idx % kAhead] = k_operand(idx + kAhead);
        if (st == 0) {
          s[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], negm, 0, 0, 0);
        } else {
          s[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[tb], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
      for (int idx = 0; idx < kQK - kAhead; ++idx) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
    };

    // Causal mask, weights P and the running max / sum of tile j.
    auto softmax_tile = [&](int j) {
      const int t0 = j * kKT;
      if (t0 + kKT - 1 > min_apos) {
#pragma unroll
        for (int tb = 0; tb < kSBlocks; ++tb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int t = t0 + 32 * tb + 8 * (v >> 2) + 4 * h2 + (v & 3);
            s[tb][v] = t <= apos ? s[tb][v] : -INFINITY;
          }
      }
      auto weights = [&](float shift) {
        float lt[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tb = 0; tb < kSBlocks; ++tb)
#pragma unroll
          for (int hs = 0; hs < 2; ++hs)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float wt = fast_exp2(s[tb][8 * hs + e] - shift);
              p[2 * tb + hs][e] = static_cast<__bf16>(wt);
              lt[e & 3] += wt;
            }
        return (lt[0] + lt[1]) + (lt[2] + lt[3]);
      };
      float lt = 0.f;
      bool exact = j == 0;
      if (!exact) {
        lt = weights(0.f);
        exact = __builtin_amdgcn_ballot_w64(!(lt <= kSumLimit)) != 0;
      }
      if (exact) {
        float T = -INFINITY;
#pragma unroll
        for (int tb = 0; tb < kSBlocks; ++tb)
#pragma unroll
          for (int v = 0; v < 16; ++v) T = fmaxf(T, s[tb][v]);
        T = fmaxf(T, __shfl_xor(T, 32));
        const float M = m == -INFINITY ? 0.f : m;
        const float mn = fmaxf(m, M + T);
        const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - mn);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
        m = mn;
        const float nm = m == -INFINITY ? 0.f : -m;
#pragma unroll
        for (int v = 0; v < 16; ++v) negm[v] = nm;
        lt = weights(m == -INFINITY ? 0.f : m - M);
      }
      l += lt;
    };

    // O^T += V^T · P^T of the tile in buffer buf.
    auto pv_tile = [&](int buf) {
      const uint32_t vb0 = lds_base + static_cast<uint32_t>(buf * kBufBytes) + v_lane[0];
      const uint32_t vb1 = lds_base + static_cast<uint32_t>(buf * kBufBytes) + v_lane[1];
      constexpr int kPV = kDBlocks * kPSteps;
      constexpr int kAhead = 4;
      auto v_operand = [&](int idx) {
        const int db = idx / kPSteps, k4 = idx % kPSteps;
        const uint32_t imm = static_cast<uint32_t>(k4 * (16 / kKeysPerLoad) * 1024 + db * 4 * kChunkBytes);
        const uint2 lo = lds_tr(vb0 + imm), hi = lds_tr(vb1 + imm);
        return __builtin_bit_cast(bf16x8v, make_uint4(lo.x, lo.y, hi.x, hi.y));
      };
      bf16x8v vop[kAhead];
#pragma unroll
      for (int u = 0; u < kAhead; ++u) vop[u] = v_operand(u);
#pragma unroll
      for (int idx = 0; idx < kPV; ++idx) {
        const int db = idx / kPSteps, k4 = idx % kPSteps;
        const bf16x8v a = vop[idx % kAhead];
        if (idx + kAhead < kPV) vop[idx % kAhead] = v_operand(idx + kAhead);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[k4], o[db], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 0);
#pragma unroll
      for (int idx = 0; idx < kPV - kAhead; ++idx) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
    };

    auto scale_q = [&]() {
#pragma unroll
      for (int st = 0; st < kKSteps; ++st) {
        const uint32_t wv[4] = {qraw[st].x, qraw[st].y, qraw[st].z, qraw[st].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          qf[st][2 * k] = static_cast<__bf16>(__uint_as_float(wv[k] << 16) * scale_log2);
          qf[st][2 * k + 1] = static_cast<__bf16>(__uint_as_float(wv[k] & 0xFFFF0000u) * scale_log2);
        }
      }
    };

    // Two wave groups, one wave of each per SIMD (waves w and w + 4): group 0
    // runs tile j as product, softmax, product; group 1 runs the softmax and
    // PV product of tile j - 1 and then the scores of tile j. Both start a tile
    // together after its barrier, so one group's softmax (VALU) meets the
    // other's matrix products and the SIMD's matrix core is fed from two
    // instruction streams in different phases. Group 1 still reads V of tile
    // j - 1 during tile j, so the ring holds four tiles: j - 1 (V), j (K, V),
    // j + 1 (landing) and j + 2 (in flight).
    const bool lag = w >= kWaves / 2;  // wave-uniform
    if (n_tiles > 0) {
      // Start-up: tile 0 loads behind q; the compiler's wait for q (it cannot
      // see the tile loads) also covers tile 0, and tile 1 is issued after it,
      // so the loop starts with exactly one tile in flight as in steady state.
      // Every path issues kLoadsPerTile loads per tile (past the end the last
      // tile is re-read), so the waits below count exactly.
      issue_tile(block_of(0), 0);
      scale_q();
      issue_tile(block_of(min(1, n_tiles - 1)), 1);
      int blk_next = block_of(min(2, n_tiles - 1));
      __builtin_amdgcn_s_waitcnt(WaitVm(kLoadsPerTile));
      zero_tail(0, 0);
      __builtin_amdgcn_s_barrier();
      // The block id of tile j + 3 loads before each barrier, so its latency
      // overlaps the wait and the barrier. This wave's loads of tile j + 1 have
      // landed once at most the kLoadsPerTile loads of tile j + 2 are pending;
      // the barrier then publishes every wave's, and ends all reads of tile
      // j - 1 before its buffer is refilled. The two groups run separate loops
      // (one barrier per tile each, so they stay matched): a shared loop body
      // with both schedules in it needs far more registers than either.
      auto end_tile = [&](int j) {
        blk_next = block_of(min(j + 3, n_tiles - 1));
        __builtin_amdgcn_s_waitcnt(WaitVm(kLoadsPerTile));
        if (j + 1 < n_tiles) zero_tail(j + 1, (j + 1) % kBufs);
        __builtin_amdgcn_s_barrier();
      };
      if (!lag) {
        for (int j = 0; j < n_tiles; ++j) {
          issue_tile(blk_next, (j + 2) % kBufs);
          __builtin_amdgcn_s_setprio(1);
          qk_tile(j % kBufs);
          __builtin_amdgcn_s_setprio(0);
          softmax_tile(j);
          __builtin_amdgcn_s_setprio(1);
          pv_tile(j % kBufs);
          end_tile(j);
        }
      } else {
        for (int j = 0; j < n_tiles; ++j) {
          issue_tile(blk_next, (j + 2) % kBufs);
          if (j > 0) {
            __builtin_amdgcn_s_setprio(0);
            softmax_tile(j - 1);
            __builtin_amdgcn_s_setprio(1);
            pv_tile((j - 1) % kBufs);
          }
          __builtin_amdgcn_s_setprio(1);
          qk_tile(j % kBufs);
          end_tile(j);
        }
        __builtin_amdgcn_s_setprio(0);
        softmax_tile(n_tiles - 1);
        __builtin_amdgcn_s_setprio(1);
        pv_tile((n_tiles - 1) % kBufs);
      }
      __builtin_amdgcn_s_waitcnt(WaitVm(0));  // no load may land in LDS after the item ends
    } else {
      scale_q();
    }

    const float lsum = l + __shfl_xor(l, 32);
    if (row_valid) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      uint16_t* orow = out + row_off;
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const int d = 32 * db + 8 * grp + 4 * h2;
          typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
          bf16x4v r;
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = static_cast<__bf16>(o[db][4 * grp + e] * inv);
          *reinterpret_cast<uint2*>(orow + d) = __builtin_bit_cast(uint2, r);
        }
    }
  }
}

template <int D, int G>
hipError_t LaunchTyped(const PrefillArgs& a, hipStream_t stream) {
  using PG = PGeom<D>;
  constexpr int QP = kRows / G;
  const int n_qtiles = (a.max_q_len + QP - 1) / QP;
  const int64_t items = PrefillWorkItems(a.Hkv, a.G, a.B, a.max_q_len);
  if (items == 0) return hipSuccess;
  if (items >= (int64_t{1} << 31) - 8) return hipErrorInvalidValue;
  // The kernel forms a block's byte offset in 32 bits.
  if (static_cast<int64_t>(a.block_size) * a.Hkv * PG::kRowBytes >= (int64_t{1} << 32)) return hipErrorInvalidValue;
  const int per_xcd = static_cast<int>((items + 7) / 8);
  // One persistent workgroup per CU (its registers, and at head_dim 128 its
  // LDS ring, leave room for no second), each serving its XCD's items in
  // turn; fewer when an XCD has fewer items than CUs.
  const int nslots = std::max(1, std::min(per_xcd, DeviceCuCount() / 8));
  // More than 64 KiB of dynamic LDS: raise the kernel's limit once.
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&PrefillKernel<D, G>), hipFuncAttributeMaxDynamicSharedMemorySize,
      PG::kLdsBytes);
  if (attr != hipSuccess) return attr;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((PrefillKernel<D, G>), dim3(nslots * 8), dim3(kThreads), PG::kLdsBytes, stream,
                     static_cast<uint16_t*>(a.out), static_cast<const uint16_t*>(a.q),
                     static_cast<const char*>(a.k_cache), static_cast<const char*>(a.v_cache),
                     a.cu_q_lens, a.block_tables, a.seq_lens, a.B, a.Hkv, a.max_blocks,
                     __builtin_ctz(a.block_size), a.num_blocks, n_qtiles, per_xcd, scale_log2,
                     a.beside_decode ? kBesideSpanAllowance : 0.f);
  return hipGetLastError();
}

template <int D>
hipError_t DispatchG(const PrefillArgs& a, hipStream_t s) {
  switch (a.G) {
    case 1: return LaunchTyped<D, 1>(a, s);
    case 2: return LaunchTyped<D, 2>(a, s);
    case 4: return LaunchTyped<D, 4>(a, s);
    case 8: return LaunchTyped<D, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t LaunchPrefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.B == 0 || a.max_q_len == 0) return hipSuccess;
  return a.D == 64 ? DispatchG<64>(a, stream) : DispatchG<128>(a, stream);
}

}  // namespace pa
