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
//    (256 / G positions x G heads), so every K/V tile staged in LDS feeds all
//    of them. Each wave owns 32 rows.
//  * The contraction runs on v_mfma_f32_32x32x16_bf16 in transposed form:
//    S^T = K · Q^T and O^T = V^T · P^T. In the accumulator layout a lane then
//    owns one query row (lane % 32) and 16 keys (or 16 dims) of it, so the
//    online softmax is lane-local (the two half-waves exchange a max only
//    when the running max is raised), and P goes from the S^T accumulators straight
//    into the B operand of the second product with no data movement: the key
//    order inside each 16-key step is permuted consistently on both sides
//    (V^T is written to LDS in that permuted order).
//  * Two ways of bringing K/V tiles of kKT tokens into LDS. head_dim 128
//    (PrefillDmaKernel, below): direct loads from the pool into LDS, V read
//    transposed from LDS, and two wave groups offset by half a tile; see its
//    own notes. head_dim 64 (PrefillKernel): staged through registers, as
//    follows. K as [token][dim], V transposed to [dim][token]
//    (transposed in registers with v_perm before the LDS write), both with
//    padded rows so that every MFMA operand read is one ds_read_b128 at a
//    per-lane base plus an immediate offset, free of bank conflicts;
//    double-buffered (70 KiB of LDS; gfx950 allows 160 KiB per workgroup).
//    Half the threads stage K, half V. Global loads run two tiles ahead of
//    the multiply (two register staging sets) and block ids three, so the
//    latency of a load is covered by two tiles of MFMA work and no load
//    waits on a table lookup. A tile's block ids take one table load per
//    lane; each thread picks its loads' ids with ds_bpermute just before the
//    per-tile barrier, and a load's address is one 32x32-bit multiply-add.
//    V rows past the causal end of the workgroup are staged as zeros (stale
//    slots of the last block may hold anything, and a zero weight does not
//    cancel a non-finite value); K rows there are left as loaded, since the
//    causal mask replaces their scores.
//  * MFMA operands are read from LDS four MFMAs ahead of their use.
//  * Wave priority: 0 during the softmax of a tile, 1 otherwise, so that of
//    the two waves sharing a SIMD the one with MFMAs to issue goes first.
//  * Online softmax in base 2 with no per-score max, subtraction or scaling
//    in the common case: q is scaled by scale·log2(e) once (rounded to
//    bf16), and each tile's score accumulators start from -m (the running
//    max), so the products are already x - m and the weights are exp2 of
//    them. The weights, packed to bf16 for the PV product, are summed two at
//    a time with v_dot2_f32_bf16 (the denominator adds exactly the values
//    the numerator multiplies). The first tile, and a tile whose half-row
//    weight sum exceeds 2^15 (so no weight is larger), take the tile max,
//    raise m to the true running max, rescale O and l, and take the weights
//    again; every weight stays ≤ 2^15, and the result is exact up to
//    rounding.
//  * Causal mask only on tiles that reach past the smallest position of the
//    workgroup. Work items are mapped XCD-major with the kv head outermost;
//    within it all query tiles of one sequence run together (they share each
//    K/V tile through L2; measured 18% faster than tile-major order), and
//    sequences are taken longest first.
#include "device_common.h"
#include "launch.h"

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
constexpr uint32_t kBf16Ones = 0x3F803F80u;  // (1.0, 1.0) as packed bf16
constexpr int kRankedBatch = 256;   // batches up to this size are ordered by cache length

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef float f32x16v __attribute__((ext_vector_type(16)));

template <int D>
struct PGeom {
  static constexpr int kKSteps = D / 16;      // MFMA k-steps for S^T = K Q^T
  static constexpr int kDBlocks = D / 32;     // 32-dim output blocks
  static constexpr int kChunks = D / 8;       // 16-byte chunks per K/V row
  static constexpr int kKPitch = D + 8;       // K tile row pitch (elements): 16 B pad
  static constexpr int kVPitch = kKT + 8;     // V^T tile row pitch (elements): 16 B pad
  static constexpr int kKElems = kKT * kKPitch;
  static constexpr int kVElems = D * kVPitch;
  static constexpr int kBufElems = kKElems + kVElems;
  static constexpr int kSBlocks = kKT / 32;   // 32-key S^T accumulator blocks per tile
  static constexpr int kPSteps = kKT / 16;    // 16-key MFMA k-steps of O^T += V^T P^T
  static constexpr int kStageThreads = kThreads / 2;                 // K stagers, then V stagers
  static constexpr int kKLoads = kKT * kChunks / kStageThreads;      // 16-byte K chunks per K stager
  // V is staged in groups of kVGroupTok consecutive tokens of one chunk (the
  // unit of the in-register transpose); each V stager moves kVGroups groups,
  // so that it issues exactly as many loads as a K stager.
  static constexpr int kVGroupTok = kKLoads < 4 ? kKLoads : 4;
  static constexpr int kVGroups = kKLoads / kVGroupTok;
  static_assert((kKT / kVGroupTok) * kChunks == kVGroups * kStageThreads, "V staging covers the tile");
  static constexpr int kSRegs = kKLoads;      // loads per staging thread per tile (both roles)
  static_assert(kKT % 32 == 0 && kKLoads >= 1, "tile geometry");
};

// Position of key t (0..kKT-1) inside a V^T row: within each 16-key MFMA step,
// half-wave h takes keys {4h..4h+3, 8+4h..8+4h+3}, which are the keys its
// S^T accumulators hold; they are stored contiguously so one 16-byte read
// fetches them.
__device__ __forceinline__ int vt_pos(int t) {
  const int blk = t >> 5, w = t & 31, s = w >> 4, w16 = w & 15;
  const int h = (w16 >> 2) & 1, e = ((w16 >> 3) << 2) | (w16 & 3);
  return (blk << 5) | (s << 4) | (h << 3) | e;
}

__device__ __forceinline__ uint32_t perm_lo(uint32_t x, uint32_t y) {  // (x.lo, y.lo)
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t x, uint32_t y) {  // (x.hi, y.hi)
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

__device__ __forceinline__ int clamp_blk(int blk, int num_blocks) {
  return (static_cast<unsigned>(blk) < static_cast<unsigned>(num_blocks)) ? blk : 0;
}

template <int D, int G>
__global__ __launch_bounds__(kThreads, 1) void PrefillKernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ cu_q_lens,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ seq_lens, int32_t B,
    int32_t Hkv, int32_t max_blocks, int32_t bs_shift, int32_t num_blocks, int32_t n_qtiles,
    int32_t per_xcd, float scale_log2) {
  using PG = PGeom<D>;
  constexpr int QP = kRows / G;  // positions per workgroup
  extern __shared__ uint16_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;   // query row within the wave (accumulator column)
  const int h2 = lane >> 5;  // half-wave

  // ---- work item: kv head outermost (one XCD's range when Hkv = 8), then
  // sequence, then query tile (last first). All query tiles of a sequence run
  // together, so each K/V tile they all read comes from L2 after the first.
  // Sequences go longest cache first (ranked here for batches up to
  // kRankedBatch), so the short ones fill the tail.
  const int wg = blockIdx.x;
  const int item = (wg & 7) * per_xcd + (wg >> 3);
  if (item >= Hkv * n_qtiles * B) return;
  const int g = item / (n_qtiles * B);
  const int rem = item - g * (n_qtiles * B);
  const int tile = n_qtiles - 1 - rem % n_qtiles;
  int b = rem / n_qtiles;
  if (B <= kRankedBatch) {
    __shared__ int s_order[kRankedBatch];
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
    b = s_order[b];
  }

  const int qbeg = cu_q_lens[b];
  const int nq = cu_q_lens[b + 1] - qbeg;
  const int q0 = tile * QP;
  if (q0 >= nq) return;
  const int bs = 1 << bs_shift;
  int L = seq_lens[b];
  L = min(max(L, 0), max_blocks * bs);
  const int ctx = L - nq;
  const int Hq = Hkv * G;

  // ---- this lane's query row
  const int mrow = w * 32 + n;
  const int hl = mrow / QP;
  const int qpos = q0 + (mrow - hl * QP);
  const bool row_valid = qpos < nq;
  const int apos = ctx + qpos;  // attends to keys 0..apos
  const int64_t row_off = (static_cast<int64_t>(qbeg + qpos) * Hq + g * G + hl) * D;

  // The query row, loaded here and scaled by scale·log2(e) (rounded to bf16)
  // once the start-up loads have arrived, so that the products give scores in
  // log2 units directly.
  uint4 qraw[PG::kKSteps];
#pragma unroll
  for (int s = 0; s < PG::kKSteps; ++s) {
    qraw[s] = make_uint4(0, 0, 0, 0);
    if (row_valid) qraw[s] = *reinterpret_cast<const uint4*>(q + row_off + (D / 2) * h2 + 8 * s);
  }
  bf16x8v qf[PG::kKSteps];

  // Keys the workgroup needs: 0 .. kv_end-1 (the last valid row's position).
  const int kv_end = max(0, ctx + min(q0 + QP, nq));
  const int n_tiles = (kv_end + kKT - 1) / kKT;
  const int min_apos = ctx + q0;

  const int32_t* trow = tables + static_cast<int64_t>(b) * max_blocks;
  const int64_t slot_stride = static_cast<int64_t>(Hkv) * D;

  // ---- staging roles: waves [0, 4) stage K chunks, waves [4, 8) stage V groups.
  // A K stager moves chunks (token, c) with c fastest across lanes (a 256-byte
  // row per 16 lanes). A V stager moves 4-token groups (tg, c) with tg fastest
  // across lanes, so the transposed LDS writes of one instruction spread over
  // the banks. Both roles issue the same number of K/V loads, with no branch
  // around them (block ids are clamped into the sequence's valid range): the
  // compiler can then count loads in flight exactly and wait only for the
  // ones a step needs.
  const bool k_stager = w < kWaves / 2;  // wave-uniform
  const int st_id = k_stager ? tid : tid - PG::kStageThreads;
  constexpr int kKTokStride = PG::kStageThreads / PG::kChunks;
  constexpr int GT = PG::kVGroupTok;
  constexpr int kGroupsPerTile = kKT / GT;

  // Load i of this thread: its token within the tile and its 16-byte chunk.
  auto stage_tok = [&](int i) {
    if (k_stager) return st_id / PG::kChunks + i * kKTokStride;
    const int pair = st_id + (i / GT) * PG::kStageThreads;
    return GT * (pair % kGroupsPerTile) + (i % GT);
  };
  auto stage_chunk = [&](int i) {
    if (k_stager) return st_id % PG::kChunks;
    return (st_id + (i / GT) * PG::kStageThreads) / kGroupsPerTile;
  };

  using StageRegs = uint4[PG::kSRegs];  // K: kKLoads chunks; V: 4 tokens per group

  // Per-thread constants of the staging pattern. A 64-token tile starts at a
  // multiple of 64, so for block sizes up to 64 the block a load falls in
  // (counted from the tile's first block) and its row inside that block are
  // the same on every tile; for larger blocks the whole tile sits in one
  // block at a row offset shared by the workgroup.
  const bool small_bs = bs <= kKT;
  const uint32_t blk_bytes = static_cast<uint32_t>(bs * slot_stride * 2);  // < 4 GiB, checked at launch
  const char* stage_pool = reinterpret_cast<const char*>(k_stager ? kc : vc);
  int st_bi4[PG::kSRegs];          // 4 x (block of load i within the tile): a ds_bpermute address
  uint64_t st_off[PG::kSRegs];     // byte offset of load i's row, head and chunk inside its block
#pragma unroll
  for (int i = 0; i < PG::kSRegs; ++i) {
    const int tk = stage_tok(i);
    st_bi4[i] = small_bs ? 4 * (tk >> bs_shift) : 0;
    const int row = small_bs ? (tk & (bs - 1)) : tk;
    st_off[i] = (static_cast<uint64_t>(row) * slot_stride + static_cast<uint64_t>(g) * D + 8 * stage_chunk(i)) * 2u;
  }

  // Block ids of one tile, one per lane (lane j: the tile's j-th block,
  // clamped to the sequence's last block): one table load per lane, issued
  // two tiles ahead of the K/V loads that use them.
  auto fetch_ids = [&](int jt) {
    const int blk0 = (jt * kKT) >> bs_shift;
    const int last = (kv_end - 1) >> bs_shift;
    return trow[min(blk0 + lane, last)];  // range-checked in spread_ids
  };
  // The block id of each of this thread's loads, taken from the lane that
  // holds it. Done just before a barrier, whose LDS wait covers the permutes.
  using LoadIds = int[PG::kSRegs];
  // (Inline assembly keeps the permutes at this point; it waits for them
  // itself, since the compiler does not count LDS operations it cannot see.)
  auto spread_ids = [&](int ids, LoadIds& out) {
    const int idc = clamp_blk(ids, num_blocks);
    if constexpr (PG::kSRegs == 4) {
      asm volatile(
          "ds_bpermute_b32 %0, %4, %8\n\t"
          "ds_bpermute_b32 %1, %5, %8\n\t"
          "ds_bpermute_b32 %2, %6, %8\n\t"
          "ds_bpermute_b32 %3, %7, %8\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3])
          : "v"(st_bi4[0]), "v"(st_bi4[1]), "v"(st_bi4[2]), "v"(st_bi4[3]), "v"(idc));
    } else {
      static_assert(PG::kSRegs == 2, "two or four loads per staging thread");
      asm volatile(
          "ds_bpermute_b32 %0, %2, %4\n\t"
          "ds_bpermute_b32 %1, %3, %4\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(out[0]), "=&v"(out[1])
          : "v"(st_bi4[0]), "v"(st_bi4[1]), "v"(idc));
    }
  };

  auto load_tile = [&](int jt, const LoadIds& ids, StageRegs& sreg) {
    const uint64_t row_off =
        small_bs ? 0 : static_cast<uint64_t>((jt * kKT) & (bs - 1)) * static_cast<uint64_t>(slot_stride) * 2u;
#pragma unroll
    for (int i = 0; i < PG::kSRegs; ++i) {
      const uint64_t off = static_cast<uint64_t>(static_cast<uint32_t>(ids[i])) * static_cast<uint64_t>(blk_bytes) + (st_off[i] + row_off);
      // Rows past the causal end (a clamped block id: in-bounds, any data)
      // are zeroed for V when stored and masked out of the scores for K.
      sreg[i] = *reinterpret_cast<const uint4*>(stage_pool + off);
    }
  };

  auto store_tile = [&](int jt, const StageRegs& sreg_in) {
    uint16_t* ks = smem + (jt & 1) * PG::kBufElems;
    uint16_t* vt = ks + PG::kKElems;
    if (k_stager) {
      // K rows past the causal end need no zeroing: every tile that holds
      // them takes the causal mask, which replaces their scores.
#pragma unroll
      for (int i = 0; i < PG::kKLoads; ++i)
        *reinterpret_cast<uint4*>(ks + stage_tok(i) * PG::kKPitch + 8 * stage_chunk(i)) = sreg_in[i];
    } else {
      // V rows past the causal end are zeroed (their weights are 0, but stale
      // slots may hold non-finite values). Only the last tile has such rows.
      StageRegs sreg;
#pragma unroll
      for (int i = 0; i < PG::kSRegs; ++i) sreg[i] = sreg_in[i];
      if (jt * kKT + kKT > kv_end) {
        asm volatile("" ::: "memory");  // keep this a branch, not selects on every tile
#pragma unroll
        for (int i = 0; i < PG::kSRegs; ++i)
          if (jt * kKT + stage_tok(i) >= kv_end) sreg[i] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int gi = 0; gi < PG::kVGroups; ++gi) {
        const int c = stage_chunk(GT * gi);
        const int pos = vt_pos(stage_tok(GT * gi));  // GT consecutive positions
        // Transpose GT tokens x 8 dims into 8 dims x GT tokens.
        const uint32_t* a = reinterpret_cast<const uint32_t*>(&sreg[GT * gi + 0]);
        const uint32_t* bq = reinterpret_cast<const uint32_t*>(&sreg[GT * gi + 1]);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int d0 = 8 * c + 2 * k;
          if constexpr (GT == 4) {
            const uint32_t* cq = reinterpret_cast<const uint32_t*>(&sreg[GT * gi + 2]);
            const uint32_t* dq = reinterpret_cast<const uint32_t*>(&sreg[GT * gi + 3]);
            uint2 lo = make_uint2(perm_lo(a[k], bq[k]), perm_lo(cq[k], dq[k]));
            uint2 hi = make_uint2(perm_hi(a[k], bq[k]), perm_hi(cq[k], dq[k]));
            *reinterpret_cast<uint2*>(vt + d0 * PG::kVPitch + pos) = lo;
            *reinterpret_cast<uint2*>(vt + (d0 + 1) * PG::kVPitch + pos) = hi;
          } else {
            *reinterpret_cast<uint32_t*>(vt + d0 * PG::kVPitch + pos) = perm_lo(a[k], bq[k]);
            *reinterpret_cast<uint32_t*>(vt + (d0 + 1) * PG::kVPitch + pos) = perm_hi(a[k], bq[k]);
          }
        }
      }
    }
  };

  // ---- accumulators: O^T blocks (lane: query row n, dims 32*db + 8*(v/4) + 4*h2 + v%4)
  f32x16v o[PG::kDBlocks];
#pragma unroll
  for (int db = 0; db < PG::kDBlocks; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[db][v] = 0.f;
  float m = -INFINITY;  // running max (log2 units); raised only when a tile's weights grow large
  float l = 0.f;        // this half-wave's share of the softmax denominator
  // -m in every element (0 while m = -inf): the score accumulators of a
  // tile start from it, so they hold s - m and the weights are exp2 of them.
  f32x16v negm;
#pragma unroll
  for (int v = 0; v < 16; ++v) negm[v] = 0.f;

  // Per-lane LDS bases: MFMA operand reads then differ only by immediates.
  const int k_lane = n * PG::kKPitch + (D / 2) * h2;   // + (32*tb)*pitch + 8*st
  const int v_lane = n * PG::kVPitch + 8 * h2;         // + (32*db)*pitch + 16*ks

  // Pipeline, two tiles deep: while tile j is multiplied out of LDS buffer
  // j % 2, tile j + 1 sits in registers (its loads were issued an iteration
  // ago) and tile j + 2's loads are in flight into the other register set;
  // block ids run one tile further ahead. The loop is unrolled by two so the
  // two register sets keep fixed registers.
  // Wave priorities: the two waves of a SIMD share its issue slots, and
  // after each tile's barrier they tend to reach the same phase together.
  // A wave in its softmax (VALU) phase drops to priority 0, so the SIMD's
  // other wave issues its MFMAs first and the matrix pipe stays fed while
  // the VALU work fills the gaps (measured about 2% faster on the 16 x 512
  // chunk workload with the GPU warmed up, identical results).
  auto compute_tile = [&](int j) {
    __builtin_amdgcn_s_setprio(1);
    const int buf = j & 1;
    const uint16_t* ks = smem + buf * PG::kBufElems;
    const uint16_t* vt = ks + PG::kKElems;

    // S^T = K · Q^T, one 32-key accumulator block at a time. The K operands
    // are read from LDS kAhead MFMAs ahead of their use, so each read's
    // latency is covered by the MFMAs in between.
    constexpr int kQK = PG::kSBlocks * PG::kKSteps;
    constexpr int kAhead = 4;
    f32x16v s[PG::kSBlocks];
    auto k_operand = [&](int idx) {
      const int tb = idx / PG::kKSteps, st = idx % PG::kKSteps;
      return __builtin_bit_cast(bf16x8v, *reinterpret_cast<const uint4*>(ks + k_lane + 32 * tb * PG::kKPitch + 8 * st));
    };
    bf16x8v kop[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) kop[u] = k_operand(u);
#pragma unroll
    for (int idx = 0; idx < kQK; ++idx) {
      const int tb = idx / PG::kKSteps, st = idx % PG::kKSteps;
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

    __builtin_amdgcn_s_setprio(0);
    // s[] now holds x - m for the tile's keys, in log2 units (x = scaled
    // score). Causal mask where the tile reaches past min_apos.
    const int t0 = j * kKT;
    if (t0 + kKT - 1 > min_apos) {
#pragma unroll
      for (int tb = 0; tb < PG::kSBlocks; ++tb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int t = t0 + 32 * tb + 8 * (v >> 2) + 4 * h2 + (v & 3);
          s[tb][v] = t <= apos ? s[tb][v] : -INFINITY;
        }
    }
    // Weights P = 2^(s[] - shift) as bf16, packed per 16-key MFMA step; the
    // returned tile sum adds the rounded weights (the values the PV product
    // uses) two at a time with v_dot2_f32_bf16.
    bf16x8v p[PG::kPSteps];
    auto weights = [&](float shift) {
      float lt = 0.f;
#pragma unroll
      for (int tb = 0; tb < PG::kSBlocks; ++tb)
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
#pragma unroll
          for (int e = 0; e < 8; ++e) p[2 * tb + hs][e] = static_cast<__bf16>(fast_exp2(s[tb][8 * hs + e] - shift));
          const uint4 w = __builtin_bit_cast(uint4, p[2 * tb + hs]);
          lt = dot2_bf16(w.x, kBf16Ones, lt);
          lt = dot2_bf16(w.y, kBf16Ones, lt);
          lt = dot2_bf16(w.z, kBf16Ones, lt);
          lt = dot2_bf16(w.w, kBf16Ones, lt);
        }
      return lt;
    };
    // Usually the running max stays: the weights are exp2(s[]) as they are,
    // with no max, subtraction or scaling per score. The first tile sets the
    // max, and a tile whose weights grow large (a half-row sum above
    // kSumLimit, so no weight exceeds it) raises it to the true running max,
    // rescaling O and l, before its weights are taken again.
    float lt = 0.f;
    bool exact = j == 0;  // wave-uniform
    if (!exact) {
      lt = weights(0.f);
      exact = __builtin_amdgcn_ballot_w64(!(lt <= kSumLimit)) != 0;
    }
    if (exact) {
      float T = -INFINITY;  // the tile's max of s[] over the row (both half-waves)
#pragma unroll
      for (int tb = 0; tb < PG::kSBlocks; ++tb)
#pragma unroll
        for (int v = 0; v < 16; ++v) T = fmaxf(T, s[tb][v]);
      T = fmaxf(T, __shfl_xor(T, 32));
      const float M = m == -INFINITY ? 0.f : m;    // what the accumulators started from
      const float mn = fmaxf(m, M + T);             // -inf only for a row with no key yet
      const float alpha = m == -INFINITY ? 0.f : fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < PG::kDBlocks; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
      m = mn;
      const float nm = m == -INFINITY ? 0.f : -m;
#pragma unroll
      for (int v = 0; v < 16; ++v) negm[v] = nm;
      lt = weights(m == -INFINITY ? 0.f : m - M);
    }
    l += lt;

    __builtin_amdgcn_s_setprio(1);
    // O^T += V^T · P^T, V operands read kAhead MFMAs ahead.
    constexpr int kPV = PG::kDBlocks * PG::kPSteps;
    auto v_operand = [&](int idx) {
      const int db = idx / PG::kPSteps, k4 = idx % PG::kPSteps;
      return __builtin_bit_cast(bf16x8v, *reinterpret_cast<const uint4*>(vt + v_lane + 32 * db * PG::kVPitch + 16 * k4));
    };
    bf16x8v vop[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) vop[u] = v_operand(u);
#pragma unroll
    for (int idx = 0; idx < kPV; ++idx) {
      const int db = idx / PG::kPSteps, k4 = idx % PG::kPSteps;
      const bf16x8v a = vop[idx % kAhead];
      if (idx + kAhead < kPV) vop[idx % kAhead] = v_operand(idx + kAhead);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[k4], o[db], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
    for (int idx = 0; idx < kPV - kAhead; ++idx) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
  };
  // Look-ahead loads are issued unconditionally (past the last tile they
  // re-read it, a cache hit) so that the count of loads in flight is the same
  // on every path and each wait covers only the data it needs.
  auto iteration = [&](int j, StageRegs& in_flight, const StageRegs& arrived, LoadIds& ids_next) {
    const int ids_after = fetch_ids(min(j + 3, n_tiles - 1));
    load_tile(min(j + 2, n_tiles - 1), ids_next, in_flight);
    compute_tile(j);
    // Unconditional: past the last tile this stores the idle buffer. A
    // conditional store would leave the register set's loads pending on one
    // path into the next iteration, and the compiler would then wait for
    // every load in flight before reusing those registers.
    store_tile(j + 1, arrived);
    spread_ids(ids_after, ids_next);
    __syncthreads();
  };

  auto scale_q = [&]() {
#pragma unroll
    for (int st = 0; st < PG::kKSteps; ++st) {
      const uint32_t w[4] = {qraw[st].x, qraw[st].y, qraw[st].z, qraw[st].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        qf[st][2 * k] = static_cast<__bf16>(__uint_as_float(w[k] << 16) * scale_log2);
        qf[st][2 * k + 1] = static_cast<__bf16>(__uint_as_float(w[k] & 0xFFFF0000u) * scale_log2);
      }
    }
  };

  StageRegs sreg_a, sreg_b;
  LoadIds ids_next;
  // Start-up: the block ids of the first three tiles load together with q,
  // and one wait covers them all, before any K/V load is in flight (the
  // loop's wait counting then never has to treat them as pending). Tiles 0
  // and 1 then load back to back, tile 0 through the register set that the
  // first iteration refills.
  if (n_tiles > 0) {
    const int raw0 = fetch_ids(0);
    const int raw1 = fetch_ids(min(1, n_tiles - 1));
    const int raw2 = fetch_ids(min(2, n_tiles - 1));
    __builtin_amdgcn_s_waitcnt(0);
    scale_q();
    LoadIds ids0, ids1;
    spread_ids(raw0, ids0);
    spread_ids(raw1, ids1);
    spread_ids(raw2, ids_next);
    load_tile(0, ids0, sreg_b);
    load_tile(min(1, n_tiles - 1), ids1, sreg_a);
    store_tile(0, sreg_b);
  } else {
    __builtin_amdgcn_s_waitcnt(0);
    scale_q();
  }
  __syncthreads();
  // Both halves of the pair run unconditionally, so every path into the next
  // iteration has consumed both register sets (the compiler's wait counting
  // merges paths and would otherwise wait for all loads in flight); an odd
  // last tile runs after the loop.
  int j = 0;
  for (; j + 1 < n_tiles; j += 2) {
    iteration(j, sreg_b, sreg_a, ids_next);
    iteration(j + 1, sreg_a, sreg_b, ids_next);
  }
  if (j < n_tiles) iteration(j, sreg_b, sreg_a, ids_next);

  // ---- normalise and store (bf16, round to nearest even)
  const float lt = l + __shfl_xor(l, 32);
  if (!row_valid) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  uint16_t* orow = out + row_off;
#pragma unroll
  for (int db = 0; db < PG::kDBlocks; ++db)
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

// ---------------------------------------------------------------------------
// D = 128: K/V tiles go from the pool straight into LDS with direct loads
// (global_load_lds_dwordx4: each lane's 16 bytes land at the instruction's
// LDS base + 16 x lane), so staging costs no registers, no LDS store
// instructions and no in-register transpose. V keeps the pool's row-major
// order in LDS and the PV product reads it transposed with
// ds_read_b64_tr_b16 (gfx950): within each 16-lane group, lane i receives
// element i % 4 of the 8-byte pieces addressed by lanes i / 4 + 4k,
// k = 0..3, so four lanes pointing at four keys' 4-dim pieces give every
// lane one dim of four keys.
//
// LDS tile layout (K and V alike; 16 KiB each): 16 key groups of 1 KiB, one
// load instruction each. Group G holds keys 4G..4G+3; its 16-byte unit
// u = 4 pc + (key & 3) holds 16-byte chunk pc ^ (G & 3) of that key (dims
// 8 chunk .. 8 chunk + 7). The XOR spreads the 32 keys of a K operand read
// over the banks; V's transposed reads touch 128 contiguous bytes per 16
// lanes either way. A ring of four tile buffers (see the wave groups below).
// Each wave loads key groups 2w and 2w + 1 of K and of V (keys 8w .. 8w + 7,
// always inside one block), so every wave issues four loads per tile with one
// block id, fetched by one scalar load a tile ahead.
namespace dmat {
constexpr int D = 128;
constexpr int kRowBytes = D * 2;                  // one key's K (or V) row
constexpr int kKeysPerLoad = 1024 / kRowBytes;    // keys per load instruction (64 lanes x 16 B)
constexpr int kGroups = kKT / kKeysPerLoad;       // key groups per tile
constexpr int kTileBytes = kKT * kRowBytes;
constexpr int kBufBytes = 2 * kTileBytes;         // K tile, then V tile
constexpr int kBufs = 4;                          // tile t in buffer t % 4
constexpr int kLdsBytes = kBufs * kBufBytes;
constexpr int kLoadsPerTile = 4;                  // per wave: 2 key groups x (K, V)
static_assert(kKeysPerLoad == 4 && kGroups == 2 * kWaves, "two key groups per wave per tile");

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]).
constexpr int WaitVm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int kWaitLgkm0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);
}  // namespace dmat

typedef short i16x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4v lds_i16x4v;

template <int G>
__global__ __launch_bounds__(kThreads, 1) void PrefillDmaKernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const char* __restrict__ kc,
    const char* __restrict__ vc, const int32_t* __restrict__ cu_q_lens,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ seq_lens, int32_t B,
    int32_t Hkv, int32_t max_blocks, int32_t bs_shift, int32_t num_blocks, int32_t n_qtiles,
    int32_t per_xcd, float scale_log2) {
  using namespace dmat;
  constexpr int QP = kRows / G;  // positions per workgroup
  constexpr int kKSteps = D / 16, kDBlocks = D / 32, kSBlocks = kKT / 32, kPSteps = kKT / 16;
  extern __shared__ char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;   // query row within the wave (accumulator column)
  const int h2 = lane >> 5;  // half-wave

  // ---- work item: as in PrefillKernel (kv head outermost, then sequence
  // longest first, then query tile, last first).
  const int wg = blockIdx.x;
  const int item = (wg & 7) * per_xcd + (wg >> 3);
  if (item >= Hkv * n_qtiles * B) return;
  const int g = item / (n_qtiles * B);
  const int rem = item - g * (n_qtiles * B);
  const int tile = n_qtiles - 1 - rem % n_qtiles;
  int b = rem / n_qtiles;
  if (B <= kRankedBatch) {
    __shared__ int s_order[kRankedBatch];
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
    b = __builtin_amdgcn_readfirstlane(s_order[b]);
  }

  const int qbeg = cu_q_lens[b];
  const int nq = cu_q_lens[b + 1] - qbeg;
  const int q0 = tile * QP;
  if (q0 >= nq) return;
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
  // key 4 Gi + (l & 3), chunk (l >> 2) ^ (Gi & 3). Its byte offset inside the
  // key's block is fixed for the kernel (tiles start on multiples of 64
  // tokens and blocks hold at most 32).
  const int32_t* trow = tables + static_cast<int64_t>(b) * max_blocks;
  const uint32_t row_bytes = static_cast<uint32_t>(Hkv) * kRowBytes;
  const uint32_t blk_bytes = static_cast<uint32_t>(bs) * row_bytes;  // < 4 GiB, checked at launch
  uint32_t ld_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int Gi = 2 * w + i;
    const int key = kKeysPerLoad * Gi + (lane & 3);
    ld_off[i] = static_cast<uint32_t>(key & (bs - 1)) * row_bytes + static_cast<uint32_t>(g) * kRowBytes +
                static_cast<uint32_t>(((lane >> 2) ^ (Gi & 3)) * 16);
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
    const uint32_t kd = lds_base + static_cast<uint32_t>(buf * kBufBytes + (2 * w) * 1024);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
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
      char* vd = lds + buf * kBufBytes + kTileBytes + (2 * w) * 1024;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (t * kKT + kKeysPerLoad * (2 * w + i) + (lane & 3) >= kv_end)
          *reinterpret_cast<uint4*>(vd + i * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    }
  };

  // ---- per-lane LDS read addresses (added to a buffer's LDS address).
  // K operand (tb, st): key 32 tb + n, chunk 2 st + h2, at group 8 tb + n / 4:
  // (2 st + h2) ^ s = 4 (st / 2) + ((2 (st % 2) + h2) ^ s) for s < 4, so two
  // bases (st even / odd) plus immediates cover all of them.
  uint32_t k_lane[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
    k_lane[e] = (n >> 2) * 1024 + (n & 3) * 16 + (((2 * e + h2) ^ ((n >> 2) & 3)) * 64);
  // V^T operand (db, k4), read r (0, 1): lane a of 16-lane group gg points at
  // key 16 k4 + 8 r + 4 h2 + a / 4, dims 32 db + 16 (gg & 1) + 4 (a & 3) .. + 3;
  // the key order matches the S^T accumulator rows (element e of a half-wave:
  // key 8 (e / 4) + 4 h2 + e % 4 of the 16-key step).
  uint32_t v_lane[2];
  {
    const int gg = lane >> 4, a = lane & 15;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int sw = 2 * r + h2;  // group 4 k4 + 2 r + h2, so its swizzle is sw
      v_lane[r] = kTileBytes + sw * 1024 + (((2 * (gg & 1) + ((a >> 1) & 1)) ^ sw) * 64) + (a >> 2) * 16 + 8 * (a & 1);
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
      return lds_b128(((st & 1) ? kb1 : kb0) + static_cast<uint32_t>(tb * 8192 + (st >> 1) * 256));
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
      float lt = 0.f;
#pragma unroll
      for (int tb = 0; tb < kSBlocks; ++tb)
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
#pragma unroll
          for (int e = 0; e < 8; ++e) p[2 * tb + hs][e] = static_cast<__bf16>(fast_exp2(s[tb][8 * hs + e] - shift));
          const uint4 wv = __builtin_bit_cast(uint4, p[2 * tb + hs]);
          lt = dot2_bf16(wv.x, kBf16Ones, lt);
          lt = dot2_bf16(wv.y, kBf16Ones, lt);
          lt = dot2_bf16(wv.z, kBf16Ones, lt);
          lt = dot2_bf16(wv.w, kBf16Ones, lt);
        }
      return lt;
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
      const uint32_t imm = static_cast<uint32_t>(k4 * 4096 + db * 256);
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
    __builtin_amdgcn_s_waitcnt(WaitVm(0));  // no load may land in LDS after the workgroup ends
  } else {
    scale_q();
  }

  const float lsum = l + __shfl_xor(l, 32);
  if (!row_valid) return;
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

template <int G>
hipError_t LaunchDma(const PrefillArgs& a, hipStream_t stream) {
  constexpr int QP = kRows / G;
  const int n_qtiles = (a.max_q_len + QP - 1) / QP;
  const int64_t items = PrefillWorkItems(a.Hkv, a.G, a.B, a.max_q_len);
  if (items == 0) return hipSuccess;
  if (items >= (int64_t{1} << 31) - 8) return hipErrorInvalidValue;
  if (static_cast<int64_t>(a.block_size) * a.Hkv * dmat::kRowBytes >= (int64_t{1} << 32)) return hipErrorInvalidValue;
  const int per_xcd = static_cast<int>((items + 7) / 8);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&PrefillDmaKernel<G>), hipFuncAttributeMaxDynamicSharedMemorySize,
      dmat::kLdsBytes);
  if (attr != hipSuccess) return attr;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((PrefillDmaKernel<G>), dim3(per_xcd * 8), dim3(kThreads), dmat::kLdsBytes, stream,
                     static_cast<uint16_t*>(a.out), static_cast<const uint16_t*>(a.q),
                     static_cast<const char*>(a.k_cache), static_cast<const char*>(a.v_cache),
                     a.cu_q_lens, a.block_tables, a.seq_lens, a.B, a.Hkv, a.max_blocks,
                     __builtin_ctz(a.block_size), a.num_blocks, n_qtiles, per_xcd, scale_log2);
  return hipGetLastError();
}

template <int D, int G>
hipError_t LaunchTyped(const PrefillArgs& a, hipStream_t stream) {
  constexpr int QP = kRows / G;
  const int n_qtiles = (a.max_q_len + QP - 1) / QP;
  const int64_t items = PrefillWorkItems(a.Hkv, a.G, a.B, a.max_q_len);
  if (items == 0) return hipSuccess;
  if (items >= (int64_t{1} << 31) - 8) return hipErrorInvalidValue;
  // The kernel forms a block's byte offset in 32 bits.
  if (static_cast<int64_t>(a.block_size) * a.Hkv * D * 2 >= (int64_t{1} << 32)) return hipErrorInvalidValue;
  const int per_xcd = static_cast<int>((items + 7) / 8);
  const size_t lds = 2 * PGeom<D>::kBufElems * sizeof(uint16_t);
  // More than 64 KiB of dynamic LDS: raise the kernel's limit once.
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&PrefillKernel<D, G>), hipFuncAttributeMaxDynamicSharedMemorySize,
      static_cast<int>(lds));
  if (attr != hipSuccess) return attr;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((PrefillKernel<D, G>), dim3(per_xcd * 8), dim3(kThreads), lds, stream,
                     static_cast<uint16_t*>(a.out), static_cast<const uint16_t*>(a.q),
                     static_cast<const uint16_t*>(a.k_cache), static_cast<const uint16_t*>(a.v_cache),
                     a.cu_q_lens, a.block_tables, a.seq_lens, a.B, a.Hkv, a.max_blocks,
                     __builtin_ctz(a.block_size), a.num_blocks, n_qtiles, per_xcd, scale_log2);
  return hipGetLastError();
}

template <int D>
hipError_t DispatchG(const PrefillArgs& a, hipStream_t s) {
  if constexpr (D == dmat::D) {
    switch (a.G) {
      case 1: return LaunchDma<1>(a, s);
      case 2: return LaunchDma<2>(a, s);
      case 4: return LaunchDma<4>(a, s);
      case 8: return LaunchDma<8>(a, s);
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.G) {
      case 1: return LaunchTyped<D, 1>(a, s);
      case 2: return LaunchTyped<D, 2>(a, s);
      case 4: return LaunchTyped<D, 4>(a, s);
      case 8: return LaunchTyped<D, 8>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
}

}  // namespace

hipError_t LaunchPrefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.B == 0 || a.max_q_len == 0) return hipSuccess;
  return a.D == 64 ? DispatchG<64>(a, stream) : DispatchG<128>(a, stream);
}

}  // namespace pa
