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
//  * One workgroup = 4 waves = 128 query rows of one (sequence, kv head): the
//    G q heads that share the kv head are packed into the row dimension
//    (128 / G positions x G heads), so every K/V tile staged in LDS feeds
//    all of them.
//  * The contraction runs on v_mfma_f32_32x32x16_bf16 in transposed form:
//    S^T = K · Q^T and O^T = V^T · P^T. In the accumulator layout a lane then
//    owns one query row (lane % 32) and 16 keys (or 16 dims) of it, so the
//    online softmax is lane-local except one max exchange between the two
//    half-waves per KV tile, and P goes from the S^T accumulators straight
//    into the B operand of the second product with no data movement: the key
//    order inside each 16-key step is permuted consistently on both sides
//    (V^T is written to LDS in that permuted order).
//  * KV tiles of 64 tokens: K as [token][dim], V transposed to [dim][token]
//    (the transpose is done in registers with v_perm before the LDS write),
//    double-buffered; the next tile's global loads are in flight while the
//    current one is multiplied. Tokens past the causal end of the workgroup
//    are staged as zeros (stale slots of the last block may hold anything).
//  * Online softmax in base 2 with a lazily updated running max: the max is
//    only raised when a tile's max exceeds it by more than 8, so most tiles
//    skip the O rescale; weights stay ≤ 2^8, exact up to rounding.
//  * Causal mask only on tiles that reach past the smallest position of the
//    workgroup. Work items are mapped XCD-major with the kv head outermost,
//    so all query tiles of one (sequence, kv head) share one XCD's L2.
#include "device_common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 128;   // query rows (positions x heads) per workgroup
constexpr int kKT = 64;      // KV tokens per tile
constexpr float kLazyMax = 8.f;

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef float f32x16v __attribute__((ext_vector_type(16)));

template <int D>
struct PGeom {
  static constexpr int kKSteps = D / 16;      // MFMA k-steps for S^T = K Q^T
  static constexpr int kDBlocks = D / 32;     // 32-dim output blocks
  static constexpr int kChunks = D / 8;       // 16-byte chunks per K/V row
  static constexpr int kKPitch = D;           // K tile row pitch (elements)
  static constexpr int kVPitch = kKT;         // V^T tile row pitch (elements)
  static constexpr int kKElems = kKT * kKPitch;
  static constexpr int kVElems = D * kVPitch;
  static constexpr int kBufElems = kKElems + kVElems;
  static constexpr int kKLoads = kKT * kChunks / kThreads;   // 16-byte K chunks per thread
  static constexpr int kVPairs = (kKT / 4) * kChunks;        // (4-token group, chunk) pairs
};

// Position of key t (0..63) inside a V^T row: within each 16-key MFMA step,
// half-wave h takes keys {4h..4h+3, 8+4h..8+4h+3}, which are the keys its
// S^T accumulators hold; they are stored contiguously so one 16-byte read
// fetches them.
__device__ __forceinline__ int vt_pos(int t) {
  const int blk = t >> 5, w = t & 31, s = w >> 4, w16 = w & 15;
  const int h = (w16 >> 2) & 1, e = ((w16 >> 3) << 2) | (w16 & 3);
  return (blk << 5) | (s << 4) | (h << 3) | e;
}

// LDS tiles are unpadded (two K + V^T tiles fit in 64 KB); 16-byte slots are
// XOR-swizzled per row instead, so that the MFMA operand reads (32 rows at one
// column) and the staging writes spread over all 64 banks.
// V^T rows: 8 slots of 8 keys.
__device__ __forceinline__ int vt_swz(int d, int pos) {
  return (((pos >> 3) ^ (((d >> 1) ^ (d >> 4)) & 7)) << 3) | (pos & 7);
}
// K rows: D / 8 slots of 8 dims.
template <int D>
__device__ __forceinline__ int k_swz(int row, int col) {
  const int f = D == 128 ? (row & 15) : ((row >> 1) & 7);
  return (((col >> 3) ^ f) << 3) | (col & 7);
}

__device__ __forceinline__ uint32_t perm_lo(uint32_t x, uint32_t y) {  // (x.lo, y.lo)
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t x, uint32_t y) {  // (x.hi, y.hi)
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

template <int D, int G>
__global__ __launch_bounds__(kThreads, 2) void PrefillKernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ cu_q_lens,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ seq_lens, int32_t B,
    int32_t Hkv, int32_t max_blocks, int32_t bs, int32_t num_blocks, int32_t n_qtiles,
    int32_t per_xcd, float scale_log2) {
  using PG = PGeom<D>;
  constexpr int QP = kRows / G;  // positions per workgroup
  extern __shared__ uint16_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 31;   // query row within the wave (accumulator column)
  const int h2 = lane >> 5;  // half-wave

  // ---- work item: kv head outermost, then query tile (last first), then sequence
  const int wg = blockIdx.x;
  const int item = (wg & 7) * per_xcd + (wg >> 3);
  if (item >= Hkv * n_qtiles * B) return;
  const int g = item / (n_qtiles * B);
  const int rem = item - g * (n_qtiles * B);
  const int tile = n_qtiles - 1 - rem / B;
  const int b = rem % B;

  const int qbeg = cu_q_lens[b];
  const int nq = cu_q_lens[b + 1] - qbeg;
  const int q0 = tile * QP;
  if (q0 >= nq) return;
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

  bf16x8v qf[PG::kKSteps];
#pragma unroll
  for (int s = 0; s < PG::kKSteps; ++s) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row_valid) v = *reinterpret_cast<const uint4*>(q + row_off + (D / 2) * h2 + 8 * s);
    qf[s] = __builtin_bit_cast(bf16x8v, v);
  }

  // Keys the workgroup needs: 0 .. kv_end-1 (the last valid row's position).
  const int kv_end = max(0, ctx + min(q0 + QP, nq));
  const int n_tiles = (kv_end + kKT - 1) / kKT;
  const int min_apos = ctx + q0;

  const int32_t* trow = tables + static_cast<int64_t>(b) * max_blocks;
  const int64_t slot_stride = static_cast<int64_t>(Hkv) * D;
  const uint16_t* kbase = kc + static_cast<int64_t>(g) * D;
  const uint16_t* vbase = vc + static_cast<int64_t>(g) * D;

  // ---- staging: K chunks (token, chunk) and V 4-token groups
  uint4 kreg[PG::kKLoads];
  uint4 vreg[4];
  const bool v_active = tid < PG::kVPairs;
  const int v_c = tid % PG::kChunks;
  const int v_tg = tid / PG::kChunks;

  auto block_of = [&](int t) -> int {
    int blk = trow[t / bs];
    return (static_cast<unsigned>(blk) < static_cast<unsigned>(num_blocks)) ? blk : 0;
  };

  auto load_tile = [&](int j) {
    const int t0 = j * kKT;
#pragma unroll
    for (int i = 0; i < PG::kKLoads; ++i) {
      const int c = tid % PG::kChunks;
      const int t = tid / PG::kChunks + i * (kThreads / PG::kChunks);
      const int tok = t0 + t;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (tok < kv_end) {
        const int64_t slot = static_cast<int64_t>(block_of(tok)) * bs + tok % bs;
        v = *reinterpret_cast<const uint4*>(kbase + slot * slot_stride + 8 * c);
      }
      kreg[i] = v;
    }
    if (v_active) {
      const int tok0 = t0 + 4 * v_tg;
      const int blk = tok0 < kv_end ? block_of(tok0) : 0;  // 4 aligned tokens share a block
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = tok0 + r;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (tok < kv_end) {
          const int64_t slot = static_cast<int64_t>(blk) * bs + tok % bs;
          v = *reinterpret_cast<const uint4*>(vbase + slot * slot_stride + 8 * v_c);
        }
        vreg[r] = v;
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t* ks = smem + buf * PG::kBufElems;
    uint16_t* vt = ks + PG::kKElems;
#pragma unroll
    for (int i = 0; i < PG::kKLoads; ++i) {
      const int c = tid % PG::kChunks;
      const int t = tid / PG::kChunks + i * (kThreads / PG::kChunks);
      *reinterpret_cast<uint4*>(ks + t * PG::kKPitch + k_swz<D>(t, 8 * c)) = kreg[i];
    }
    if (v_active) {
      // Transpose 4 tokens x 8 dims into 8 dims x 4 tokens.
      const uint32_t* a = reinterpret_cast<const uint32_t*>(&vreg[0]);
      const uint32_t* bq = reinterpret_cast<const uint32_t*>(&vreg[1]);
      const uint32_t* cq = reinterpret_cast<const uint32_t*>(&vreg[2]);
      const uint32_t* dq = reinterpret_cast<const uint32_t*>(&vreg[3]);
      const int pos = vt_pos(4 * v_tg);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int d0 = 8 * v_c + 2 * k;
        uint2 lo = make_uint2(perm_lo(a[k], bq[k]), perm_lo(cq[k], dq[k]));
        uint2 hi = make_uint2(perm_hi(a[k], bq[k]), perm_hi(cq[k], dq[k]));
        *reinterpret_cast<uint2*>(vt + d0 * PG::kVPitch + vt_swz(d0, pos)) = lo;
        *reinterpret_cast<uint2*>(vt + (d0 + 1) * PG::kVPitch + vt_swz(d0 + 1, pos)) = hi;
      }
    }
  };

  // ---- accumulators: O^T blocks (lane: query row n, dims 32*db + 8*(v/4) + 4*h2 + v%4)
  f32x16v o[PG::kDBlocks];
#pragma unroll
  for (int db = 0; db < PG::kDBlocks; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[db][v] = 0.f;
  float m = -INFINITY;  // running max (log2 units), lazily raised
  float l = 0.f;        // this half-wave's share of the softmax denominator

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < n_tiles) load_tile(j + 1);

    const uint16_t* ks = smem + buf * PG::kBufElems;
    const uint16_t* vt = ks + PG::kKElems;

    // S^T = K · Q^T for the two 32-key halves of the tile.
    f32x16v s[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[tb][v] = 0.f;
      const int kr = 32 * tb + n;
      const uint16_t* krow = ks + kr * PG::kKPitch;
#pragma unroll
      for (int st = 0; st < PG::kKSteps; ++st) {
        const bf16x8v a = __builtin_bit_cast(
            bf16x8v, *reinterpret_cast<const uint4*>(krow + k_swz<D>(kr, (D / 2) * h2 + 8 * st)));
        s[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[tb], 0, 0, 0);
      }
    }

    // Scores in log2 units; causal mask where the tile reaches past min_apos.
    const int t0 = j * kKT;
    float tmax = -INFINITY;
    if (t0 + kKT - 1 > min_apos) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int t = t0 + 32 * tb + 8 * (v >> 2) + 4 * h2 + (v & 3);
          const float x = s[tb][v] * scale_log2;
          s[tb][v] = t <= apos ? x : -INFINITY;
          tmax = fmaxf(tmax, s[tb][v]);
        }
    } else {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          s[tb][v] *= scale_log2;
          tmax = fmaxf(tmax, s[tb][v]);
        }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));

    // Lazy max: raise m only when the tile exceeds it by more than kLazyMax.
    const bool raise = tmax > m + kLazyMax;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float mn = raise ? tmax : m;
      const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < PG::kDBlocks; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
      m = mn;
    }
    const float msafe = (m == -INFINITY) ? 0.f : m;

    // P = 2^(s - m) as bf16, packed per 16-key MFMA step.
    bf16x8v p[4];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int hs = 0; hs < 2; ++hs)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pe = fast_exp2(s[tb][8 * hs + e] - msafe);
          l += pe;
          p[2 * tb + hs][e] = static_cast<__bf16>(pe);
        }

    // O^T += V^T · P^T.
#pragma unroll
    for (int db = 0; db < PG::kDBlocks; ++db) {
      const int d = 32 * db + n;
      const uint16_t* vrow = vt + d * PG::kVPitch;
#pragma unroll
      for (int ks4 = 0; ks4 < 4; ++ks4) {
        const int pos = 16 * ks4 + 8 * h2;
        const bf16x8v a =
            __builtin_bit_cast(bf16x8v, *reinterpret_cast<const uint4*>(vrow + vt_swz(d, pos)));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[ks4], o[db], 0, 0, 0);
      }
    }

    if (j + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

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

template <int D, int G>
hipError_t LaunchTyped(const PrefillArgs& a, hipStream_t stream) {
  constexpr int QP = kRows / G;
  const int n_qtiles = (a.max_q_len + QP - 1) / QP;
  const int64_t items = static_cast<int64_t>(a.Hkv) * n_qtiles * a.B;
  if (items == 0) return hipSuccess;
  if (items >= (int64_t{1} << 31) - 8) return hipErrorInvalidValue;
  const int per_xcd = static_cast<int>((items + 7) / 8);
  const size_t lds = 2 * PGeom<D>::kBufElems * sizeof(uint16_t);
  const float scale_log2 = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((PrefillKernel<D, G>), dim3(per_xcd * 8), dim3(kThreads), lds, stream,
                     static_cast<uint16_t*>(a.out), static_cast<const uint16_t*>(a.q),
                     static_cast<const uint16_t*>(a.k_cache), static_cast<const uint16_t*>(a.v_cache),
                     a.cu_q_lens, a.block_tables, a.seq_lens, a.B, a.Hkv, a.max_blocks, a.block_size,
                     a.num_blocks, n_qtiles, per_xcd, scale_log2);
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
