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
//  * Decode is a GEMV per head group: every K/V byte is used for G FMAs. It is
//    HBM-bound, so it runs on VALU (no MFMA) and is organised around bytes in
//    flight, not flops.
//  * Pass 1 (PartitionKernel): one workgroup per (sequence, kv head, KV
//    partition of partition_tokens tokens). The G q heads of the group share
//    every K/V row read. 4 waves split the partition into 4 token ranges.
//    Within a wave, 8 lanes cover one 256-byte K/V row with 16-byte loads (8
//    rows per load instruction, each half-row a full 128-byte line), so each
//    load instruction is fully coalesced. The wave's block ids are fetched
//    once (one lane per table entry) and broadcast per 8-row step with
//    v_readlane into SGPRs, keeping the table lookup off the per-row chain.
//  * q·k: v_dot2_f32_bf16 (bf16 pairs, fp32 accumulate) then a 3-step DPP sum
//    over the 8 lanes of a row. Scores (in log2 units) go to LDS; the wave
//    takes the exact max of its range, turns scores into weights
//    2^(s - m) with one exp per (token, head), and sums them.
//  * P·V: fp32 FMAs of the weights into per-lane accumulators, reduced
//    across the wave's row groups (DPP + shuffles), then across the 4 waves
//    with a log-sum-exp rescale through LDS.
//  * A sequence that fits in one partition writes its normalised output
//    directly. Longer ones write fp32 partial states (max, sum, Σ w·V) and
//    pass 2 (MergeKernel) combines them: out = Σ 2^(m_p - M) acc_p /
//    Σ 2^(m_p - M) l_p.
//  * Work items are mapped XCD-major: consecutive hardware workgroup ids go to
//    different XCDs, so item = (wg % 8) * per_xcd + wg / 8 gives each XCD a
//    contiguous run of items ordered (kv head, sequence, partition). With
//    Hkv = 8 each XCD owns one kv head; shared prefix blocks of a head are
//    then re-read from one XCD's L2 instead of eight.
#include "device_common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kLanesPerRow = 8;
constexpr int kRowsPerStep = 64 / kLanesPerRow;  // tokens per wave per load step

template <typename T, int D>
struct RowGeom {
  static constexpr int kElemPerChunk = 16 / static_cast<int>(sizeof(T));
  static constexpr int kChunks = D * static_cast<int>(sizeof(T)) / 16;
  static constexpr int kChunksPerLane = kChunks / kLanesPerRow;  // 1, 2 or 4
  static constexpr int kElemPerLane = kChunksPerLane * kElemPerChunk;
  static_assert(kChunks % kLanesPerRow == 0, "row must split into 8 lanes of 16-byte chunks");
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

// Unpack one 16-byte chunk of V to fp32.
__device__ __forceinline__ void chunk_unpack(const uint4& v, float* o, uint16_t) {
  o[0] = bf16lo(v.x); o[1] = bf16hi(v.x);
  o[2] = bf16lo(v.y); o[3] = bf16hi(v.y);
  o[4] = bf16lo(v.z); o[5] = bf16hi(v.z);
  o[6] = bf16lo(v.w); o[7] = bf16hi(v.w);
}
__device__ __forceinline__ void chunk_unpack(const uint4& v, float* o, float) {
  o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
  o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
}

__device__ __forceinline__ int clamp_block(int blk, int num_blocks) {
  return (static_cast<unsigned>(blk) < static_cast<unsigned>(num_blocks)) ? blk : 0;
}

template <typename T, int D, int G>
__global__ __launch_bounds__(kThreads) void PartitionKernel(
    T* __restrict__ out, const T* __restrict__ q, const T* __restrict__ kc,
    const T* __restrict__ vc, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ seq_lens, float* __restrict__ ws, int32_t B, int32_t Hkv,
    int32_t max_blocks, int32_t bs, int32_t num_blocks, int32_t max_seq_len, int32_t PT,
    int32_t P, int32_t per_xcd, float scale_log2) {
  using RG = RowGeom<T, D>;
  constexpr int CPL = RG::kChunksPerLane;
  constexpr int EPC = RG::kElemPerChunk;
  constexpr int EPL = RG::kElemPerLane;
  extern __shared__ float lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane >> 3;  // row within a load step
  const int j = lane & 7;   // lane within the row

  // XCD-major work mapping.
  const int wg = blockIdx.x;
  const int item = (wg & 7) * per_xcd + (wg >> 3);
  if (item >= P * B * Hkv) return;
  const int p = item % P;
  const int bg = item / P;
  const int b = bg % B;
  const int g = bg / B;

  int L = seq_lens[b];
  L = min(max(L, 0), max_seq_len);
  const int p0 = p * PT;
  if (p > 0 && p0 >= L) return;
  const int p1 = min(p0 + PT, L);
  const int Pb = max(1, (L + PT - 1) / PT);
  const int Hq = Hkv * G;

  const int TPW = PT / kWaves;  // tokens per wave (multiple of 16)
  const int w0 = p0 + w * TPW;
  const int ntok = max(0, min(w0 + TPW, p1) - w0);
  const int nsteps = (ntok + kRowsPerStep - 1) / kRowsPerStep;

  float* s_lds = lds + w * TPW * G;                   // [TPW][G] this wave's scores / weights
  float* m_acc = lds + PT * G;                         // [4][G][D]
  float* m_ml = m_acc + kWaves * G * D;                // [4][G][2]

  // q fragments: this lane's chunks (j, j+8, ...) of the G heads.
  uint4 qf[G][CPL];
  {
    const T* qb = q + (static_cast<int64_t>(b) * Hq + g * G) * D;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < CPL; ++i)
        qf[h][i] = *reinterpret_cast<const uint4*>(qb + h * D + (j + kLanesPerRow * i) * EPC);
  }

  // Block ids of this wave's token range: lane x holds logical block lb0 + x.
  const int lb0 = w0 / bs;
  int my_blk = 0;
  {
    const int nlb = (TPW + bs - 1) / bs + 1;
    const int lb = lb0 + lane;
    if (lane < nlb && lb < max_blocks)
      my_blk = clamp_block(tables[static_cast<int64_t>(b) * max_blocks + lb], num_blocks);
  }

  const int64_t row_stride = static_cast<int64_t>(Hkv) * D;  // elements between slots
  const T* kbase = kc + static_cast<int64_t>(g) * D;
  const T* vbase = vc + static_cast<int64_t>(g) * D;

  // ---------------- pass over K: scores (log2 units) to LDS, running max.
  float mrun[G];
#pragma unroll
  for (int h = 0; h < G; ++h) mrun[h] = -INFINITY;

  constexpr int U = 4;  // load steps in flight per lane
  for (int st0 = 0; st0 < nsteps; st0 += U) {
    uint4 kf[U][CPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int st = st0 + u;
      if (st < nsteps) {
        const int tok = w0 + st * kRowsPerStep;
        const int blk = __builtin_amdgcn_readlane(my_blk, tok / bs - lb0);
        const int64_t slot = static_cast<int64_t>(blk) * bs + (tok % bs) + r;
        const T* row = kbase + slot * row_stride;
#pragma unroll
        for (int i = 0; i < CPL; ++i)
          kf[u][i] = *reinterpret_cast<const uint4*>(row + (j + kLanesPerRow * i) * EPC);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int st = st0 + u;
      if (st < nsteps) {
        const int t = st * kRowsPerStep + r;  // token index within the wave range
        float s[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float a = 0.f;
#pragma unroll
          for (int i = 0; i < CPL; ++i) a = chunk_dot(kf[u][i], qf[h][i], a, T{});
          s[h] = sum8(a);
        }
        const bool valid = t < ntok;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          s[h] = valid ? s[h] * scale_log2 : -INFINITY;
          mrun[h] = fmaxf(mrun[h], s[h]);
        }
        if (j == 0) {
#pragma unroll
          for (int h = 0; h < G; ++h) s_lds[t * G + h] = s[h];
        }
      }
    }
  }

  // Wave max per head; an all-empty range keeps m = -inf and uses 0 as shift.
  float m[G];
#pragma unroll
  for (int h = 0; h < G; ++h) m[h] = max_over_groups8(mrun[h]);

  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // ---------------- weights: one exp per (token, head); lane handles head lane % G.
  float msel = m[0];
#pragma unroll
  for (int h = 1; h < G; ++h) msel = (lane % G == h) ? m[h] : msel;
  const float mshift = (msel == -INFINITY) ? 0.f : msel;
  float lsum = 0.f;
  const int nent = nsteps * kRowsPerStep * G;
  for (int e = lane; e < nent; e += 64) {
    const float pw = fast_exp2(s_lds[e] - mshift);
    s_lds[e] = pw;
    lsum += pw;
  }
#pragma unroll
  for (int x = G; x < 64; x <<= 1) lsum += __shfl_xor(lsum, x);  // lane l: sum of head l % G

  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // ---------------- pass over V: acc[h][e] += w[t][h] * V[t][e].
  float acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;

  for (int st0 = 0; st0 < nsteps; st0 += U) {
    uint4 vf[U][CPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int st = st0 + u;
      if (st < nsteps) {
        const int tok = w0 + st * kRowsPerStep;
        const int blk = __builtin_amdgcn_readlane(my_blk, tok / bs - lb0);
        const int64_t slot = static_cast<int64_t>(blk) * bs + (tok % bs) + r;
        const T* row = vbase + slot * row_stride;
#pragma unroll
        for (int i = 0; i < CPL; ++i)
          vf[u][i] = *reinterpret_cast<const uint4*>(row + (j + kLanesPerRow * i) * EPC);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int st = st0 + u;
      if (st < nsteps) {
        const int t = st * kRowsPerStep + r;
        float pw[G];
#pragma unroll
        for (int h = 0; h < G; ++h) pw[h] = s_lds[t * G + h];
        float v[EPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) chunk_unpack(vf[u][i], v + i * EPC, T{});
        if ((st + 1) * kRowsPerStep > ntok && t >= ntok) {
          // Rows past the sequence end in its last block hold stale data.
#pragma unroll
          for (int e = 0; e < EPL; ++e) v[e] = 0.f;
        }
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pw[h], v[e], acc[h][e]);
      }
    }
  }

  // Reduce the 8 row groups of the wave; lanes 0..7 keep the wave's result.
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = sum_over_groups8(acc[h][e]);

  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < CPL; ++i)
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          m_acc[(w * G + h) * D + (j + kLanesPerRow * i) * EPC + e] = acc[h][i * EPC + e];
  }
  if (lane < G) {
    m_ml[(w * G + lane) * 2 + 0] = msel;  // lane < G: msel = m[lane]
    m_ml[(w * G + lane) * 2 + 1] = lsum;
  }
  __syncthreads();

  // ---------------- merge the 4 waves and write.
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int h = idx / D;
    const int d = idx - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, m_ml[(ww * G + h) * 2]);
    float a = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float mw = m_ml[(ww * G + h) * 2];
        const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
        a = fmaf(f, m_acc[(ww * G + h) * D + d], a);
        l = fmaf(f, m_ml[(ww * G + h) * 2 + 1], l);
      }
    }
    const int hq = g * G + h;
    if (Pb == 1) {
      out[(static_cast<int64_t>(b) * Hq + hq) * D + d] = from_f32<T>(l > 0.f ? a / l : 0.f);
    } else {
      float* st = ws + ((static_cast<int64_t>(b) * Hq + hq) * P + p) * (D + 2);
      st[2 + d] = a;
      if (d == 0) {
        st[0] = M;
        st[1] = l;
      }
    }
  }
}

// Pass 2: log-sum-exp merge of the partitions of each (sequence, q head).
template <typename T, int D>
__global__ __launch_bounds__(D) void MergeKernel(T* __restrict__ out, const float* __restrict__ ws,
                                                 const int32_t* __restrict__ seq_lens, int32_t Hq,
                                                 int32_t max_seq_len, int32_t PT, int32_t P) {
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  const int d = threadIdx.x;
  int L = seq_lens[b];
  L = min(max(L, 0), max_seq_len);
  const int Pb = (L + PT - 1) / PT;
  if (Pb <= 1) return;  // written by pass 1
  const float* st = ws + static_cast<int64_t>(bh) * P * (D + 2);
  float M = -INFINITY;
  for (int p = 0; p < Pb; ++p) M = fmaxf(M, st[p * (D + 2)]);
  float a = 0.f, l = 0.f;
  for (int p = 0; p < Pb; ++p) {
    const float* s = st + p * (D + 2);
    const float f = (s[0] == -INFINITY) ? 0.f : fast_exp2(s[0] - M);
    a = fmaf(f, s[2 + d], a);
    l = fmaf(f, s[1], l);
  }
  out[static_cast<int64_t>(bh) * D + d] = from_f32<T>(l > 0.f ? a / l : 0.f);
}

template <typename T, int D, int G>
hipError_t LaunchTyped(const DecodeArgs& a, hipStream_t stream) {
  const int P = a.num_partitions;
  const int items = P * a.B * a.Hkv;
  const int per_xcd = (items + 7) / 8;
  const size_t lds = (static_cast<size_t>(a.partition_tokens) * G + kWaves * G * D +
                      kWaves * G * 2) * sizeof(float);
  const float scale_log2 = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((PartitionKernel<T, D, G>), dim3(per_xcd * 8), dim3(kThreads), lds, stream,
                     static_cast<T*>(a.out), static_cast<const T*>(a.q),
                     static_cast<const T*>(a.k_cache), static_cast<const T*>(a.v_cache),
                     a.block_tables, a.seq_lens, a.ws, a.B, a.Hkv, a.max_blocks, a.block_size,
                     a.num_blocks, a.max_seq_len, a.partition_tokens, P, per_xcd, scale_log2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || P == 1) return e;
  hipLaunchKernelGGL((MergeKernel<T, D>), dim3(a.B * a.Hq), dim3(D), 0, stream,
                     static_cast<T*>(a.out), a.ws, a.seq_lens, a.Hq, a.max_seq_len,
                     a.partition_tokens, P);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t DispatchG(const DecodeArgs& a, hipStream_t s) {
  switch (a.G) {
    case 1: return LaunchTyped<T, D, 1>(a, s);
    case 2: return LaunchTyped<T, D, 2>(a, s);
    case 4: return LaunchTyped<T, D, 4>(a, s);
    case 8: return LaunchTyped<T, D, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t DispatchD(const DecodeArgs& a, hipStream_t s) {
  return a.D == 64 ? DispatchG<T, 64>(a, s) : DispatchG<T, 128>(a, s);
}

}  // namespace

hipError_t LaunchDecode(const DecodeArgs& a, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  return a.dtype == 0 ? DispatchD<float>(a, stream) : DispatchD<uint16_t>(a, stream);
}

}  // namespace pa
