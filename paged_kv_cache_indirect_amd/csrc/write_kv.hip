// KV append scatter ("reshape and cache"): row t of key/value goes to slot
// slot_mapping[t] of the paged pools.
//
// Paging turns the append of a new token into a constant-cost write of one
// row into its page ("LLM推理优化：技术原理解析总览", dpshk.com, §2.2). The pool
// layout [num_blocks, block_size, Hkv, D] makes slot s a contiguous row of
// Hkv·D elements at s·row_bytes, so the scatter is a row copy.
//
// HBM-bound (read T rows, write T rows, twice: K and V). One thread moves one
// 16-byte chunk of K and the same chunk of V; consecutive threads cover
// consecutive chunks of a row, so both reads and writes are fully coalesced.
#include "device_common.h"
#include "launch.h"

#include <algorithm>

namespace pa {

__global__ __launch_bounds__(256) void WriteKvKernel(const uint4* __restrict__ key,
                                                     const uint4* __restrict__ value,
                                                     const int64_t* __restrict__ slots,
                                                     uint4* __restrict__ kc, uint4* __restrict__ vc,
                                                     int64_t total_chunks, int64_t chunks_per_row,
                                                     int64_t num_slots) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total_chunks) return;
  const int64_t t = idx / chunks_per_row;
  const int64_t c = idx - t * chunks_per_row;
  const int64_t s = slots[t];
  if (s < 0 || s >= num_slots) return;  // padding / out of range: skipped
  const int64_t dst = s * chunks_per_row + c;
  kc[dst] = key[idx];
  vc[dst] = value[idx];
}

// Copy-on-write of shared blocks: for each pair p of the list, block
// src[p] of both pools to block dst[p] (block_bytes each, a multiple of 16).
// The pairs of one launch run concurrently, so the host puts a pair whose
// blocks an earlier pair of the list writes or reads (a chain a->b, b->c)
// into a later launch. blockIdx.y picks the pair.
__global__ __launch_bounds__(256) void CopyBlocksKernel(uint4* __restrict__ kc, uint4* __restrict__ vc,
                                                        BlockCopyList list, int64_t chunks) {
  const int64_t src = list.src[blockIdx.y], dst = list.dst[blockIdx.y];
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < chunks;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    kc[dst * chunks + i] = kc[src * chunks + i];
    vc[dst * chunks + i] = vc[src * chunks + i];
  }
}

hipError_t LaunchCopyBlocks(void* k_cache, void* v_cache, const BlockCopyList& list, int64_t block_bytes,
                            hipStream_t stream) {
  if (list.n <= 0) return hipSuccess;
  const int64_t chunks = block_bytes / 16;
  const int64_t blocks = std::min<int64_t>((chunks + 255) / 256, 64);
  hipLaunchKernelGGL(CopyBlocksKernel, dim3(static_cast<uint32_t>(blocks), static_cast<uint32_t>(list.n)),
                     dim3(256), 0, stream, static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), list,
                     chunks);
  return hipGetLastError();
}

// FP8 scatter: one thread quantises 16 elements (two 16-byte bf16 chunks of
// the input row) into one 16-byte chunk of E4M3 codes, for K and for V.
// Per element: fp32 quotient x / scale (IEEE division, round to nearest
// even), clamp to ±448, then the hardware conversion (round to nearest even).
// A NaN quotient is not clamped (fmaxf would return the bound): its code is
// the E4M3 NaN, 0x7F with the input's sign bit.
__device__ __forceinline__ float clamp_e4m3(float q) {
  return q != q ? q : fminf(fmaxf(q, -448.f), 448.f);
}

__device__ __forceinline__ uint32_t quantize4_e4m3(uint32_t w0, uint32_t w1, float scale) {
  const float x0 = __uint_as_float(w0 << 16), x1 = __uint_as_float(w0 & 0xFFFF0000u);
  const float x2 = __uint_as_float(w1 << 16), x3 = __uint_as_float(w1 & 0xFFFF0000u);
  const float q0 = clamp_e4m3(x0 / scale);
  const float q1 = clamp_e4m3(x1 / scale);
  const float q2 = clamp_e4m3(x2 / scale);
  const float q3 = clamp_e4m3(x3 / scale);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);  // bytes 0, 1
  r = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, r, true);        // bytes 2, 3
  uint32_t codes = static_cast<uint32_t>(r);
  const uint32_t nan_bytes = (q0 != q0 ? 0x000000FFu : 0u) | (q1 != q1 ? 0x0000FF00u : 0u) |
                             (q2 != q2 ? 0x00FF0000u : 0u) | (q3 != q3 ? 0xFF000000u : 0u);
  if (nan_bytes) {
    // bf16 sign bits (bits 15 and 31 of each word) become bit 7 of their byte.
    const uint32_t signs = ((w0 >> 8) & 0x80u) | ((w0 >> 16) & 0x8000u) |
                           (((w1 >> 8) & 0x80u) << 16) | (((w1 >> 16) & 0x8000u) << 16);
    codes = (codes & ~nan_bytes) | ((0x7F7F7F7Fu | signs) & nan_bytes);
  }
  return codes;
}

__device__ __forceinline__ uint4 quantize16_e4m3(const uint4& a, const uint4& b, float scale) {
  uint4 o;
  o.x = quantize4_e4m3(a.x, a.y, scale);
  o.y = quantize4_e4m3(a.z, a.w, scale);
  o.z = quantize4_e4m3(b.x, b.y, scale);
  o.w = quantize4_e4m3(b.z, b.w, scale);
  return o;
}

__global__ __launch_bounds__(256) void WriteKvFp8Kernel(const uint4* __restrict__ key,
                                                        const uint4* __restrict__ value,
                                                        const int64_t* __restrict__ slots,
                                                        uint4* __restrict__ kc, uint4* __restrict__ vc,
                                                        int64_t total_chunks, int64_t chunks_per_row,
                                                        int64_t num_slots, float k_scale, float v_scale) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total_chunks) return;
  const int64_t t = idx / chunks_per_row;
  const int64_t c = idx - t * chunks_per_row;
  const int64_t s = slots[t];
  if (s < 0 || s >= num_slots) return;  // padding / out of range: skipped
  const int64_t dst = s * chunks_per_row + c;
  kc[dst] = quantize16_e4m3(key[2 * idx], key[2 * idx + 1], k_scale);
  vc[dst] = quantize16_e4m3(value[2 * idx], value[2 * idx + 1], v_scale);
}

hipError_t LaunchWriteKvFp8(const void* key, const void* value, const int64_t* slots, void* k_cache,
                            void* v_cache, int32_t T, int64_t row_elems, int64_t num_slots, float k_scale,
                            float v_scale, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const int64_t cpr = row_elems / 16;
  const int64_t total = static_cast<int64_t>(T) * cpr;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(WriteKvFp8Kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                     static_cast<const uint4*>(key), static_cast<const uint4*>(value), slots,
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), total, cpr, num_slots,
                     k_scale, v_scale);
  return hipGetLastError();
}

hipError_t LaunchWriteKv(const void* key, const void* value, const int64_t* slots, void* k_cache,
                         void* v_cache, int32_t T, int64_t row_bytes, int64_t num_slots,
                         hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const int64_t cpr = row_bytes / 16;
  const int64_t total = static_cast<int64_t>(T) * cpr;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(WriteKvKernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                     static_cast<const uint4*>(key), static_cast<const uint4*>(value), slots,
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), total, cpr,
                     num_slots);
  return hipGetLastError();
}

}  // namespace pa
