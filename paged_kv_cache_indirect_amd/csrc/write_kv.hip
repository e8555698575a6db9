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
