// Wave64 helpers for gfx950 (CDNA4): DPP cross-lane reductions, bf16 <-> fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// DPP control words (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7-i within each 8 lanes
constexpr int kDppRowMirror = 0x140;     // lane i <- lane 15-i within each 16 lanes
constexpr int kDppRowRor8 = 0x128;       // lane i <- lane (i+8) mod 16 within each 16 lanes

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// op(x, x of lane i ^ 16) and op(x, x of lane i ^ 32) for every lane i, with
// gfx950's row swaps (v_permlane16_swap: odd 16-lane rows of one register
// with even rows of the other; v_permlane32_swap: the two 32-lane halves).
// Swapping a value with itself leaves each lane its own value in one result
// and its partner's in the other, so a symmetric op of the two is the
// reduction over the pair. VALU only: no LDS round trip, unlike
// ds_bpermute-based shuffles.
template <typename V, typename Op>
__device__ __forceinline__ V across16(V v, Op op) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return op(__builtin_bit_cast(V, static_cast<uint32_t>(r[0])), __builtin_bit_cast(V, static_cast<uint32_t>(r[1])));
}
template <typename V, typename Op>
__device__ __forceinline__ V across32(V v, Op op) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return op(__builtin_bit_cast(V, static_cast<uint32_t>(r[0])), __builtin_bit_cast(V, static_cast<uint32_t>(r[1])));
}

struct OpAdd {
  template <typename V>
  __device__ __forceinline__ V operator()(V a, V b) const { return a + b; }
};
struct OpMax {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};

// Sum over each aligned group of 8 lanes; every lane of the group gets the sum.
__device__ __forceinline__ float sum8(float v) {
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppRowHalfMirror>(v);
  return v;
}

// Reduction over the whole wave; every lane gets the result. Quad swaps,
// the mirror of each 8 lanes and of each 16 pair every lane with a lane of
// the other half of its 4, 8 and 16 (all of whose lanes hold the same value
// by then), then the row swaps across 16 and 32.
template <typename V, typename Op>
__device__ __forceinline__ V wave_reduce(V v, Op op) {
  v = op(v, dpp<kDppQuadXor1>(v));
  v = op(v, dpp<kDppQuadXor2>(v));
  v = op(v, dpp<kDppRowHalfMirror>(v));
  v = op(v, dpp<kDppRowMirror>(v));
  v = across16(v, op);
  return across32(v, op);
}

// Reductions over lanes that differ in bits 3..5 (the eight 8-lane groups of a
// wave). Lane i ends with the reduction over {i ^ (8k)}.
__device__ __forceinline__ float sum_over_groups8(float v) {
  v += dpp<kDppRowRor8>(v);
  v = across16(v, OpAdd{});
  return across32(v, OpAdd{});
}
__device__ __forceinline__ float max_over_groups8(float v) {
  v = fmaxf(v, dpp<kDppRowRor8>(v));
  v = across16(v, OpMax{});
  return across32(v, OpMax{});
}

__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// a.x*b.x + a.y*b.y + c with bf16 pairs packed in 32-bit words (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa
