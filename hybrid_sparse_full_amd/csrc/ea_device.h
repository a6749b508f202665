// Device-side utilities shared by the kernels of libea.so (gfx950, wave64).
#pragma once

#include "ea_internal.h"

namespace ea {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ inline int lane_id() { return threadIdx.x & 63; }

// Inclusive prefix sum inside a wavefront (64 lanes).
template <typename T>
__device__ inline T wave_inclusive_sum(T v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    T u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

// A value known to be equal on every lane, stated so that it lives in SGPRs.
__device__ inline int64_t uniform64(int64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uint64_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// max / sum of x over lanes l and l ^ 32 (the two half-waves), in registers:
// v_permlane32_swap exchanges the upper half of one copy with the lower half
// of the other, so the two results hold both halves' values on every lane.
__device__ inline float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum / max of a 32-bit value over all 64 lanes, every lane getting the
// result, without LDS: DPP within each 16-lane row (lane ^ 1, lane ^ 2, the
// half-row mirror, the row mirror), then v_permlane16_swap across row pairs
// and v_permlane32_swap across the half-waves.  (The generic wave_sum below
// goes through ds_bpermute, one LDS round trip per step.)
template <int CTRL, typename T>
__device__ inline T dpp_move(T v) {
  return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
template <typename T, typename Op>
__device__ inline T wave_reduce_dpp(T x, Op op) {
  static_assert(sizeof(T) == 4, "32-bit values");
  x = op(x, dpp_move<0xB1>(x));   // quad_perm [1, 0, 3, 2]
  x = op(x, dpp_move<0x4E>(x));   // quad_perm [2, 3, 0, 1]
  x = op(x, dpp_move<0x141>(x));  // row_half_mirror
  x = op(x, dpp_move<0x140>(x));  // row_mirror
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  x = op(__builtin_bit_cast(T, (uint32_t)r[0]), __builtin_bit_cast(T, (uint32_t)r[1]));
  const auto h = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  return op(__builtin_bit_cast(T, (uint32_t)h[0]), __builtin_bit_cast(T, (uint32_t)h[1]));
}
__device__ inline uint32_t wave_sum_u32(uint32_t x) {
  return wave_reduce_dpp(x, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ inline uint32_t wave_max_u32(uint32_t x) {
  return wave_reduce_dpp(x, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ inline float wave_sum_f32(float x) {
  return wave_reduce_dpp(x, [](float a, float b) { return a + b; });
}
__device__ inline float wave_max_f32(float x) {
  return wave_reduce_dpp(x, [](float a, float b) { return fmaxf(a, b); });
}

template <typename T>
__device__ inline T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Block-wide exclusive prefix sum for blocks of NT threads (NT % 64 == 0).
// `smem` needs NT / 64 + 1 elements.  Returns the exclusive prefix of the
// calling thread; *total receives the block sum.  Contains barriers: every
// thread of the block must call it.
template <int NT, typename T>
__device__ inline T block_exclusive_sum(T v, T* smem, T* total) {
  constexpr int NW = NT / 64;
  const int lane = lane_id();
  const int w = threadIdx.x >> 6;
  T inc = wave_inclusive_sum(v);
  if (lane == 63) smem[w] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    T acc = 0;
    for (int i = 0; i < NW; ++i) {
      T t = smem[i];
      smem[i] = acc;
      acc += t;
    }
    smem[NW] = acc;
  }
  __syncthreads();
  T res = smem[w] + inc - v;
  *total = smem[NW];
  __syncthreads();
  return res;
}

// Block-wide exclusive prefix maximum (identity `lo`), same contract as above.
template <int NT, typename T>
__device__ inline T block_exclusive_max(T v, T lo, T* smem) {
  constexpr int NW = NT / 64;
  const int lane = lane_id();
  const int w = threadIdx.x >> 6;
  T inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    T u = __shfl_up(inc, o, 64);
    if (lane >= o) inc = u > inc ? u : inc;
  }
  T exc = __shfl_up(inc, 1, 64);
  if (lane == 0) exc = lo;
  if (lane == 63) smem[w] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    T acc = lo;
    for (int i = 0; i < NW; ++i) {
      T t = smem[i];
      smem[i] = acc;
      acc = t > acc ? t : acc;
    }
  }
  __syncthreads();
  T res = smem[w] > exc ? smem[w] : exc;
  __syncthreads();
  return res;
}

// Largest index p in [0, n) with a[p] <= x, for nondecreasing a with a[0] <= x.
template <typename T>
__device__ inline int upper_index(const T* a, int n, T x) {
  int lo = 0, hi = n;  // a[lo] <= x, answer in [lo, hi)
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid;
    else hi = mid;
  }
  return lo;
}

}  // namespace ea
