// Device helpers shared by the builder's kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dt {

constexpr int WAVE = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// Round to the nearest bf16, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Order-preserving 32-bit key of an fp32 value: a larger value has a larger
// key; -0 and +0 share one key; NaN maps below every number (key 0).
__device__ __forceinline__ uint32_t f32_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_f32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// 64-bit candidate key: value key high, then the complement of the token id,
// so that a larger composite means (value desc, id asc).
__device__ __forceinline__ uint64_t cand_pack(uint32_t key, uint32_t id) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
__device__ __forceinline__ uint32_t cand_key(uint64_t c) { return (uint32_t)(c >> 32); }
__device__ __forceinline__ uint32_t cand_id(uint64_t c) { return 0xFFFFFFFFu - (uint32_t)c; }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor((uint32_t)v, m);
  uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

// Wave-wide max / sum through DPP row shifts (lane 15 of each row gathers its
// row), then the four row results combined in a fixed order; the result is
// the same in every lane.
template <int CTRL>
__device__ __forceinline__ float dpp_row(float identity, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_row<0x111>(-INFINITY, v));  // row_shr:1
  v = fmaxf(v, dpp_row<0x112>(-INFINITY, v));  // row_shr:2
  v = fmaxf(v, dpp_row<0x114>(-INFINITY, v));  // row_shr:4
  v = fmaxf(v, dpp_row<0x118>(-INFINITY, v));  // row_shr:8
  return fmaxf(fmaxf(lane_f(v, 15), lane_f(v, 31)), fmaxf(lane_f(v, 47), lane_f(v, 63)));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_row<0x111>(0.f, v);
  v += dpp_row<0x112>(0.f, v);
  v += dpp_row<0x114>(0.f, v);
  v += dpp_row<0x118>(0.f, v);
  return (lane_f(v, 15) + lane_f(v, 31)) + (lane_f(v, 47) + lane_f(v, 63));
}

// The same reductions over each half of the wave (lanes 0-31, 32-63); every
// lane gets its half's result.  A half's order of operations is that of
// wave_*_dpp when the other half holds the identity.
__device__ __forceinline__ float half_max_dpp(float v) {
  v = fmaxf(v, dpp_row<0x111>(-INFINITY, v));
  v = fmaxf(v, dpp_row<0x112>(-INFINITY, v));
  v = fmaxf(v, dpp_row<0x114>(-INFINITY, v));
  v = fmaxf(v, dpp_row<0x118>(-INFINITY, v));
  const float h0 = fmaxf(lane_f(v, 15), lane_f(v, 31)), h1 = fmaxf(lane_f(v, 47), lane_f(v, 63));
  const float o0 = fmaxf(h0, -INFINITY), o1 = fmaxf(h1, -INFINITY);
  return (threadIdx.x & 32) ? o1 : o0;
}
__device__ __forceinline__ float half_sum_dpp(float v) {
  v += dpp_row<0x111>(0.f, v);
  v += dpp_row<0x112>(0.f, v);
  v += dpp_row<0x114>(0.f, v);
  v += dpp_row<0x118>(0.f, v);
  const float h0 = lane_f(v, 15) + lane_f(v, 31), h1 = lane_f(v, 47) + lane_f(v, 63);
  return (threadIdx.x & 32) ? h1 + 0.f : h0 + 0.f;
}

// Lane l gets lane l - 1's value (lane 0 gets 0).
__device__ __forceinline__ uint32_t dpp_wave_shr1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x138, 0xF, 0xF, false);  // wave_shr:1
}

// Inclusive OR-scan over the lanes of a wave: within each row of 16 by
// doubling shifts, then each row takes the totals of the rows before it.
__device__ __forceinline__ uint32_t wave_or_scan_incl(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15 to rows 1, 3
  v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31 to rows 2, 3
  return v;
}

// Sort one value per lane of a wave in descending order (bitonic network).
__device__ __forceinline__ uint64_t wave_sort_desc_u64(uint64_t v) {
  const int lane = threadIdx.x & 63;
  for (int k = 2; k <= 64; k <<= 1) {
    for (int j = k >> 1; j >= 1; j >>= 1) {
      uint64_t o = shfl_xor_u64(v, j);
      bool lower = (lane & j) == 0;
      bool desc_block = (lane & k) == 0;  // blocks alternate; the last (k = 64) is descending
      bool keep_max = (lower == desc_block);
      v = keep_max ? (o > v ? o : v) : (o < v ? o : v);
    }
  }
  return v;
}

// Block reductions for a 256-thread block; `red` must hold 4 floats.
template <int NT>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < NT / 64; ++i) r = fmaxf(r, red[i]);
  return r;
}
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = 0.f;
  for (int i = 0; i < NT / 64; ++i) r += red[i];
  return r;
}

// Integer sums over a wave (every lane gets it) and over a 256-thread block
// (`red` holds 4 ints; every thread must call it).
__device__ __forceinline__ int wave_reduce_add(int v) {
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}
__device__ __forceinline__ int block_reduce_add(int v, int* red) {
  v = wave_reduce_add(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// Suffix sums over the threads of a block in thread order:
// returns sum of v over threads with a larger index (exclusive).
template <int NT>
__device__ __forceinline__ int block_suffix_excl(int v, int* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_down(x, d);
    if (lane + d < 64) x += y;
  }
  __syncthreads();
  if (lane == 0) red[w] = x;  // wave total
  __syncthreads();
  int above = 0;
  for (int i = w + 1; i < NT / 64; ++i) above += red[i];
  return x - v + above;
}

// Exclusive prefix over the threads of a block of a 0/1 flag, in thread
// order; also returns the block total.  `red` must hold NT/64 ints.
template <int NT>
__device__ __forceinline__ int block_rank_flag(bool f, int* red, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  unsigned long long b = __ballot(f);
  int inwave = __popcll(b & ((1ull << lane) - 1ull));
  __syncthreads();
  if (lane == 0) red[w] = __popcll(b);
  __syncthreads();
  int before = 0, tot = 0;
  for (int i = 0; i < NT / 64; ++i) {
    if (i < w) before += red[i];
    tot += red[i];
  }
  *total = tot;
  return before + inwave;
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

}  // namespace dt
