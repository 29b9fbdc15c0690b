// Device helpers shared by the indexer kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8idx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kHeads = 32;   // indexer heads
constexpr int kDim = 128;    // indexer head dim (bytes per fp8 row)
constexpr int kQRowBytes = kHeads * kDim;  // 4096 bytes of q per query row

// One v_mfma_f32_16x16x128_f8f6f4 with both operands in fp8 e4m3 (format code 0).
// Passing zero scales selects the unscaled instruction.
// Lane layout (verified on the device): lane l holds row (l % 16) of A and
// column (l % 16) of B, bytes [32 * (l / 16), 32 * (l / 16) + 32) of the K=128
// dimension; the result gives lane l rows 4 * (l / 16) + r, r = 0..3, of
// column l % 16.
__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Cross-lane reduction of four per-lane partial sums P0..P3 over the four
// 16-lane rows of the wave.  On return, lanes of row G (= lane / 16) hold the
// full sum of partial qsel(G) for their lane % 16 column, where
// qsel(0)=0, qsel(1)=2, qsel(2)=1, qsel(3)=3.
// permlane32_swap exchanges the upper half of the first operand with the
// lower half of the second; permlane16_swap exchanges odd rows of the first
// with even rows of the second.
__device__ __forceinline__ float reduce_rows4(float p0, float p1, float p2, float p3) {
  auto s01 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
  float x = __uint_as_float(s01[0]) + __uint_as_float(s01[1]);
  auto s23 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p2), __float_as_uint(p3), false, false);
  float y = __uint_as_float(s23[0]) + __uint_as_float(s23[1]);
  auto sxy = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(sxy[0]) + __uint_as_float(sxy[1]);
}

__device__ __forceinline__ int reduce_rows4_qsel(int lane) {
  const int G = lane >> 4;
  return ((G & 1) << 1) | (G >> 1);
}

// Order-preserving map float32 -> uint32 (radix-sort order): -0.0 is
// canonicalised to +0.0 first so equal floats give equal keys.
__device__ __forceinline__ uint32_t float_to_ordered(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Largest value over each 16-lane row of the wave, in every lane of the row (DPP: quad swaps, then
// the half-row and row mirrors).
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)0, (int)x, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)0, (int)x, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)0, (int)x, 0x141, 0xF, 0xF, false));  // row_half_mirror
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)0, (int)x, 0x140, 0xF, 0xF, false));  // row_mirror
  return x;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Number of set bits of a 64-bit wave mask below this lane.
__device__ __forceinline__ uint32_t mbcnt64(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
  return x;
}

__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Equal split of `total` items over `parts`: part i gets [first, first + count).
__device__ __forceinline__ void split_range(int64_t total, int64_t parts, int64_t i, int64_t& first,
                                            int64_t& count) {
  const int64_t base = total / parts, rem = total - base * parts;
  first = i * base + min(i, rem);
  count = base + (i < rem ? 1 : 0);
}

}  // namespace fp8idx
