// Per-row fp8 e4m3fn quantisation for gfx950: the step that produces the
// indexer's fp8 inputs (kv codes with per-token kv_scale, q codes), named
// `act_quant` on the vessl-ai/sglang PR #87 page, whose encoder test pins
// nearest-even rounding, subnormals and saturation to +-448.
//
//   amax  = max_d |x[r, d]|   (a row of zeros takes amax = 448)
//   y     = x[r, d] * (448 / amax)          float32 division, float32 multiply
//   codes[r, d] = e4m3fn(y)                 nearest, ties to even, saturating
//   scale[r]    = amax / 448                so x ~ decode(code) * scale
//
// HBM work: 4 bytes read and 1 byte written per element, plus 4 bytes of
// scale per row.  Rows of up to 256 floats (D / 4 a power of two) pack
// several rows into a wave, with several row groups in flight per wave;
// longer rows take one wave per row.  Each lane loads its 16-byte vectors of
// the row once, the row maximum is a reduction over the row's lanes, and the codes are
// formed with the hardware pack-convert (v_cvt_pk_fp8_f32, OCP e4m3fn on
// gfx950) after clamping y to [-448, 448], so no conversion ever sees a
// value past the largest finite code.  Codes leave as 4-byte stores.

#include "device_common.hpp"
#include "launch.hpp"

namespace fp8idx {

constexpr int kQuantWaves = 4;
constexpr int kQuantMaxVec = 8;   // 16-byte vectors per lane: rows of up to 64 * 8 * 4 = 2048 floats

template <int NV>
__global__ __launch_bounds__(64 * kQuantWaves) void quant_fp8_kernel(QuantArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kQuantWaves + (threadIdx.x >> 6);
  if (row >= a.rows) return;   // no barriers: waves are independent
  const int nvec = a.D / 4;
  const v4f* xr = reinterpret_cast<const v4f*>(a.x + row * a.ld_x);
  v4f v[NV];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = lane + 64 * i;
    v[i] = v4f{0.f, 0.f, 0.f, 0.f};
    if (idx < nvec) v[i] = __builtin_nontemporal_load(xr + idx);
#pragma unroll
    for (int c = 0; c < 4; ++c) amax = fmaxf(amax, fabsf(v[i][c]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if (!(amax > 0.f)) amax = 448.f;
  const float inv = 448.f / amax;
  uint32_t* cr = reinterpret_cast<uint32_t*>(a.codes + row * a.ld_codes);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = lane + 64 * i;
    if (idx < nvec) {
      float y[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) y[c] = fminf(fmaxf(v[i][c] * inv, -448.f), 448.f);
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
      cr[idx] = (uint32_t)w;
    }
  }
  if (lane == 0) a.scale[row] = amax / 448.f;
}

// Rows of D = 4 * LPR floats (LPR a power of two <= 64): each lane holds one
// 16-byte vector of a row, a wave holds 64 / LPR rows at once, and it loads
// kIter such row groups before converting any, so several loads are in flight
// per wave.  The row maximum is a reduction within the row's LPR lanes.
constexpr int kIter = 4;

template <int LPR>
__global__ __launch_bounds__(64 * kQuantWaves) void quant_fp8_small_kernel(QuantArgs a) {
  constexpr int kRowsPerWave = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR;   // row of the group
  const int col = lane % LPR;   // vector of the row
  const int64_t wave_row0 = ((int64_t)blockIdx.x * kQuantWaves + (threadIdx.x >> 6)) * (kRowsPerWave * kIter);
  v4f v[kIter];
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    const int64_t row = wave_row0 + it * kRowsPerWave + sub;
    v[it] = v4f{0.f, 0.f, 0.f, 0.f};
    if (row < a.rows) v[it] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(a.x + row * a.ld_x) + col);
  }
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    const int64_t row = wave_row0 + it * kRowsPerWave + sub;
    float amax = fmaxf(fmaxf(fabsf(v[it][0]), fabsf(v[it][1])), fmaxf(fabsf(v[it][2]), fabsf(v[it][3])));
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if (!(amax > 0.f)) amax = 448.f;
    const float inv = 448.f / amax;
    float y[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) y[c] = fminf(fmaxf(v[it][c] * inv, -448.f), 448.f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
    if (row < a.rows) {
      reinterpret_cast<uint32_t*>(a.codes + row * a.ld_codes)[col] = (uint32_t)w;
      if (col == 0) a.scale[row] = amax / 448.f;
    }
  }
}

template <int LPR>
static void launch_small(const QuantArgs& a, hipStream_t s) {
  constexpr int64_t kRowsPerBlock = (int64_t)kQuantWaves * (64 / LPR) * kIter;
  const int64_t blocks = (a.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(quant_fp8_small_kernel<LPR>, dim3((unsigned)blocks), dim3(64 * kQuantWaves), 0, s, a);
}

hipError_t launch_quant_fp8(const QuantArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  const int64_t blocks = (a.rows + kQuantWaves - 1) / kQuantWaves;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  switch (a.D) {
    case 4: launch_small<1>(a, s); return hipGetLastError();
    case 8: launch_small<2>(a, s); return hipGetLastError();
    case 16: launch_small<4>(a, s); return hipGetLastError();
    case 32: launch_small<8>(a, s); return hipGetLastError();
    case 64: launch_small<16>(a, s); return hipGetLastError();
    case 128: launch_small<32>(a, s); return hipGetLastError();
    case 256: launch_small<64>(a, s); return hipGetLastError();
    default: break;
  }
  const int nv = (a.D / 4 + 63) / 64;
  const dim3 grid((unsigned)blocks), block(64 * kQuantWaves);
  switch (nv) {
    case 1: hipLaunchKernelGGL(quant_fp8_kernel<1>, grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL(quant_fp8_kernel<2>, grid, block, 0, s, a); break;
    case 3:
    case 4: hipLaunchKernelGGL(quant_fp8_kernel<4>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(quant_fp8_kernel<kQuantMaxVec>, grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace fp8idx
