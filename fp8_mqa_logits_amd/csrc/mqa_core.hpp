// Register-resident q fragments and the per-fragment logit core shared by the
// ragged and paged logits kernels.
#pragma once

#include "device_common.hpp"

namespace fp8idx {

// q of 4 query rows (32 heads x 128 fp8 bytes each) as 16x16x128 MFMA
// A-operands, plus the weights of the heads this lane's accumulator rows hold.
struct QFrags {
  v8i a[4][2];  // [row in wave][head tile]
  v4f w[4][2];  // weights of the 4 heads this lane's accumulator rows hold
};

__device__ __forceinline__ v8i load_q_frag(const uint8_t* __restrict__ q, int row, bool ok, int t, int lane) {
  v8i r = {0, 0, 0, 0, 0, 0, 0, 0};
  if (ok) {
    const v4i* p = reinterpret_cast<const v4i*>(q + (size_t)row * kQRowBytes +
                                                (16 * t + (lane & 15)) * kDim + 32 * (lane >> 4));
    const v4i x = p[0];
    const v4i y = p[1];
    r = v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  }
  return r;
}

__device__ __forceinline__ v4f load_w4(const float* __restrict__ w, int row, bool ok, int t, int lane) {
  v4f r = {0.f, 0.f, 0.f, 0.f};
  if (ok) r = *reinterpret_cast<const v4f*>(w + (size_t)row * kHeads + 16 * t + 4 * (lane >> 4));
  return r;
}

// ReLU as one integer max on the float's bits: a set sign bit makes the
// int32 negative, so negative values (and -0.0) become +0.0 and non-negative
// values pass unchanged.  fmaxf would first canonicalise its input (NaN
// quieting), costing a second VALU op per score.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Scores of the wave's 4 rows against one 16-key B fragment, reduced over heads.
// Returns the unscaled logit of (row qsel(lane), key lane % 16).
__device__ __forceinline__ float fragment_logit(const QFrags& f, const v8i& b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  float p[4];
#pragma unroll
  for (int qi = 0; qi < 4; ++qi) {
    const v4f s0 = mfma_fp8_16x16x128(f.a[qi][0], b, zero);
    const v4f s1 = mfma_fp8_16x16x128(f.a[qi][1], b, zero);
    float acc = f.w[qi][0][0] * relu_bits(s0[0]);
    acc = fmaf(f.w[qi][0][1], relu_bits(s0[1]), acc);
    acc = fmaf(f.w[qi][0][2], relu_bits(s0[2]), acc);
    acc = fmaf(f.w[qi][0][3], relu_bits(s0[3]), acc);
    acc = fmaf(f.w[qi][1][0], relu_bits(s1[0]), acc);
    acc = fmaf(f.w[qi][1][1], relu_bits(s1[1]), acc);
    acc = fmaf(f.w[qi][1][2], relu_bits(s1[2]), acc);
    acc = fmaf(f.w[qi][1][3], relu_bits(s1[3]), acc);
    p[qi] = acc;
  }
  return reduce_rows4(p[0], p[1], p[2], p[3]);
}

}  // namespace fp8idx
