// Sparse MLA attention over the indexer's top-k slots, for gfx950 (the sparse
// MLA prefill / decode step that consumes the indexer on the vessl-ai/sglang
// PR #87 page, which keeps the MLA KV pool in fp8 e4m3 and widens it to bf16
// inside the kernel, and runs few-token decode as split-K partials plus a
// combine).
//
//   s[t, h, i] = sm_scale * dot(q[t, h, :], kv_scale[j] * e4m3(kv[j, :]))      j = idx[t, i], 0 <= j < S
//   o[t, h, :] = softmax_i(s[t, h, :]) @ (kv_scale[j] * e4m3(kv[j, :512]))
//   lse[t, h]  = log sum_i exp(s[t, h, i])
//
// Work decomposition
// - A workgroup takes one token, one range of its top-k list (a split) and one
//   block of 64 heads.  Each of its 4 waves owns 16 heads: their q stays in
//   VGPRs as bf16 MFMA operands and their output (16 heads x 512 values, in
//   accumulation registers) with its online-softmax state.  One wave per SIMD
//   leaves each wave the whole register file.  The splits merge in a second
//   kernel.
// - Keys stream through LDS in 64-key steps, double buffered, as fp8 rows
//   (576 bytes per key, 8 bytes of bank skew).  Each thread gathers two
//   16-byte latent chunks of 4 keys and one rotary chunk.  The split's slot ids
//   are read into LDS once, so a gather never waits on an id load; the gather
//   of step i + 2 is in flight while step i is computed.
// - Scores are computed transposed, S^T = K Q^T (16x16x32 bf16 MFMA, fp8
//   widened to bf16 exactly at operand load): a lane then holds 4 consecutive
//   keys of one head, which is exactly the A-operand layout of P in P V, so
//   the probabilities never leave registers.  The value operand comes from the
//   same row-major tile through the LDS transpose read (ds_read_b64_tr_b8):
//   within 16 lanes, lane i < 8 receives byte i of the 8-byte rows that the
//   even lanes address and lane 8 + i byte i of the odd lanes' rows, so lanes
//   2t and 2t + 1 pointing at key t's row (columns c .. c + 7 and c + 8 ..
//   c + 15) hand lane n column c + n of the 8 keys.
// - Softmax works in log2 units; the running maximum is raised (and the
//   output rescaled) only when a step's maximum exceeds it by more than 8,
//   which keeps every weight below 2^8 and skips most rescales.  Powers of 2
//   use the hardware exp2 directly: weights below 2^-126 flush to 0, which
//   is far below what the bf16 probabilities can carry.

#include "device_common.hpp"
#include "launch.hpp"

#include <algorithm>

namespace fp8idx {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kMlaThreads = 256;
constexpr int kMlaHeadsPerWg = 64;
constexpr int kKRow = kMlaDqk + 16;           // LDS bytes per key, row-major (16 bytes of bank skew)
constexpr int kKBytes = kMlaBlock * kKRow;    // 37888
constexpr int kLatChunks = kMlaDv / 128;      // 4 fp8 score chunks of 128 latent values
constexpr int kVTiles = kMlaDv / 16;          // 32 output tiles of 16 values
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;                 // log2 slack before the running maximum moves
constexpr int kMlaMaxSplitKeys = 2048;        // slot ids of one split held in LDS

struct MlaStage {
  uint8_t k[2][kKBytes];
  float mul[2][kMlaBlock];   // sm_scale * log2(e) * kv_scale; NaN marks a masked key
  float vsc[2][kMlaBlock];   // kv_scale; 0 for a masked key
  int32_t idx[kMlaMaxSplitKeys];   // the split's slot ids (-1 past its end)
};

// One step's gather held in registers by one thread.
struct MlaGather {
  v4i lat[4][2];   // two 16-byte latent chunks of each key of the thread's quad
  v4i rot;         // one rotary chunk
  float scale;
  bool ok;
};
// 8 e4m3fn bytes (w0 bytes 0..3, then w1 bytes 0..3) -> 8 bf16, exactly.
__device__ __forceinline__ v8bf fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ v4f mfma_bf16(const v8bf& a, const v8bf& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(kMlaThreads, 1) void sparse_mla_kernel(SparseMlaArgs a, int nsplit,
                                                                    int keys_per_split, float* part_o,
                                                                    float* part_lse) {
  __shared__ __attribute__((aligned(16))) MlaStage sh;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ht = wave;   // head tile of the block
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int t = blockIdx.x / nsplit;
  const int sp = blockIdx.x - t * nsplit;
  const int hb = blockIdx.y;
  const int k_begin = sp * keys_per_split;
  const int k_end = min(a.topk, k_begin + keys_per_split);
  const int nblk = k_end > k_begin ? (k_end - k_begin + kMlaBlock - 1) / kMlaBlock : 0;
  const int32_t* __restrict__ idx_row = a.indices + (int64_t)t * a.ld_idx;

  // ---- q of this wave's head tile, the B operand of S^T.
  // The 512 latent values go to the fp8 MFMA as two e4m3fn parts with a power-of-2 scale per
  // hardware k-block of 32: q 2^e = hi + lo, the block maximum scaled into [128, 256).  hi holds 4
  // significant bits and lo the rest of bf16's 8, so the split is exact for every value above
  // 2^-10 times its block maximum (smaller ones fall under e4m3's subnormal grid and lose bits).
  // In the 16x16x128 fp8 operand, bytes 0-15 of lane group g feed k-block g/2 and bytes 16-31 feed
  // k-block 2 + g/2, and k-block G takes its scale from lane group G: so a block is the same half
  // of lanes l and l ^ 16, and its exponent is moved to lane group G by a shuffle.  The 64 rotary
  // values stay bf16 (two k-steps of 32 values).
  const int head0 = hb * kMlaHeadsPerWg + ht * 16;   // first head of the tile (H is a multiple of 16)
  const bool head_ok = head0 < a.H;
  v8i qh[kLatChunks], ql[kLatChunks];
  int qsc[kLatChunks];   // E8M0 code of 2^-e of k-block g of chunk c
  v8bf qr[2];
  {
    const uint16_t* qrow = a.q + ((int64_t)t * a.H + (head_ok ? head0 + l16 : 0)) * kMlaDqk;
    const int src = l16 + 32 * (g & 1);   // a lane of the first pair holding k-block g
#pragma unroll
    for (int c = 0; c < kLatChunks; ++c) {
      float x[32];
      float amax[2] = {0.f, 0.f};   // of bytes 0-15 and 16-31
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        v4i raw = {0, 0, 0, 0};
        if (head_ok) raw = *reinterpret_cast<const v4i*>(qrow + 128 * c + 32 * g + 8 * v);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          x[8 * v + 2 * w] = __uint_as_float((uint32_t)raw[w] << 16);
          x[8 * v + 2 * w + 1] = __uint_as_float((uint32_t)raw[w] & 0xffff0000u);
          amax[v >> 1] = fmaxf(amax[v >> 1], fmaxf(fabsf(x[8 * v + 2 * w]), fabsf(x[8 * v + 2 * w + 1])));
        }
      }
      int e[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int ex = 0;
        frexpf(fmaxf(amax[h], __shfl_xor(amax[h], 16)), &ex);   // max = m 2^ex, m in [0.5, 1)
        e[h] = min(max(8 - ex, -127), 127);
      }
      const int e_lo = __shfl(e[0], src), e_hi = __shfl(e[1], src);
      qsc[c] = 127 - (g < 2 ? e_lo : e_hi);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ei = e[i >> 2];
        const float y0 = ldexpf(x[4 * i], ei), y1 = ldexpf(x[4 * i + 1], ei);
        const float y2 = ldexpf(x[4 * i + 2], ei), y3 = ldexpf(x[4 * i + 3], ei);
        int hw = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
        hw = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, hw, true);
        const auto d0 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, false);   // the hi values, exactly
        const auto d1 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, true);
        int lw = __builtin_amdgcn_cvt_pk_fp8_f32(y0 - d0[0], y1 - d0[1], 0, false);
        lw = __builtin_amdgcn_cvt_pk_fp8_f32(y2 - d1[0], y3 - d1[1], lw, true);
        qh[c][i] = hw;
        ql[c][i] = lw;
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      v4i raw = {0, 0, 0, 0};
      if (head_ok) raw = *reinterpret_cast<const v4i*>(qrow + kMlaDv + 32 * j + 8 * g);
      qr[j] = __builtin_bit_cast(v8bf, raw);
    }
  }
  // The rotary q goes straight from its load into the step loop's MFMAs.  Without this wait the
  // compiler's wait counter carries that load into the loop, merges it with the key gathers in
  // flight at the loop's back edge, and waits for all of them (vmcnt(0)) in every step's scores.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), before any gather is issued
  // q's fp8 parts are only ever MFMA operands: placing them in accumulation registers frees 64
  // VGPRs, which the score loop uses to load the next key fragment ahead of each MFMA pair.
#pragma unroll
  for (int c = 0; c < kLatChunks; ++c) {
    asm volatile("; q parts to AGPRs" : "+a"(qh[c]), "+a"(ql[c]));
  }

  // ---- staging: this thread's two latent chunks of a key quad, one rotary chunk, one scale
  const int sq = tid >> 4;            // keys 4 sq .. 4 sq + 3 of the step
  const int sc = tid & 15;            // latent chunks sc and sc + 16 (16 values each)
  const int rk = tid >> 2;            // rotary: key rk, chunk 32 + (tid & 3)
  const int rc = 32 + (tid & 3);
  // Every load is unconditional: a masked key (past the range, or an invalid
  // slot) reads slot 0 and is masked by its scale entry.
  auto slot_of = [&](int blk, int key, bool& ok) -> int64_t {
    const int32_t j = sh.idx[blk * kMlaBlock + key];
    ok = j >= 0 && (int64_t)j < a.num_slots;
    return ok ? (int64_t)j : 0;
  };
  auto stage_load = [&](int blk, MlaGather& st) {
    bool ok;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const uint8_t* row = a.kv + slot_of(blk, 4 * sq + q4, ok) * kMlaDqk;
      st.lat[q4][0] = *reinterpret_cast<const v4i*>(row + 16 * sc);
      st.lat[q4][1] = *reinterpret_cast<const v4i*>(row + 16 * (sc + 16));
    }
    st.rot = *reinterpret_cast<const v4i*>(a.kv + slot_of(blk, rk, ok) * kMlaDqk + 16 * rc);
    st.ok = false;
    st.scale = 0.f;
    if (tid < kMlaBlock) {
      const int64_t j = slot_of(blk, tid, st.ok);
      st.scale = a.kv_scale[j];
    }
  };
  auto stage_store = [&](int buf, const MlaGather& st) {
    uint8_t* K = sh.k[buf];
    auto put16 = [](uint8_t* dst, const v4i& v) { *reinterpret_cast<v4i*>(dst) = v; };
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      put16(K + (4 * sq + q4) * kKRow + 16 * sc, st.lat[q4][0]);
      put16(K + (4 * sq + q4) * kKRow + 16 * (sc + 16), st.lat[q4][1]);
    }
    put16(K + rk * kKRow + 16 * rc, st.rot);
    if (tid < kMlaBlock) {
      sh.mul[buf][tid] = st.ok ? a.sm_scale * kLog2e * st.scale : __builtin_nanf("");
      sh.vsc[buf][tid] = st.ok ? st.scale : 0.f;
    }
  };

  // the split's slot ids, padded with -1 to whole steps
  for (int i = tid; i < nblk * kMlaBlock; i += kMlaThreads) {
    const int kk = k_begin + i;
    sh.idx[i] = kk < k_end ? idx_row[kk] : -1;
  }
  __syncthreads();

  // ---- online softmax state (head l16; equal in the 4 lane groups) and output
  float mrun = -INFINITY;
  float lrun = 0.f;   // this lane's share of the denominator
  v4f O[kVTiles];
#pragma unroll
  for (int n = 0; n < kVTiles; ++n) O[n] = v4f{0.f, 0.f, 0.f, 0.f};

  // One step of scores, softmax and value product on LDS buffer cb.
  auto compute = [&](int cb) {
    const uint8_t* K = sh.k[cb];

    // scores S^T: tile kt rows = keys 16 kt + 4 g + r, column = head l16.  Latent chunk c: the key
    // codes straight from LDS (lane: key 16 kt + l16, bytes 128 c + 32 g .. +32) against q's hi and
    // lo parts, scaled by 2^-e; rotary: bf16 MFMAs on the widened codes.
    v4f S[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) S[kt] = v4f{0.f, 0.f, 0.f, 0.f};
    // the key fragment of the next MFMA pair is loaded before this pair is issued
    auto kfrag = [&](int i) -> v8i {
      const v4i* p = reinterpret_cast<const v4i*>(K + (16 * (i & 3) + l16) * kKRow + 128 * (i >> 2) + 32 * g);
      const v4i w0 = p[0], w1 = p[1];
      return v8i{w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
    };
    v8i kf = kfrag(0);
#pragma unroll
    for (int i = 0; i < 4 * kLatChunks; ++i) {
      const int c = i >> 2, kt = i & 3;
      v8i kn = kf;
      if (i + 1 < 4 * kLatChunks) kn = kfrag(i + 1);
      S[kt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, qh[c], S[kt], 0, 0, 0, 127, 0, qsc[c]);
      S[kt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, ql[c], S[kt], 0, 0, 0, 127, 0, qsc[c]);
      kf = kn;
    }
    // rotary: the eight 8-byte key slices load together; each is widened one MFMA ahead
    uint2 rw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      rw[i] = *reinterpret_cast<const uint2*>(K + (16 * (i & 3) + l16) * kKRow + kMlaDv + 32 * (i >> 2) + 8 * g);
    v8bf rb = fp8x8_to_bf16(rw[0].x, rw[0].y);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v8bf rn = rb;
      if (i + 1 < 8) rn = fp8x8_to_bf16(rw[i + 1].x, rw[i + 1].y);
      S[i & 3] = mfma_bf16(rb, qr[i >> 2], S[i & 3]);
      rb = rn;
    }

    // to log2 units, masked keys to -inf; the step's maximum per head
    float bm = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const v4f mul = *reinterpret_cast<const v4f*>(&sh.mul[cb][16 * kt + 4 * g]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = mul[r] != mul[r] ? -INFINITY : S[kt][r] * mul[r];
        S[kt][r] = x;
        bm = fmaxf(bm, x);
      }
    }
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    // lazy rescale: move the running maximum only when this step exceeds it by more than kLazy
    const bool need = bm > mrun + kLazy || (mrun == -INFINITY && bm > -INFINITY);
    if (ballot64(need) != 0ull) {
      const float mnew = need ? bm : mrun;
      const float alpha = mnew == mrun ? 1.f : __builtin_amdgcn_exp2f(mrun - mnew);
      lrun *= alpha;
      mrun = mnew;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * g + r);
#pragma unroll
        for (int n = 0; n < kVTiles; ++n) O[n][r] *= ar;
      }
    }
    // probabilities times kv_scale, as the A operands of P V: key step ks2 holds
    // keys 32 ks2 + 4 g .. +4 (tile 2 ks2) and 32 ks2 + 16 + 4 g .. +4 (tile 2 ks2 + 1)
    v8bf P[2];
    {
      float ps = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const v4f vsc = *reinterpret_cast<const v4f*>(&sh.vsc[cb][16 * kt + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pr = mrun == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(S[kt][r] - mrun);
          ps += pr;
          P[kt >> 1][4 * (kt & 1) + r] = (__bf16)(pr * vsc[r]);
        }
      }
      lrun += ps;
    }
    // O += P V: value tile n, lane column 16 n + l16.  The B operand of key step ks2 holds keys
    // 32 ks2 + 4 g .. +4 and 32 ks2 + 16 + 4 g .. +4 (the order of P's elements); lane pair
    // (2 t, 2 t + 1) of each 16 points at the t-th of those keys' row, columns 16 n and 16 n + 8.
    const int tkey = (l16 >> 1) < 4 ? 4 * g + (l16 >> 1) : 16 + 4 * g + (l16 >> 1) - 4;
    const uint8_t* vrow = K + tkey * kKRow + 8 * (l16 & 1);
    // MFMA i: key step i / 32, value tile i % 32, so consecutive MFMAs update different tiles; the
    // transpose reads run kVAhead MFMAs ahead.
    typedef int v2i_t __attribute__((ext_vector_type(2)));
    auto vfrag = [&](int i) -> v2i_t {
      return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) v2i_t*)(vrow + 32 * (i / kVTiles) * kKRow + 16 * (i % kVTiles)));
    };
    constexpr int kVAhead = 4;
    v2i_t vq[kVAhead];
#pragma unroll
    for (int j = 0; j < kVAhead; ++j) vq[j] = vfrag(j);
    // the widened operand of MFMA i + 1 is formed before MFMA i is issued
    v8bf vb = fp8x8_to_bf16((uint32_t)vq[0][0], (uint32_t)vq[0][1]);
    vq[0] = vfrag(kVAhead);
#pragma unroll
    for (int i = 0; i < 2 * kVTiles; ++i) {
      v8bf vn = vb;
      if (i + 1 < 2 * kVTiles) {
        const v2i_t w = vq[(i + 1) % kVAhead];
        if (i + 1 + kVAhead < 2 * kVTiles) vq[(i + 1) % kVAhead] = vfrag(i + 1 + kVAhead);
        vn = fp8x8_to_bf16((uint32_t)w[0], (uint32_t)w[1]);
      }
      O[i % kVTiles] = mfma_bf16(P[i / kVTiles], vb, O[i % kVTiles]);
      vb = vn;
    }

  };

  // Step i sits in LDS buffer i & 1; the gather of step i + 2 is in flight in
  // registers while step i is computed.
  MlaGather ga;
  if (nblk > 0) {
    stage_load(0, ga);
    stage_store(0, ga);
  }
  if (nblk > 1) stage_load(1, ga);
  __syncthreads();
  for (int blk = 0; blk < nblk; ++blk) {
    if (head_ok) compute(blk & 1);   // a wave past the last head only helps stage the keys
    if (blk + 1 < nblk) stage_store((blk + 1) & 1, ga);
    if (blk + 2 < nblk) stage_load(blk + 2, ga);
    __syncthreads();
  }

  // ---- normalise and store
  lrun += __shfl_xor(lrun, 16);
  lrun += __shfl_xor(lrun, 32);
  if (!head_ok) return;
  const float inv = lrun > 0.f ? 1.f / lrun : 0.f;   // per head l16
  if (g == 0) {
    const float lse = lrun > 0.f ? (mrun + __log2f(lrun)) * kLn2 : -INFINITY;
    const int head = head0 + l16;
    if (nsplit == 1) {
      if (a.lse) a.lse[(int64_t)t * a.H + head] = lse;
    } else {
      part_lse[((int64_t)t * nsplit + sp) * a.H + head] = lse;
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float c = __shfl(inv, 4 * g + r);
    const int head = head0 + 4 * g + r;
    float* dst = nsplit == 1 ? a.out + ((int64_t)t * a.H + head) * kMlaDv
                             : part_o + (((int64_t)t * nsplit + sp) * a.H + head) * kMlaDv;
#pragma unroll
    for (int n = 0; n < kVTiles; ++n) dst[16 * n + l16] = O[n][r] * c;
  }
}

// Merges the splits of each (token, head): weights exp(lse_s - lse), lse = log sum exp(lse_s).
constexpr int kCombineThreads = kMlaDv / 4;   // 128: one float4 of the 512 outputs each
constexpr int kCombineChunk = 256;            // split weights held in LDS at a time

// One workgroup per (token, head): the splits' lse values are read together, their weights
// exp(lse_s - max) kept in LDS (kCombineChunk splits at a time), and the outputs summed over the
// splits in split order with several partial rows in flight.
__global__ __launch_bounds__(kCombineThreads) void sparse_mla_combine_kernel(SparseMlaArgs a, int nsplit,
                                                                           const float* part_o,
                                                                           const float* part_lse) {
  __shared__ float s_w[kCombineChunk];
  __shared__ float s_red[kCombineThreads / 64];
  const int t = blockIdx.x;
  const int head = blockIdx.y;
  const int tid = threadIdx.x;
  const float* lse_th = part_lse + (int64_t)t * nsplit * a.H + head;   // split s at lse_th[s * H]
  float m = -INFINITY;
  for (int s = tid; s < nsplit; s += kCombineThreads) m = fmaxf(m, lse_th[(int64_t)s * a.H]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) s_red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(s_red[0], s_red[1]);
  float z = 0.f;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  const float* po = part_o + ((int64_t)t * nsplit * a.H + head) * kMlaDv + 4 * tid;
  const int64_t stride = (int64_t)a.H * kMlaDv;
  for (int b = 0; b < nsplit; b += kCombineChunk) {
    const int nb = min(kCombineChunk, nsplit - b);
    for (int s = tid; s < nb; s += kCombineThreads) {
      const float ls = lse_th[(int64_t)(b + s) * a.H];
      s_w[s] = (m == -INFINITY || ls == -INFINITY) ? 0.f : __expf(ls - m);
    }
    __syncthreads();
    if (m != -INFINITY) {
#pragma unroll 8
      for (int s = 0; s < nb; ++s) {
        const float w = s_w[s];
        z += w;
        acc += *reinterpret_cast<const v4f*>(po + (int64_t)(b + s) * stride) * w;
      }
    }
    __syncthreads();   // the next chunk rewrites s_w
  }
  const float inv = z > 0.f ? 1.f / z : 0.f;
  *reinterpret_cast<v4f*>(a.out + ((int64_t)t * a.H + head) * kMlaDv + 4 * tid) = acc * inv;
  if (tid == 0 && a.lse) a.lse[(int64_t)t * a.H + head] = z > 0.f ? m + __logf(z) : -INFINITY;
}

// Splits each top-k list so that about kMlaTargetWgs workgroups run (one per
// CU of the 256-CU part), never below one 64-key step and never above the
// 2048 slot ids a workgroup holds in LDS.  A pure function of the shape, so
// the workspace size needs no device.
constexpr int64_t kMlaTargetWgs = 256;

SparseMlaPlan plan_sparse_mla(int32_t T, int32_t H, int32_t topk) {
  SparseMlaPlan p{};
  const int64_t blocks = std::max<int64_t>(1, ((int64_t)topk + kMlaBlock - 1) / kMlaBlock);
  const int64_t groups = std::max<int64_t>(1, (int64_t)T * ((H + kMlaHeadsPerWg - 1) / kMlaHeadsPerWg));
  int64_t nsplit = std::min<int64_t>(blocks, std::max<int64_t>(1, (kMlaTargetWgs + groups - 1) / groups));
  const int64_t blocks_per_split =
      std::min<int64_t>((blocks + nsplit - 1) / nsplit, kMlaMaxSplitKeys / kMlaBlock);
  nsplit = (blocks + blocks_per_split - 1) / blocks_per_split;
  p.nsplit = (int32_t)nsplit;
  p.keys_per_split = (int32_t)(blocks_per_split * kMlaBlock);
  p.ws_bytes = nsplit > 1 ? (size_t)T * (size_t)nsplit * (size_t)H * (kMlaDv + 1) * sizeof(float) + 256 : 0;
  return p;
}

hipError_t launch_sparse_mla(const SparseMlaArgs& a, const SparseMlaPlan& plan, void* ws, hipStream_t s) {
  if (a.T <= 0 || a.H <= 0) return hipSuccess;
  float* part_o = nullptr;
  float* part_lse = nullptr;
  if (plan.nsplit > 1) {
    part_o = static_cast<float*>(ws);
    part_lse = part_o + (size_t)a.T * plan.nsplit * a.H * kMlaDv;
  }
  const int64_t gx = (int64_t)a.T * plan.nsplit;
  const int gy = (a.H + kMlaHeadsPerWg - 1) / kMlaHeadsPerWg;
  if (gx > 0x7fffffffLL || gy > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sparse_mla_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(kMlaThreads), 0, s, a, plan.nsplit,
                     plan.keys_per_split, part_o, part_lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.nsplit == 1) return e;
  hipLaunchKernelGGL(sparse_mla_combine_kernel, dim3((unsigned)a.T, (unsigned)a.H), dim3(kCombineThreads), 0, s, a,
                     plan.nsplit, part_o, part_lse);
  return hipGetLastError();
}

}  // namespace fp8idx
