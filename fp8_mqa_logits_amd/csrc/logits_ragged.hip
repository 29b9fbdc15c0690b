// Ragged-prefill fp8 MQA logits for gfx950.
//
//   logits[i, j] = sum_h w[i, h] * max(dot(q[i, h, :], kv[j, :]) * kv_scale[j], 0),  ks[i] <= j < ke[i]
//
// (the `fp8_mqa_logits(q, (kv, kv_scales), weights, ks, ke, clean_logits)` call of
// the indexer loop on the bench_mqa_logits_chunking.py page).
//
// Work decomposition
// - Work items are (block of kRows = 4 * WAVES consecutive query rows, slice
//   of the keys); each wave of a workgroup owns 4 of the item's rows, whose
//   q (4 rows x 32 heads x 128 bytes) stays in VGPRs as eight 16x16x128 MFMA
//   A-operands next to the matching weights.  The grid holds only as many
//   workgroups as are resident at once and each loops over items, so the
//   last round is never mostly empty; splits come in multiples of 8 so a
//   workgroup (and its XCD, blocks being dealt to the 8 XCDs round-robin)
//   keeps streaming the same kv slice, which then stays in that XCD's L2.
// - Keys stream through LDS in tiles of 64 keys x 128 bytes (8 KiB, double
//   buffered), loaded with coalesced 16-byte global loads.  Inside a row the
//   16-byte chunks are XOR-swizzled by (key & 7) so that the B-operand reads
//   (lane l: key l % 16, bytes 32 * (l / 16) .. +32) hit distinct banks.
// - Per 16-key fragment a wave issues 8 MFMAs (4 rows x 2 head tiles of 16);
//   each lane then holds 8 heads of one (row, key) score set.  ReLU and the
//   head weights are applied in registers (max + fma per score), the four
//   16-lane rows are combined with permlane32/permlane16 swaps so that every
//   lane ends with one finished (row, key) logit, which is scaled by
//   kv_scale[j] (factored out of the head sum: valid because kv_scale >= 0)
//   and stored.  The per-head scores never leave registers.
// - Tiles outside the union of the workgroup's row windows are skipped.  A
//   tile inside every window of a wave's 4 rows (the common case) stores its
//   logits without masks, at fixed offsets from one per-tile row pointer; only
//   the partially covered edge tiles are masked element by element.

#include "device_common.hpp"
#include "launch.hpp"
#include "mqa_core.hpp"

#include <algorithm>

namespace fp8idx {

constexpr int kTileKeys = 64;

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES, 3) void logits_ragged_kernel(RaggedLogitsArgs a, int splits,
                                                                       int keys_per_split, int items) {
  constexpr int kThreads = 64 * WAVES;
  constexpr int kRows = 4 * WAVES;
  constexpr int kChunks = kTileKeys * (kDim / 16);   // 16-byte chunks per tile
  constexpr int kChunksPerThread = kChunks / kThreads;
  static_assert(kChunks % kThreads == 0, "tile chunks must divide the workgroup");

  __shared__ __attribute__((aligned(16))) uint8_t s_kv[2][kTileKeys * kDim];
  __shared__ float s_scale[2][kTileKeys];
  __shared__ int s_ks[kRows];
  __shared__ int s_ke[kRows];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = a.n;
  const bool clean = a.clean != 0;

  // Persistent loop over (row block, key split) items.  The grid is a
  // multiple of 8 and so is `splits` on large problems, so a workgroup keeps
  // the same split residue, i.e. the same XCD streams the same kv slice.
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int rb = item / splits;
    const int split = item - rb * splits;
    const int row0 = rb * kRows;
    __syncthreads();   // the previous item is done with s_ks/s_ke and the kv tiles

    if (tid < kRows) {
      const int r = row0 + tid;
      int s = 0, e = 0;
      if (r < a.m) {
        e = min(max(a.ke[r], 0), n);
        s = min(max(a.ks[r], 0), e);
      }
      s_ks[tid] = s;
      s_ke[tid] = e;
    }
    __syncthreads();

    int lo = n, hi = 0;
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      const int s = s_ks[i], e = s_ke[i];
      if (e > s) {
        lo = min(lo, s);
        hi = max(hi, e);
      }
    }
    const int split_lo = split * keys_per_split;
    const int split_hi = min(n, split_lo + keys_per_split);
    const int klo = max(lo, split_lo);
    const int khi = min(hi, split_hi);
    int tile_lo = split_lo, tile_end = split_lo;   // computed range [tile_lo, tile_end)
    int ntiles = 0;
    if (klo < khi) {
      tile_lo = max(split_lo, klo & ~(kTileKeys - 1));
      ntiles = (khi - tile_lo + kTileKeys - 1) / kTileKeys;
      tile_end = min(split_hi, tile_lo + ntiles * kTileKeys);
    }
    const int rows_here = min(kRows, a.m - row0);

    if (clean) {
      // -inf over the split's columns that no tile below covers
      const int w0 = tile_lo - split_lo;
      const int w1 = split_hi - tile_end;
      for (int r = 0; r < rows_here; ++r) {
        float* out = a.logits + (int64_t)(row0 + r) * a.ld;
        for (int c = tid; c < w0; c += kThreads) out[split_lo + c] = -INFINITY;
        for (int c = tid; c < w1; c += kThreads) out[tile_end + c] = -INFINITY;
      }
    }
    if (ntiles == 0) continue;

    // q fragments and weights of this wave's 4 rows
    QFrags qf;
#pragma unroll
    for (int qi = 0; qi < 4; ++qi) {
      const int row = row0 + 4 * wave + qi;
      const bool ok = row < a.m;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        qf.a[qi][t] = load_q_frag(a.q, row, ok, t, lane);
        qf.w[qi][t] = load_w4(a.weights, row, ok, t, lane);
      }
    }
    const int my_r = 4 * wave + reduce_rows4_qsel(lane);
    const int my_row = row0 + my_r;
    const bool row_ok = my_row < a.m;
    const int my_ks = s_ks[my_r];
    const int my_ke = s_ke[my_r];
    float* __restrict__ out_row = a.logits + (int64_t)(row_ok ? my_row : 0) * a.ld;
    // Keys every row of this wave keeps: tiles inside [w_lo, w_hi) store unmasked.
    int w_lo = 0, w_hi = 0;
    if (row0 + 4 * wave + 3 < a.m) {
      w_lo = max(max(s_ks[4 * wave], s_ks[4 * wave + 1]), max(s_ks[4 * wave + 2], s_ks[4 * wave + 3]));
      w_hi = min(min(s_ke[4 * wave], s_ke[4 * wave + 1]), min(s_ke[4 * wave + 2], s_ke[4 * wave + 3]));
    }
    w_hi = min(w_hi, tile_end);
    // This lane's two 16-byte B chunks inside a tile: key f * 16 + l % 16, swizzled by key & 7,
    // which is l & 7 for every fragment f.
    const int kl = lane & 15;
    const int boff0 = kl * kDim + (((2 * (lane >> 4)) ^ (kl & 7)) * 16);
    const int boff1 = kl * kDim + (((2 * (lane >> 4) + 1) ^ (kl & 7)) * 16);

    v4i stage[kChunksPerThread];
    float stage_scale = 0.f;
    auto gload = [&](int tile) {
#pragma unroll
      for (int c = 0; c < kChunksPerThread; ++c) {
        const int ci = tid + c * kThreads;
        const int key = ci >> 3;
        const int j = tile + key;
        v4i v = {0, 0, 0, 0};
        if (j < n) v = *reinterpret_cast<const v4i*>(a.kv + (size_t)j * kDim + (ci & 7) * 16);
        stage[c] = v;
      }
      if (tid < kTileKeys) {
        const int j = tile + tid;
        stage_scale = j < n ? a.kv_scale[j] : 0.f;
      }
    };
    auto lstore = [&](int buf) {
#pragma unroll
      for (int c = 0; c < kChunksPerThread; ++c) {
        const int ci = tid + c * kThreads;
        const int key = ci >> 3;
        *reinterpret_cast<v4i*>(&s_kv[buf][key * kDim + (((ci & 7) ^ (key & 7)) * 16)]) = stage[c];
      }
      if (tid < kTileKeys) s_scale[buf][tid] = stage_scale;
    };

    gload(tile_lo);
    for (int it = 0; it < ntiles; ++it) {
      const int buf = it & 1;
      const int tile = tile_lo + it * kTileKeys;
      lstore(buf);
      __syncthreads();
      if (it + 1 < ntiles) gload(tile + kTileKeys);
      const uint8_t* tbase = &s_kv[buf][0];
      if (tile >= w_lo && tile + kTileKeys <= w_hi) {
        // interior tile: every key is inside every row's window
        float* __restrict__ optr = out_row + tile + kl;
#pragma unroll
        for (int f = 0; f < kTileKeys / 16; ++f) {
          const v4i b0 = *reinterpret_cast<const v4i*>(tbase + f * 16 * kDim + boff0);
          const v4i b1 = *reinterpret_cast<const v4i*>(tbase + f * 16 * kDim + boff1);
          const v8i b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
          optr[f * 16] = fragment_logit(qf, b) * s_scale[buf][f * 16 + kl];
        }
      } else {
#pragma unroll
        for (int f = 0; f < kTileKeys / 16; ++f) {
          const int key = f * 16 + kl;
          const v4i b0 = *reinterpret_cast<const v4i*>(tbase + f * 16 * kDim + boff0);
          const v4i b1 = *reinterpret_cast<const v4i*>(tbase + f * 16 * kDim + boff1);
          const v8i b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
          const float v = fragment_logit(qf, b) * s_scale[buf][key];
          const int j = tile + key;
          if (row_ok && j < tile_end) {
            if (j >= my_ks && j < my_ke) {
              out_row[j] = v;
            } else if (clean) {
              out_row[j] = -INFINITY;
            }
          }
        }
      }
    }
  }
}

void query_ragged_occupancy(DeviceInfo& d) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, logits_ragged_kernel<4>, 256, 0) != hipSuccess)
    per_cu = 1;
  d.ragged_wgs_per_cu = per_cu > 0 ? per_cu : 1;
}

hipError_t launch_logits_ragged(const RaggedLogitsArgs& a, const DeviceInfo& dev, hipStream_t s) {
  if (a.m <= 0) return hipSuccess;
  constexpr int kWaves = 4;
  constexpr int kRows = 4 * kWaves;
  const int64_t row_blocks = (a.m + kRows - 1) / kRows;
  // resident workgroups of this kernel on the whole device, rounded to XCDs
  const int per_cu = dev.ragged_wgs_per_cu > 0 ? dev.ragged_wgs_per_cu : 1;
  int64_t resident = (int64_t)(dev.cu_count > 0 ? dev.cu_count : 256) * per_cu;
  if (resident >= 8) resident = resident / 8 * 8;
  // key splits: multiples of 8 (one residue per XCD), doubled until there are
  // about 8 items per resident workgroup, keeping >= 128 keys (2 tiles) per split
  const int64_t max_splits = std::max<int64_t>(1, a.n / 128);
  int64_t splits = std::min<int64_t>(8, max_splits);
  while (splits * 2 <= max_splits && row_blocks * splits < 8 * resident) splits *= 2;
  int64_t kps = (a.n + splits - 1) / splits;
  kps = (kps + kTileKeys - 1) / kTileKeys * kTileKeys;
  splits = (a.n + kps - 1) / kps;
  const int64_t items = row_blocks * splits;
  if (items > 0x7fffffffLL) return hipErrorInvalidValue;
  const int64_t grid = std::min<int64_t>(items, resident);
  hipLaunchKernelGGL(logits_ragged_kernel<kWaves>, dim3((unsigned)grid), dim3(64 * kWaves), 0, s, a,
                     (int)splits, (int)kps, (int)items);
  return hipGetLastError();
}

}  // namespace fp8idx
