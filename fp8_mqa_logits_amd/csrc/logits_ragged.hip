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
//   A-operands next to the matching weights.
// - The grid is persistent: as many workgroups as are resident at once.  The
//   items sit in 8 queues, one per XCD: queue x holds the key slices x, x + 8,
//   x + 16, ... of every row block, row blocks from the last (the longest
//   causal windows) to the first.  Workgroups are dealt to the XCDs
//   round-robin, so queue blockIdx % 8 is served by one XCD and its kv slices
//   stay in that XCD's L2.  A workgroup's first item is fixed (item
//   blockIdx / 8 of its queue); after that it claims items with one atomic
//   per item on its queue's counter, and once that queue is empty it moves to
//   another queue that still has items.  Co-resident workgroups are not
//   served at equal rates (issue favours older waves), so dynamic claims
//   balance the finish times where any static split leaves the slowest
//   workgroup of each CU last.
// - The counters (8 words) live in a buffer that the caller's workspace
//   brings in, one per launch.  The launcher clears them with a one-wave
//   kernel on the same stream right before the logits kernel, so a launch
//   never depends on what an earlier one left there; when the fixed first
//   items cover every queue (small problems) neither the clear nor any
//   atomic runs.  Two launches that may run at the same time must therefore
//   be given different counter buffers.
// - Keys stream through LDS in tiles of 128 keys x 128 bytes (16 KiB, double
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
#include <mutex>

namespace fp8idx {

constexpr int kTileKeys = 128;
constexpr int kWaves = 4;
constexpr int kRowsPerItem = 4 * kWaves;

// Tiles of one item: row block with key window union [lo, hi), split [split_lo, split_hi).
struct ItemGeom {
  int tile_lo, tile_end, ntiles;
};

__device__ __forceinline__ ItemGeom item_geom(int lo, int hi, int split_lo, int split_hi) {
  ItemGeom g{split_lo, split_lo, 0};
  const int klo = max(lo, split_lo), khi = min(hi, split_hi);
  if (klo < khi) {
    g.tile_lo = max(split_lo, klo & ~(kTileKeys - 1));
    g.ntiles = (khi - g.tile_lo + kTileKeys - 1) / kTileKeys;
    g.tile_end = min(split_hi, g.tile_lo + g.ntiles * kTileKeys);
  }
  return g;
}

constexpr unsigned int kNoItem = 0xffffffffu;

// Splits served by queue x: x, x + 8, x + 16, ... below `splits`.
__device__ __forceinline__ int queue_splits(int splits, int x) { return splits > x ? (splits - x + 7) / 8 : 0; }

// Workgroups whose fixed first item comes from queue x (those with blockIdx % 8 == x).
__host__ __device__ __forceinline__ unsigned int queue_fixed(unsigned int grid, int x) {
  return (grid + 7u - (unsigned int)x) / 8u;
}

// Items of queue x.
__host__ __device__ __forceinline__ unsigned int queue_items(int splits, int row_blocks, int x) {
  return (unsigned int)((splits > x ? (splits - x + 7) / 8 : 0) * row_blocks);
}

// True when the fixed first items (one per workgroup) leave some queue with items to claim.
__host__ __device__ __forceinline__ bool queues_needed(unsigned int grid, int splits, int row_blocks) {
  bool need = false;
  for (int x = 0; x < 8; ++x) need = need || queue_items(splits, row_blocks, x) > queue_fixed(grid, x);
  return need;
}

// Next item of a workgroup as (index in queue) * 8 + queue, or kNoItem once every queue is empty.
// `state` (thread 0's own) is 0 before the fixed first item, 1 while the home queue may hold items,
// 2 after it ran out.  Other queues are probed by reading their counters first: counters only
// grow, so one read at or past a queue's end proves that queue empty.  With fixed_only (the fixed
// first items cover every queue) no counter is read or written at all.
__device__ __forceinline__ unsigned int claim_item(unsigned int* queue, int home, int& state, int splits,
                                                   int row_blocks, bool fixed_only) {
  const unsigned int home_items = queue_items(splits, row_blocks, home);
  if (state == 0) {
    state = 1;
    const unsigned int c = blockIdx.x >> 3;
    if (c < home_items) return c * 8u + (unsigned int)home;
  }
  if (fixed_only) return kNoItem;
  if (state == 1) {
    const unsigned int c = atomicAdd(&queue[home], 1u) + queue_fixed(gridDim.x, home);
    if (c < home_items) return c * 8u + (unsigned int)home;
    state = 2;
  }
  for (;;) {
    int pick = -1;
#pragma unroll
    for (int d = 1; d < 8; ++d) {
      const int x = (home + d) & 7;
      const unsigned int taken = __hip_atomic_load(&queue[x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (pick < 0 && taken + queue_fixed(gridDim.x, x) < queue_items(splits, row_blocks, x)) pick = x;
    }
    if (pick < 0) return kNoItem;
    const unsigned int c = atomicAdd(&queue[pick], 1u) + queue_fixed(gridDim.x, pick);
    if (c < queue_items(splits, row_blocks, pick)) return c * 8u + (unsigned int)pick;
  }
}

// Zeroes one launch's work-queue counters (a kernel rather than a memset node, so that the
// pair captures into a graph as two kernel nodes).
__global__ __launch_bounds__(64) void queue_clear_kernel(unsigned int* queue) {
  if (threadIdx.x < kRaggedQueueWords) queue[threadIdx.x] = 0u;
}

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES, 3) void logits_ragged_kernel(RaggedLogitsArgs a, int splits, int kps,
                                                                       int use_queue) {
  constexpr int kThreads = 64 * WAVES;
  constexpr int kRows = 4 * WAVES;
  constexpr int kChunks = kTileKeys * (kDim / 16);   // 16-byte chunks per tile
  constexpr int kChunksPerThread = kChunks / kThreads;
  static_assert(kChunks % kThreads == 0, "tile chunks must divide the workgroup");

  __shared__ __attribute__((aligned(16))) uint8_t s_kv[2][kTileKeys * kDim];
  __shared__ float s_scale[2][kTileKeys];
  __shared__ int s_ks[kRows];
  __shared__ int s_ke[kRows];
  __shared__ unsigned int s_claim;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = a.n;
  const bool clean = a.clean != 0;
  const int row_blocks = (a.m + kRows - 1) / kRows;
  unsigned int* const queue = a.queue;

  // Queue x holds the items of the splits x, x + 8, x + 16, ...: row blocks from the last (the
  // longest causal windows) to the first, each with all of the queue's splits.  Workgroups are
  // dealt to the 8 XCDs round-robin, so queue blockIdx % 8 is served by one XCD, whose L2 keeps
  // those kv slices.  A workgroup's first item is fixed (item blockIdx / 8 of its queue); the
  // counters hand out the rest.  A workgroup whose queue is empty moves on
  // to a queue that is not.
  const int home = blockIdx.x & 7;
  // When the fixed first items cover every queue (the host checks this with the same formula),
  // the counters are not needed at all.
  const bool fixed_only = use_queue == 0;
  int claim_state = 0;
  for (;;) {
    __syncthreads();   // the previous item is done with s_ks/s_ke, the tiles and s_claim
    if (tid == 0) {
      s_claim = claim_item(queue, home, claim_state, splits, row_blocks, fixed_only);
    }
    __syncthreads();
    const unsigned int claim = s_claim;
    if (claim == kNoItem) break;
    const int xq = (int)(claim & 7u);
    const int nsx = queue_splits(splits, xq);
    const unsigned int c = claim >> 3;
    const int rb = row_blocks - 1 - (int)(c / (unsigned int)nsx);
    const int split = xq + 8 * (int)(c % (unsigned int)nsx);
    const int row0 = rb * kRows;
    const int split_lo = split * kps;
    const int split_hi = n - split_lo < kps ? n : split_lo + kps;

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
    const ItemGeom geo = item_geom(lo, hi, split_lo, split_hi);
    const int tile_lo = geo.tile_lo, tile_end = geo.tile_end, ntiles = geo.ntiles;
    const int rows_here = min(kRows, a.m - row0);

    if (clean) {
      // -inf over the split's columns that no tile below covers
      const int w0 = tile_lo - split_lo;
      const int w1 = split_hi - tile_end;
      for (int r = 0; r < rows_here; ++r) {
        float* out = a.logits + (int64_t)(row0 + r) * a.ld;
        for (int c2 = tid; c2 < w0; c2 += kThreads) out[split_lo + c2] = -INFINITY;
        for (int c2 = tid; c2 < w1; c2 += kThreads) out[tile_end + c2] = -INFINITY;
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

    // A tile's 128 key rows are 16 KiB contiguous in kv, so this thread's 16-byte chunk ci = tid + c2 *
    // kThreads lies ci * 16 bytes from the tile's first key: a whole tile loads from one uniform base
    // plus per-thread constant offsets, with no bounds checks.  Only a tile that runs past the last
    // key clamps its key index to n - 1; those keys' logits are never stored (interior tiles end at or
    // before every row's window end, edge tiles store only keys below tile_end <= n).
    v4i stage[kChunksPerThread];
    float stage_scale = 0.f;
    auto gload = [&](int tile) {
      if (tile + kTileKeys <= n) {
        const uint8_t* tb = a.kv + (size_t)tile * kDim;
#pragma unroll
        for (int c2 = 0; c2 < kChunksPerThread; ++c2)
          stage[c2] = *reinterpret_cast<const v4i*>(tb + (tid + c2 * kThreads) * 16);
        if (tid < kTileKeys) stage_scale = a.kv_scale[tile + tid];
      } else {
#pragma unroll
        for (int c2 = 0; c2 < kChunksPerThread; ++c2) {
          const int ci = tid + c2 * kThreads;
          const int j = min(tile + (ci >> 3), n - 1);
          stage[c2] = *reinterpret_cast<const v4i*>(a.kv + (size_t)j * kDim + (ci & 7) * 16);
        }
        if (tid < kTileKeys) stage_scale = a.kv_scale[min(tile + tid, n - 1)];
      }
    };
    // LDS offsets of this thread's chunks in a tile buffer (rows swizzled by key & 7), fixed per thread
    int soff[kChunksPerThread];
#pragma unroll
    for (int c2 = 0; c2 < kChunksPerThread; ++c2) {
      const int ci = tid + c2 * kThreads;
      const int key = ci >> 3;
      soff[c2] = key * kDim + (((ci & 7) ^ (key & 7)) * 16);
    }
    auto lstore = [&](int buf) {
      uint8_t* sb = &s_kv[buf][0];
#pragma unroll
      for (int c2 = 0; c2 < kChunksPerThread; ++c2) *reinterpret_cast<v4i*>(sb + soff[c2]) = stage[c2];
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

// Work-queue counters of indexer_logits_ragged_noalloc, for callers that cannot allocate: one set
// per device (each GPU holds its own copy of this array until the process ends), shared by every
// call of that entry on the device.  Host code must not use the array's name as an address: it
// names a host-side stand-in.  The device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is passed to kernels.
static __device__ __align__(256) unsigned int scratch[kRaggedQueueBytes / sizeof(unsigned int)];

constexpr int kScratchDevices = 64;
static std::once_flag g_scratch_once[kScratchDevices];
static unsigned int* g_scratch_ptr[kScratchDevices];
static hipError_t g_scratch_err[kScratchDevices];

hipError_t ragged_noalloc_queue(unsigned int** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev]() {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? static_cast<unsigned int*>(ptr) : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

void query_ragged_occupancy(DeviceInfo& d) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, logits_ragged_kernel<kWaves>, 64 * kWaves, 0) != hipSuccess)
    per_cu = 1;
  d.ragged_wgs_per_cu = per_cu > 0 ? per_cu : 1;
}

hipError_t launch_logits_ragged(const RaggedLogitsArgs& a, const DeviceInfo& dev, hipStream_t s) {
  if (a.m <= 0) return hipSuccess;
  const int64_t row_blocks = (a.m + kRowsPerItem - 1) / kRowsPerItem;
  // resident workgroups of this kernel on the whole device, rounded to XCDs
  int per_cu = dev.ragged_wgs_per_cu > 0 ? dev.ragged_wgs_per_cu : 1;
  if (a.wgs_per_cu > 0) per_cu = std::min(per_cu, (int)a.wgs_per_cu);
  int64_t resident = (int64_t)(dev.cu_count > 0 ? dev.cu_count : 256) * per_cu;
  if (resident >= 8) resident = resident / 8 * 8;
  // key splits: multiples of 8 (one queue per XCD), doubled until there are
  // about 8 items per resident workgroup, keeping >= 128 keys (1 tile) per split
  const int64_t max_splits = std::max<int64_t>(1, a.n / 128);
  int64_t splits = std::min<int64_t>(8, max_splits);
  while (splits * 2 <= max_splits && row_blocks * splits < 8 * resident) splits *= 2;
  int64_t kps = (std::max<int64_t>(a.n, 1) + splits - 1) / splits;
  kps = (kps + kTileKeys - 1) / kTileKeys * kTileKeys;
  splits = (std::max<int64_t>(a.n, 1) + kps - 1) / kps;
  const int64_t items = row_blocks * splits;
  if (items > 0x7fffffffLL) return hipErrorInvalidValue;
  const int64_t grid = std::min<int64_t>(items, resident);
  const bool use_queue = queues_needed((unsigned int)grid, (int)splits, (int)row_blocks);
  if (use_queue) {
    if (a.queue == nullptr) return hipErrorInvalidValue;
    hipLaunchKernelGGL(queue_clear_kernel, dim3(1), dim3(64), 0, s, a.queue);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(logits_ragged_kernel<kWaves>, dim3((unsigned)grid), dim3(64 * kWaves), 0, s, a,
                     (int)splits, (int)kps, use_queue ? 1 : 0);
  return hipGetLastError();
}

}  // namespace fp8idx
