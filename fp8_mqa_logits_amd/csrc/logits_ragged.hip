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
//   buffered), loaded by 16-byte LDS-DMA loads (global_load_lds_dwordx4: no
//   staging registers, each instruction a coalesced 1 KiB).  Inside a row the
//   16-byte chunks are XOR-swizzled by (key & 7) so that the B-operand reads
//   (lane l: key l % 16, bytes 32 * (l / 16) .. +32) hit distinct banks.  A
//   tile's logits are stored after the next tile's barrier, so the wait for
//   each tile's loads before that barrier never waits on fresh stores.
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
  constexpr int kFrags = kTileKeys / 16;                           // 16-key MFMA fragments per tile
  constexpr int kDmaPerWave = kTileKeys * kDim / (1024 * WAVES);   // 1 KiB LDS-DMA blocks per wave per tile
  static_assert(kTileKeys * kDim % (1024 * WAVES) == 0, "tile blocks must divide the workgroup");
  static_assert(kTileKeys % 64 == 0, "scales load 64 per instruction");

  // Two tile buffers as separate arrays, so the compiler can tell the buffer being read from the one
  // being filled and puts no wait for the fill before the reads.
  __shared__ __attribute__((aligned(16))) uint8_t s_kv0[kTileKeys * kDim];
  __shared__ __attribute__((aligned(16))) uint8_t s_kv1[kTileKeys * kDim];
  __shared__ __attribute__((aligned(16))) float s_sc0[kTileKeys];
  __shared__ __attribute__((aligned(16))) float s_sc1[kTileKeys];
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

    // Tiles go from kv straight into LDS (16-byte LDS-DMA loads, no staging registers).  Lane l of
    // DMA block b (keys 8b .. 8b + 7 of the tile, 1 KiB) fills LDS bytes 1024 b + 16 l: key 8b + l / 8,
    // slot l % 8, which holds that key's 16-byte chunk (l % 8) ^ (key & 7) = (l % 8) ^ (l / 8), the
    // swizzle the B-operand reads expect.  Keys past the last one are clamped to n - 1; their logits
    // are never stored (interior tiles end at or before every row's window end, edge tiles store only
    // keys below tile_end <= n).
    const int dma_key = lane >> 3;
    const int dma_chunk = (lane & 7) ^ (lane >> 3);
    auto dma = [&](int tile, uint8_t* skv, float* ssc) {
#pragma unroll
      for (int i = 0; i < kDmaPerWave; ++i) {
        const int blk = wave * kDmaPerWave + i;
        const int key = min(tile + 8 * blk + dma_key, n - 1);
        __builtin_amdgcn_global_load_lds(a.kv + (size_t)key * kDim + dma_chunk * 16,
                                         (__attribute__((address_space(3))) void*)(skv + blk * 1024), 16, 0, 0);
      }
      for (int i = wave; i < kTileKeys / 64; i += WAVES) {
        const int key = min(tile + 64 * i + lane, n - 1);
        __builtin_amdgcn_global_load_lds(a.kv_scale + key, (__attribute__((address_space(3))) void*)(ssc + 64 * i),
                                         4, 0, 0);
      }
    };

    // A tile's logits are stored after the next tile's barrier, so that the wait for each tile's
    // loads before that barrier never waits on freshly issued stores.
    float pv[kFrags];
    int p_tile = -1;
    bool p_interior = false;
    auto store_tile = [&]() {
      const int tile = p_tile;
      if (p_interior) {
        // interior tile: every key is inside every row's window
        float* __restrict__ optr = out_row + tile + kl;
#pragma unroll
        for (int f = 0; f < kFrags; ++f) optr[f * 16] = pv[f];
      } else {
#pragma unroll
        for (int f = 0; f < kFrags; ++f) {
          const int j = tile + f * 16 + kl;
          if (row_ok && j < tile_end) {
            if (j >= my_ks && j < my_ke) {
              out_row[j] = pv[f];
            } else if (clean) {
              out_row[j] = -INFINITY;
            }
          }
        }
      }
    };
    auto tile_step = [&](int it, const uint8_t* cur_kv, const float* cur_sc, uint8_t* nxt_kv, float* nxt_sc) {
      const int tile = tile_lo + it * kTileKeys;
      __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of the tile have landed (and its older stores)
      __syncthreads();                 // ... and every wave's: the tile is in LDS, the other buffer is free
      if (it + 1 < ntiles) dma(tile + kTileKeys, nxt_kv, nxt_sc);
      if (p_tile >= 0) store_tile();
#pragma unroll
      for (int f = 0; f < kFrags; ++f) {
        const v4i b0 = *reinterpret_cast<const v4i*>(cur_kv + f * 16 * kDim + boff0);
        const v4i b1 = *reinterpret_cast<const v4i*>(cur_kv + f * 16 * kDim + boff1);
        const v8i b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        pv[f] = fragment_logit(qf, b) * cur_sc[f * 16 + kl];
      }
      p_tile = tile;
      p_interior = tile >= w_lo && tile + kTileKeys <= w_hi;
    };

    dma(tile_lo, s_kv0, s_sc0);
    for (int it = 0; it < ntiles; it += 2) {
      tile_step(it, s_kv0, s_sc0, s_kv1, s_sc1);
      if (it + 1 < ntiles) tile_step(it + 1, s_kv1, s_sc1, s_kv0, s_sc0);
    }
    store_tile();
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
