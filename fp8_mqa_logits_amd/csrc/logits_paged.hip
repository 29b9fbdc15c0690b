// Paged-decode fp8 MQA logits for gfx950 (the paged form of the indexer named
// on the vessl-ai/sglang PR #87 page).
//
// Request b has next_n query rows (multi-token prediction); row t sees keys
// [0, row_len[b * next_n + t]).  Key j of request b is slot j % 64 of physical
// page block_table[b, j / 64] in the kv pool ([pages, 64, 128] fp8) and the
// scale pool ([pages, 64] float32).
//
// Work decomposition
// - A unit is (request, group of 4 query rows); it owns ceil(L / 64) pages,
//   L being the longest of its rows' lengths (clamped to the width), claimed
//   in chunks of 16 pages (4 for small batches).  The units' chunks, laid end
//   to end, are split into equal contiguous ranges, one per workgroup of a
//   persistent grid (one 8-wave workgroup per CU), found by each workgroup
//   with a wave-wide prefix scan of the chunk counts computed from the
//   device-side lengths: no host schedule or workspace.  Inside a workgroup, waves take chunks from its
//   range one at a time through an LDS counter.  Every CU gets the same work,
//   and a wave that its SIMD serves less often (issue favours older waves)
//   simply takes fewer chunks, so the waves finish together.
// - A wave holds the 4 query rows of its current unit (q and weights in
//   VGPRs, reloaded when the unit changes).  The next chunk is claimed and its
//   page ids loaded while the current chunk is scored; each page's 64 keys x
//   128 bytes (8 KiB, contiguous) stream straight from HBM into four MFMA
//   B-operands one page ahead of the page being scored, across chunk
//   boundaries.  Every kv byte is read once and is shared by the 4 query rows.
// - Scoring, ReLU, head weighting and the cross-lane head reduction are the
//   same register-resident core as the ragged kernel.
// - A chunk's logits (4 rows x 16 pages) collect in the wave's LDS buffer and
//   leave as contiguous 1 KiB stores, four per row, so each row receives an
//   aligned 4 KiB block at once (16 bytes per lane), when the rows are 16-byte
//   aligned; otherwise each key is stored on its own.
// - With clean set, keys past a unit's scored range are filled with -inf by a
//   second balanced split over (unit, 64-key block) pairs.  Keys inside a
//   row's window whose page id lies outside the pool get -inf in any case.
// - On request, each row's largest logit code per 16-key fragment is written
//   too (a 16-lane DPP max of the stored values): the top-k that follows in
//   the fused entry takes its threshold from these maxima and reads only the
//   fragments that reach it.

#include "device_common.hpp"
#include "launch.hpp"
#include "mqa_core.hpp"

namespace fp8idx {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kPage = 64;
constexpr int kPagedWaves = 8;         // one workgroup per CU (2 waves per SIMD)
constexpr int kPagedDepth = 2;         // pages in flight per wave, the scored one included
// Pages a wave claims at a time: 16 when the grid has pages to spare (each row's logits then leave in
// aligned 4 KiB blocks), 4 for small batches, whose few chunks would leave most waves idle.
constexpr int kChunkLarge = 16;
constexpr int kChunkSmall = 4;
// The launcher takes the large chunk when the block tables can hold this many pages in total.
constexpr int64_t kChunkLargeMinPages = 131072;
constexpr int kMinChunksPerWg = 2;     // small totals run on fewer workgroups
constexpr int kFragsPerPage = kPage / 16;   // 16-key MFMA fragments per page

// One page's four B-operands (lane l: key l % 16 of each 16-key fragment,
// bytes 32 * (l / 16) .. +32) and its 64 kv scales (lane l: key l).  The loads are unconditional (an
// invalid page id reads page 0, whose values the caller never stores), so
// every path through the page loop has the same loads in flight and the
// compiler's wait counts stay exact.
struct PageFrags {
  v8i b[kFragsPerPage];
  float sc;
};

__device__ __forceinline__ void load_page(const PagedLogitsArgs& a, int32_t page, int lane, PageFrags& pf) {
  const bool ok = page >= 0 && page < a.num_pages;
  const int64_t pidx = ok ? page : 0;
#pragma unroll
  for (int f = 0; f < kFragsPerPage; ++f) {
    const int64_t slot = pidx * kPage + f * 16 + (lane & 15);
    const v4i* ptr = reinterpret_cast<const v4i*>(a.kv_pool + slot * kDim + 32 * (lane >> 4));
    const v4i x = ptr[0];
    const v4i y = ptr[1];
    pf.b[f] = v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  }
  pf.sc = a.scale_pool[pidx * kPage + lane];
}

// Rows, lengths and page count of unit u = (request u / qgroups, row group u % qgroups).
struct Unit {
  int b, r_base, nq, lmax;
  int len[4];
};

__device__ __forceinline__ Unit unit_at(const PagedLogitsArgs& a, int qgroups, int u) {
  Unit t;
  t.b = u / qgroups;
  const int qg = u - t.b * qgroups;
  t.r_base = t.b * a.next_n + 4 * qg;
  t.nq = min(4, a.next_n - 4 * qg);
  t.lmax = 0;
#pragma unroll
  for (int qi = 0; qi < 4; ++qi) {
    t.len[qi] = qi < t.nq ? min(max(a.row_len[t.r_base + qi], 0), a.width) : 0;
    t.lmax = max(t.lmax, t.len[qi]);
  }
  return t;
}

// Claimable chunks of unit u: its pages in runs of CHUNK (the last run may be shorter).
template <int CHUNK>
__device__ __forceinline__ int unit_chunks(const Unit& t) { return ((t.lmax + kPage - 1) / kPage + CHUNK - 1) / CHUNK; }

template <int CHUNK>
__device__ __forceinline__ int unit_chunks_at(const PagedLogitsArgs& a, int qgroups, int units, int u) {
  if (u >= units) return 0;
  return unit_chunks<CHUNK>(unit_at(a, qgroups, u));
}

static_assert(kPagedDepth == 2, "the chunk loop keeps one page in flight ahead of the scored one");

// VEC_STORE: the logits rows are 16-byte aligned (ld a multiple of 4, base aligned), so a chunk's
// logits go out as 16-byte stores, CHUNK / 4 contiguous 1 KiB stores per row (see below); otherwise
// as one 4-byte store per key.  CHUNK: pages per claimed chunk (kChunkLarge or kChunkSmall).
template <int DEPTH, bool VEC_STORE, int CHUNK>
__global__ __launch_bounds__(64 * kPagedWaves, 1) void logits_paged_kernel(PagedLogitsArgs a, int qgroups) {
  static_assert(CHUNK % kPagedDepth == 0, "chunks start on the first page buffer");
  static_assert(CHUNK * kPage % 256 == 0, "a chunk's logits leave in 256-key slices, 4 keys per lane");
  constexpr int kStageLd = CHUNK * kPage + 16;   // row stride of a wave's logits staging buffer (floats)
  __shared__ int s_next;   // next chunk of this workgroup's range to hand out
  // Per wave: one chunk's logits of the unit's 4 rows, rows kStageLd floats apart (16 floats of
  // padding keep the four rows' writes on different banks).
  __shared__ float s_stage[kPagedWaves][4 * kStageLd];
  // Per wave: the chunk's fragment maxima of the unit's 4 rows (rows 4 * CHUNK apart, as they leave).
  __shared__ uint32_t s_fstage[kPagedWaves][4 * 4 * CHUNK];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t waves_total = (int64_t)gridDim.x * kPagedWaves;
  const int64_t gw = (int64_t)blockIdx.x * kPagedWaves + wave;
  const int units = a.B * qgroups;
  const bool clean = a.clean != 0;
  const int my_q = reduce_rows4_qsel(lane);

  // Total chunks over all units (the first 64 units' counts are kept for the search below).
  const int c_first = unit_chunks_at<CHUNK>(a, qgroups, units, lane);
  int64_t total = __builtin_amdgcn_readfirstlane(wave_sum(c_first));
  for (int c = 64; c < units; c += 64)
    total += __builtin_amdgcn_readfirstlane(wave_sum(unit_chunks_at<CHUNK>(a, qgroups, units, c + lane)));
  total = uniform64(total);

  // This workgroup's equal share of the chunks.  Its waves take chunks from the share one at a time
  // through an LDS counter, so a wave that the SIMD serves less often simply takes fewer.
  const int64_t ng = min((int64_t)gridDim.x, max<int64_t>((total + kMinChunksPerWg - 1) / kMinChunksPerWg, 1));
  int64_t c0 = 0, ccount = 0;
  if (blockIdx.x < ng) split_range(total, ng, blockIdx.x, c0, ccount);
  if (threadIdx.x == 0) s_next = 0;
  __syncthreads();

  // Cursor: the unit holding the latest claimed chunk and the index of its first chunk.  Claims of
  // one wave only grow, so the cursor only moves forward.
  int cu = 0;
  int64_t cstart = 0;
  if (ccount > 0) {
    int64_t run = 0;
    for (int c = 0; c < units; c += 64) {
      const int p = c == 0 ? c_first : unit_chunks_at<CHUNK>(a, qgroups, units, c + lane);
      const int incl = wave_inclusive_scan(p, lane);
      const int chunk = __builtin_amdgcn_readlane(incl, 63);
      if (c0 - run < chunk) {
        const int t = (int)(c0 - run);
        const int first = __builtin_amdgcn_readfirstlane(__builtin_ctzll(ballot64(incl > t)));
        cu = c + first;
        cstart = run + __builtin_amdgcn_readlane(incl, first) - __builtin_amdgcn_readlane(p, first);
        break;
      }
      run += chunk;
    }
  }
  Unit ct = unit_at(a, qgroups, min(cu, units - 1));
  int ct_chunks = unit_chunks<CHUNK>(ct);

  // Claims the next chunk: its unit, first page, page count (0: none left) and page ids (lane l:
  // page l, lanes past the count repeat the last one).  The id load is unconditional (entry 0 of the
  // table when nothing is left), so every path leaves the same loads in flight, and its value is not
  // touched here: the wait for it comes where it is used, after the loads issued before it.
  int nx_u = 0, nx_pg = 0, nx_n = 0;
  int32_t nx_ids = -1;
  auto claim = [&]() {
    int rel = 0;
    if (lane == 0) rel = atomicAdd(&s_next, 1);
    rel = __builtin_amdgcn_readfirstlane(rel);
    int64_t idx = 0;
    nx_n = 0;
    if (rel < ccount) {
      const int64_t c = c0 + rel;
      while (c >= cstart + ct_chunks) {
        cstart += ct_chunks;
        ++cu;
        ct = unit_at(a, qgroups, cu);
        ct_chunks = unit_chunks<CHUNK>(ct);
      }
      nx_u = cu;
      nx_pg = (int)(c - cstart) * CHUNK;
      nx_n = min(CHUNK, (ct.lmax + kPage - 1) / kPage - nx_pg);
      idx = (int64_t)ct.b * a.max_pages + nx_pg + min(lane, nx_n - 1);
    }
    nx_ids = a.block_table[idx];
  };

  claim();
  PageFrags buf[DEPTH];
  load_page(a, nx_n > 0 ? __builtin_amdgcn_readfirstlane(nx_ids) : -1, lane, buf[0]);
  Unit t{};
  QFrags qf;
  int q_u = -1;
  int covered = 0, my_len = 0;
  bool row_ok = false;
  float* __restrict__ out_row = a.logits;
  float* const stage = s_stage[wave];
  uint32_t* const fstage = s_fstage[wave];

  while (nx_n > 0) {
    // the claimed chunk becomes the current one; the cursor still sits on its unit
    const int cur_pg = nx_pg, cur_n = nx_n;
    const int32_t cur_pidv = lane < cur_n ? nx_ids : -1;
    if (nx_u != q_u) {
      q_u = nx_u;
      t = ct;
      // a unit with fewer than 4 rows repeats its first row in the missing
      // slots (unconditional loads again); those lanes never store
#pragma unroll
      for (int qi = 0; qi < 4; ++qi) {
        const int row = qi < t.nq ? t.r_base + qi : t.r_base;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          qf.a[qi][h] = load_q_frag(a.q, row, true, h, lane);
          qf.w[qi][h] = load_w4(a.weights, row, true, h, lane);
        }
      }
      // scored keys of this unit: whole 16-key fragments up to the longest row
      covered = min(a.width, (t.lmax + 15) / 16 * 16);
      row_ok = my_q < t.nq;
      // selects instead of an indexed read, which would put the array in LDS
      my_len = (my_q & 2) ? ((my_q & 1) ? t.len[3] : t.len[2]) : ((my_q & 1) ? t.len[1] : t.len[0]);
      out_row = a.logits + (int64_t)(row_ok ? t.r_base + my_q : 0) * a.ld;
    }
    claim();   // the next chunk's page ids load while this chunk is scored

    // Scores chunk page i from pf; a step past the chunk's end (live false)
    // computes on page 0's data and stores nothing.  Keys of the row's window
    // on a page id outside the pool hold no kv: they get -inf (whatever
    // `clean` says), so a top-k over the window never reads a stale value.
    auto score_page = [&](int i, const PageFrags& pf) {
      const bool live = i < cur_n;
      const int32_t pid = __builtin_amdgcn_readlane(cur_pidv, i);
      const bool ok = pid >= 0 && pid < a.num_pages;
      // all four fragments are scored before any store, so their MFMAs and
      // epilogues share one scheduling region
      float v[kFragsPerPage];
#pragma unroll
      for (int f = 0; f < kFragsPerPage; ++f)
        v[f] = fragment_logit(qf, pf.b[f]) * __shfl(pf.sc, f * 16 + (lane & 15));
      uint32_t fmax[kFragsPerPage];
#pragma unroll
      for (int f = 0; f < kFragsPerPage; ++f) {
        const int j = (cur_pg + i) * kPage + f * 16 + (lane & 15);
        const bool inwin = j < my_len;
        const float st = ok && inwin ? v[f] : -INFINITY;
        if constexpr (VEC_STORE)
          stage[my_q * kStageLd + i * kPage + f * 16 + (lane & 15)] = st;
        else if (live && row_ok && j < covered && (inwin || clean))
          out_row[j] = st;
        // the fragment's largest in-window code for the top-k (0 for keys outside the window)
        if (a.frag_max) fmax[f] = row16_max_u32(live && row_ok && inwin ? float_to_ordered(st) : 0u);
      }
      if constexpr (VEC_STORE) {
        if (a.frag_max) {
          // lanes 0..3 of each 16-lane row stage that row's four fragment maxima of this page
          // (0 past the chunk's pages, past the row's window and for rows the unit lacks)
          const int c = lane & 15;
          const uint32_t m = c == 0 ? fmax[0] : c == 1 ? fmax[1] : c == 2 ? fmax[2] : fmax[3];
          if (c < kFragsPerPage) fstage[my_q * (4 * CHUNK) + i * kFragsPerPage + c] = m;
        }
      }
    };
    // One page loads while the previous one is scored; the chunk's last step
    // loads the next chunk's first page.
#pragma unroll
    for (int d = 0; d < CHUNK; ++d) {
      int32_t np;
      if (d + 1 < CHUNK)
        np = d + 1 < cur_n ? __builtin_amdgcn_readlane(cur_pidv, d + 1) : -1;
      else
        np = nx_n > 0 ? __builtin_amdgcn_readfirstlane(nx_ids) : -1;
      load_page(a, np, lane, buf[(d + 1) % DEPTH]);
      score_page(d, buf[d % DEPTH]);
    }
    if constexpr (VEC_STORE) {
      // The chunk's logits leave the staging buffer in 256-key slices, one contiguous 1 KiB store
      // per row and slice: lane l writes keys 4 l .. 4 l + 3 of the slice.  LDS operations of one
      // wave complete in order, so these reads see the chunk's writes and the next chunk's writes
      // come after them; the wave barriers keep the compiler from moving them.  Staged values already hold -inf outside each
      // row's window; a lane stores the keys of the window (all keys with clean) below the unit's
      // scored range on the chunk's pages.
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int sl = 0; sl < CHUNK * kPage; sl += 256) {
        const int c0 = sl + 4 * lane;
        const int j0 = cur_pg * kPage + c0;
        const bool page_live = c0 < cur_n * kPage;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const v4f x = *reinterpret_cast<const v4f*>(stage + r * kStageLd + c0);
          const int len = t.len[r];
          const bool rok = page_live && r < t.nq;
          bool p[4];
          bool all = true;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            p[c] = rok && j0 + c < covered && (j0 + c < len || clean);
            all = all && p[c];
          }
          float* dst = a.logits + (int64_t)(r < t.nq ? t.r_base + r : 0) * a.ld + j0;
          if (all) {
            *reinterpret_cast<v4f*>(dst) = x;
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (p[c]) dst[c] = x[c];
          }
        }
      }
      if (a.frag_max) {
        // the chunk's maxima block (a.frag.rows rows of 4 * CHUNK fragments, contiguous): lane l
        // writes elements 4 l .. 4 l + 3
        const int blk = a.frag.rows * (4 * CHUNK);
        if (4 * lane < blk) {
          const v4u x = *reinterpret_cast<const v4u*>(fstage + 4 * lane);
          const int64_t idx = (int64_t)q_u * a.frag.unit_stride + (int64_t)(cur_pg / CHUNK) * blk + 4 * lane;
          if (idx + 4 <= a.frag.elems) *reinterpret_cast<v4u*>(a.frag_max + idx) = x;
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }

  if (!clean) return;
  // -inf for keys [covered, width) of every row, split evenly over all waves
  // in (unit, 64-key block) steps.
  const int blocks = (a.width + kPage - 1) / kPage;
  int64_t f0 = 0, fn = 0;
  split_range((int64_t)units * blocks, waves_total, gw, f0, fn);
  int cur = -1;
  Unit ft{};
  int fcovered = 0;
  for (int64_t x = f0; x < f0 + fn; ++x) {
    const int fu = (int)(x / blocks);
    const int j = (int)(x - (int64_t)fu * blocks) * kPage + lane;
    if (fu != cur) {
      cur = fu;
      ft = unit_at(a, qgroups, fu);
      fcovered = min(a.width, (ft.lmax + 15) / 16 * 16);
    }
    if (j >= fcovered && j < a.width) {
      for (int qi = 0; qi < ft.nq; ++qi) a.logits[(int64_t)(ft.r_base + qi) * a.ld + j] = -INFINITY;
    }
  }
}

void query_paged_occupancy(DeviceInfo& d) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, logits_paged_kernel<kPagedDepth, true, kChunkLarge>,
                                                   64 * kPagedWaves, 0) != hipSuccess)
    per_cu = 1;
  d.paged_wgs_per_cu = per_cu > 0 ? per_cu : 1;
}

// Pages per claimed chunk: the large chunk when the block tables can name at least
// kChunkLargeMinPages pages in all (every unit's rows clamped to the table and the width).
static int chunk_pages(int32_t B, int qgroups, int32_t max_pages, int32_t width) {
  const int64_t table_pages = std::min<int64_t>(max_pages, ((int64_t)width + kPage - 1) / kPage);
  return (int64_t)B * qgroups * table_pages >= kChunkLargeMinPages ? kChunkLarge : kChunkSmall;
}

static int chunk_pages(const PagedLogitsArgs& a, int qgroups) { return chunk_pages(a.B, qgroups, a.max_pages, a.width); }

FragLayout paged_frag_layout(int32_t B, int32_t next_n, int32_t max_pages, int32_t width) {
  FragLayout f{};
  const int qgroups = (next_n + 3) / 4;
  const int chunk = chunk_pages(B, qgroups, max_pages, width);
  const int64_t pages = ((int64_t)std::max(width, 0) + kPage - 1) / kPage;
  f.rows = std::min(4, std::max(next_n, 1));
  f.fpc = 4 * chunk;
  f.unit_stride = (pages + chunk - 1) / chunk * (int64_t)f.rows * f.fpc;
  f.elems = 0;
  return f;
}

hipError_t launch_logits_paged(const PagedLogitsArgs& a, const DeviceInfo& dev, hipStream_t s) {
  if (a.B <= 0 || a.width <= 0) return hipSuccess;
  const int qgroups = (a.next_n + 3) / 4;
  if ((int64_t)a.B * qgroups > 0x7fffffffLL) return hipErrorInvalidValue;
  const int per_cu = dev.paged_wgs_per_cu > 0 ? dev.paged_wgs_per_cu : 1;
  const int64_t grid = (int64_t)(dev.cu_count > 0 ? dev.cu_count : 256) * per_cu;
  const bool vec = (a.ld & 3) == 0 && (reinterpret_cast<uintptr_t>(a.logits) & 15) == 0;
  // the fragment maxima leave as 16-byte stores from the staged chunk: aligned rows only
  if (a.frag_max != nullptr &&
      (!vec || (reinterpret_cast<uintptr_t>(a.frag_max) & 15) != 0 || a.frag.fpc != 4 * chunk_pages(a, qgroups)))
    return hipErrorInvalidValue;
  const bool large = chunk_pages(a, qgroups) == kChunkLarge;
  const dim3 g((unsigned)grid), blk(64 * kPagedWaves);
  if (vec && large)
    hipLaunchKernelGGL((logits_paged_kernel<kPagedDepth, true, kChunkLarge>), g, blk, 0, s, a, qgroups);
  else if (vec)
    hipLaunchKernelGGL((logits_paged_kernel<kPagedDepth, true, kChunkSmall>), g, blk, 0, s, a, qgroups);
  else if (large)
    hipLaunchKernelGGL((logits_paged_kernel<kPagedDepth, false, kChunkLarge>), g, blk, 0, s, a, qgroups);
  else
    hipLaunchKernelGGL((logits_paged_kernel<kPagedDepth, false, kChunkSmall>), g, blk, 0, s, a, qgroups);
  return hipGetLastError();
}

}  // namespace fp8idx
