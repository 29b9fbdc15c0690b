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
//   L being the longest of its rows' lengths (clamped to the width).  The
//   units' pages, laid end to end, are split into equal contiguous ranges,
//   one per wave of a persistent grid (every resident wave of the device), so
//   each wave gets the same number of pages whatever the mix of context
//   lengths: no tail round of half-empty workgroups.  Each wave finds its
//   first (unit, page) with a wave-wide prefix scan of the units' page counts,
//   computed from the device-side lengths, so no host schedule or workspace
//   is needed.  Waves never synchronise with each other.
// - A wave holds the 4 query rows of its current unit (q and weights in
//   VGPRs), reads the page ids of its range with one vector load, and streams
//   each page's 64 keys x 128 bytes (8 KiB, contiguous) straight from HBM into
//   four MFMA B-operands, DEPTH pages deep: while one page is scored the next
//   DEPTH - 1 pages' loads are in flight.  Every kv byte is read once and is
//   shared by the 4 query rows.
// - Scoring, ReLU, head weighting and the cross-lane head reduction are the
//   same register-resident core as the ragged kernel.
// - With clean set, keys past a unit's scored range are filled with -inf by a
//   second balanced split over (unit, 64-key block) pairs.

#include "device_common.hpp"
#include "launch.hpp"
#include "mqa_core.hpp"

namespace fp8idx {

constexpr int kPage = 64;
constexpr int kPagedWaves = 4;
constexpr int kPagedDepth = 2;         // pages in flight per wave, the scored one included
constexpr int kMinPagesPerWave = 4;    // small totals run on fewer waves
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

__device__ __forceinline__ int unit_pages(const PagedLogitsArgs& a, int qgroups, int units, int u) {
  if (u >= units) return 0;
  return (unit_at(a, qgroups, u).lmax + kPage - 1) / kPage;
}

template <int DEPTH>
__global__ __launch_bounds__(64 * kPagedWaves, 2) void logits_paged_kernel(PagedLogitsArgs a, int qgroups) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t waves_total = (int64_t)gridDim.x * kPagedWaves;
  const int64_t gw = (int64_t)blockIdx.x * kPagedWaves + wave;
  const int units = a.B * qgroups;
  const bool clean = a.clean != 0;
  const int my_q = reduce_rows4_qsel(lane);

  // Total pages over all units (the first 64 units' counts are kept for the search below).
  int p_first = unit_pages(a, qgroups, units, lane);
  int64_t total = __builtin_amdgcn_readfirstlane(wave_sum(p_first));
  for (int c = 64; c < units; c += 64)
    total += __builtin_amdgcn_readfirstlane(wave_sum(unit_pages(a, qgroups, units, c + lane)));
  total = uniform64(total);

  const int64_t nw = min(waves_total, max<int64_t>((total + kMinPagesPerWave - 1) / kMinPagesPerWave, 1));
  int64_t start = 0, count = 0;
  if (gw < nw) split_range(total, nw, gw, start, count);

  // Locate the unit holding page `start` of the concatenation, and the page within it.
  int u = 0;
  int off = 0;
  if (count > 0) {
    int64_t run = 0;
    for (int c = 0; c < units; c += 64) {
      const int p = c == 0 ? p_first : unit_pages(a, qgroups, units, c + lane);
      const int incl = wave_inclusive_scan(p, lane);
      const int chunk = __builtin_amdgcn_readlane(incl, 63);
      if (start - run < chunk) {
        const int t = (int)(start - run);
        const int first = __builtin_amdgcn_readfirstlane(__builtin_ctzll(ballot64(incl > t)));
        u = c + first;
        off = t - (__builtin_amdgcn_readlane(incl, first) - __builtin_amdgcn_readlane(p, first));
        break;
      }
      run += chunk;
    }
  }

  for (int64_t remaining = count; remaining > 0 && u < units; ++u, off = 0) {
    const Unit t = unit_at(a, qgroups, u);
    const int pages = (t.lmax + kPage - 1) / kPage;
    const int n_here = (int)min<int64_t>(pages - off, remaining);
    remaining -= max(n_here, 0);
    if (n_here <= 0) continue;
    const int32_t* __restrict__ bt = a.block_table + (int64_t)t.b * a.max_pages + off;
    // scored keys of this unit: whole 16-key fragments up to the longest row
    const int covered = min(a.width, (t.lmax + 15) / 16 * 16);
    const bool row_ok = my_q < t.nq;
    const int my_len = t.len[my_q];
    float* __restrict__ out_row = a.logits + (int64_t)(row_ok ? t.r_base + my_q : 0) * a.ld;

    for (int s0 = 0; s0 < n_here; s0 += 64) {
      const int seg = min(64, n_here - s0);
      // page ids of this segment, one per lane; loaded before q so q's loads
      // overlap the wait for them
      const int32_t pidv = lane < seg ? bt[s0 + lane] : -1;
      // a unit with fewer than 4 rows repeats its first row in the missing
      // slots (unconditional loads again); those lanes never store
      QFrags qf;
#pragma unroll
      for (int qi = 0; qi < 4; ++qi) {
        const int row = qi < t.nq ? t.r_base + qi : t.r_base;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          qf.a[qi][h] = load_q_frag(a.q, row, true, h, lane);
          qf.w[qi][h] = load_w4(a.weights, row, true, h, lane);
        }
      }
      const int page0 = off + s0;   // first page of the segment within the unit
      // page id of segment page i; -1 past the segment's end
      auto pid_of = [&](int i) { return i < seg ? __builtin_amdgcn_readlane(pidv, min(i, 63)) : -1; };
      // Scores segment page i from pf; a step past the segment's end (live
      // false) computes on page 0's data and stores nothing.
      auto score_page = [&](int i, const PageFrags& pf) {
        const bool live = i < seg;
        const int32_t pid = pid_of(i);
        const bool ok = pid >= 0 && pid < a.num_pages;
        // all four fragments are scored before any store, so their MFMAs and
        // epilogues share one scheduling region
        float v[kFragsPerPage];
#pragma unroll
        for (int f = 0; f < kFragsPerPage; ++f)
          v[f] = fragment_logit(qf, pf.b[f]) * __shfl(pf.sc, f * 16 + (lane & 15));
#pragma unroll
        for (int f = 0; f < kFragsPerPage; ++f) {
          const int j = (page0 + i) * kPage + f * 16 + (lane & 15);
          const bool val = ok && j < my_len;
          if (live && row_ok && j < covered && (val || clean)) out_row[j] = val ? v[f] : -INFINITY;
        }
      };
      // DEPTH - 1 pages are loading while one is scored; the loop runs whole
      // groups of DEPTH steps, the steps past the segment's end storing nothing.
      PageFrags buf[DEPTH];
#pragma unroll
      for (int d = 0; d < DEPTH - 1; ++d) load_page(a, pid_of(d), lane, buf[d]);
      for (int i = 0; i < seg; i += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
          load_page(a, pid_of(i + d + DEPTH - 1), lane, buf[(d + DEPTH - 1) % DEPTH]);
          score_page(i + d, buf[d]);
        }
      }
    }
  }

  if (!clean) return;
  // -inf for keys [covered, width) of every row, split evenly over all waves
  // in (unit, 64-key block) steps.
  const int blocks = (a.width + kPage - 1) / kPage;
  int64_t f0 = 0, fn = 0;
  split_range((int64_t)units * blocks, waves_total, gw, f0, fn);
  int cur = -1;
  Unit t{};
  int covered = 0;
  for (int64_t x = f0; x < f0 + fn; ++x) {
    const int fu = (int)(x / blocks);
    const int j = (int)(x - (int64_t)fu * blocks) * kPage + lane;
    if (fu != cur) {
      cur = fu;
      t = unit_at(a, qgroups, fu);
      covered = min(a.width, (t.lmax + 15) / 16 * 16);
    }
    if (j >= covered && j < a.width) {
      for (int qi = 0; qi < t.nq; ++qi) a.logits[(int64_t)(t.r_base + qi) * a.ld + j] = -INFINITY;
    }
  }
}

void query_paged_occupancy(DeviceInfo& d) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, logits_paged_kernel<kPagedDepth>, 64 * kPagedWaves,
                                                   0) != hipSuccess)
    per_cu = 1;
  d.paged_wgs_per_cu = per_cu > 0 ? per_cu : 1;
}

hipError_t launch_logits_paged(const PagedLogitsArgs& a, const DeviceInfo& dev, hipStream_t s) {
  if (a.B <= 0 || a.width <= 0) return hipSuccess;
  const int qgroups = (a.next_n + 3) / 4;
  if ((int64_t)a.B * qgroups > 0x7fffffffLL) return hipErrorInvalidValue;
  const int per_cu = dev.paged_wgs_per_cu > 0 ? dev.paged_wgs_per_cu : 1;
  const int64_t grid = (int64_t)(dev.cu_count > 0 ? dev.cu_count : 256) * per_cu;
  hipLaunchKernelGGL(logits_paged_kernel<kPagedDepth>, dim3((unsigned)grid), dim3(64 * kPagedWaves), 0, s, a,
                     qgroups);
  return hipGetLastError();
}

}  // namespace fp8idx
