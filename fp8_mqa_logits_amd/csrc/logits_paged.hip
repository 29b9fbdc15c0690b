// Paged-decode fp8 MQA logits for gfx950 (the paged form of the indexer named
// on the vessl-ai/sglang PR #87 page).
//
// Request b has next_n query rows (multi-token prediction); row t sees keys
// [0, row_len[b * next_n + t]).  Key j of request b is slot j % 64 of physical
// page block_table[b, j / 64] in the kv pool ([pages, 64, 128] fp8) and the
// scale pool ([pages, 64] float32).
//
// Work decomposition
// - Grid x: (request, group of 4 query rows); grid y: chunks of kKeysPerWG
//   keys.  A workgroup first reads its rows' lengths and exits when its key
//   chunk lies past all of them, so the split of each request's keys over
//   workgroups follows the device-side lengths without any host schedule.
// - All 4 waves hold the same 4 query rows (q and weights in VGPRs) and take
//   interleaved whole pages of the chunk: one wave-uniform page-id lookup per
//   page, then the page's 64 keys x 128 bytes (8 KiB, contiguous) go straight
//   from HBM into four MFMA B-operands.  Every kv byte is read once and is
//   shared by the 4 query rows of the request; two pages per wave are in
//   flight before any is scored.
// - Scoring, ReLU, head weighting and the cross-lane head reduction are the
//   same register-resident core as the ragged kernel.

#include "device_common.hpp"
#include "launch.hpp"
#include "mqa_core.hpp"

namespace fp8idx {

constexpr int kPage = 64;
constexpr int kKeysPerWG = 1024;
constexpr int kPagedWaves = 4;
constexpr int kPagesInFlight = 2;                 // pages loaded ahead per wave
constexpr int kFragsPerPage = kPage / 16;         // 16-key MFMA fragments per page

__global__ __launch_bounds__(64 * kPagedWaves, 2) void logits_paged_kernel(PagedLogitsArgs a, int qgroups) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b = blockIdx.x / qgroups;
  const int qg = blockIdx.x - b * qgroups;
  const int nn = a.next_n;
  const int r_base = b * nn + 4 * qg;
  const int nq = min(4, nn - 4 * qg);

  int len[4];
  int lmax = 0;
#pragma unroll
  for (int qi = 0; qi < 4; ++qi) {
    len[qi] = qi < nq ? min(max(a.row_len[r_base + qi], 0), a.width) : 0;
    lmax = max(lmax, len[qi]);
  }
  const int c_lo = blockIdx.y * kKeysPerWG;
  const int c_hi = min(a.width, c_lo + kKeysPerWG);
  if (c_lo >= c_hi) return;
  const int khi = min(c_hi, lmax);
  const int nfrag = khi > c_lo ? (khi - c_lo + 15) / 16 : 0;
  const int covered = min(c_hi, c_lo + nfrag * 16);   // [c_lo, covered) handled by fragments

  if (a.clean && covered < c_hi) {
    for (int qi = 0; qi < nq; ++qi) {
      float* out = a.logits + (int64_t)(r_base + qi) * a.ld;
      for (int c = covered + tid; c < c_hi; c += 64 * kPagedWaves) out[c] = -INFINITY;
    }
  }
  if (nfrag == 0) return;

  QFrags qf;
#pragma unroll
  for (int qi = 0; qi < 4; ++qi) {
    const bool ok = qi < nq;
    const int row = ok ? r_base + qi : 0;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      qf.a[qi][t] = load_q_frag(a.q, row, ok, t, lane);
      qf.w[qi][t] = load_w4(a.weights, row, ok, t, lane);
    }
  }
  const int my_q = reduce_rows4_qsel(lane);
  const bool row_ok = my_q < nq;
  const int my_len = len[my_q];
  float* __restrict__ out_row = a.logits + (int64_t)(row_ok ? r_base + my_q : 0) * a.ld;
  const int32_t* __restrict__ bt = a.block_table + (int64_t)b * a.max_pages;
  const bool clean = a.clean != 0;

  // Wave w takes pages w, w + kPagedWaves, ... of the chunk, kPagesInFlight at a
  // time: the page ids are read first (wave-uniform scalar loads), then every
  // kv and scale load of those pages is issued, then the fragments are scored.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int first_page = c_lo / kPage;
  const int npages = (covered - c_lo + kPage - 1) / kPage;
  for (int pg0 = wave_u; pg0 < npages; pg0 += kPagedWaves * kPagesInFlight) {
    int64_t page[kPagesInFlight];
#pragma unroll
    for (int u = 0; u < kPagesInFlight; ++u) {
      const int pg = pg0 + u * kPagedWaves;
      page[u] = pg < npages ? (int64_t)bt[first_page + pg] : -1;
    }
    v8i bfrag[kPagesInFlight][kFragsPerPage];
    float sc[kPagesInFlight][kFragsPerPage];
#pragma unroll
    for (int u = 0; u < kPagesInFlight; ++u) {
      const bool ok = page[u] >= 0 && page[u] < a.num_pages;
      const int64_t pidx = ok ? page[u] : 0;
#pragma unroll
      for (int f = 0; f < kFragsPerPage; ++f) {
        const int64_t slot = pidx * kPage + f * 16 + (lane & 15);
        const v4i* ptr = reinterpret_cast<const v4i*>(a.kv_pool + slot * kDim + 32 * (lane >> 4));
        v4i x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
        float s = 0.f;
        if (ok) {
          x = ptr[0];
          y = ptr[1];
          s = a.scale_pool[slot];
        }
        bfrag[u][f] = v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
        sc[u][f] = s;
      }
    }
#pragma unroll
    for (int u = 0; u < kPagesInFlight; ++u) {
      const int pg = pg0 + u * kPagedWaves;
      if (pg < npages) {
        const bool ok = page[u] >= 0 && page[u] < a.num_pages;
#pragma unroll
        for (int f = 0; f < kFragsPerPage; ++f) {
          const float v = fragment_logit(qf, bfrag[u][f]) * sc[u][f];
          const int j = c_lo + pg * kPage + f * 16 + (lane & 15);
          if (row_ok && j < covered) {
            if (ok && j < my_len) {
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

hipError_t launch_logits_paged(const PagedLogitsArgs& a, const DeviceInfo& dev, hipStream_t s) {
  (void)dev;
  if (a.B <= 0 || a.width <= 0) return hipSuccess;
  const int qgroups = (a.next_n + 3) / 4;
  const int64_t gx = (int64_t)a.B * qgroups;
  const int64_t gy = (a.width + kKeysPerWG - 1) / kKeysPerWG;
  if (gx > 0x7fffffffLL || gy > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(logits_paged_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(64 * kPagedWaves), 0, s, a,
                     qgroups);
  return hipGetLastError();
}

}  // namespace fp8idx
