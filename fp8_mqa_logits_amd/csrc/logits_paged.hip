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
// - All 4 waves hold the same 4 query rows (q and weights in VGPRs); each
//   wave takes 16 consecutive pages of the 4096-key chunk, reads their ids up
//   front (wave-uniform scalar loads), and streams each page's 64 keys x 128
//   bytes (8 KiB, contiguous) straight from HBM into four MFMA B-operands,
//   double buffered: the next page loads while the current one is scored.
//   Every kv byte is read once and is shared by the 4 query rows.
// - Scoring, ReLU, head weighting and the cross-lane head reduction are the
//   same register-resident core as the ragged kernel.

#include "device_common.hpp"
#include "launch.hpp"
#include "mqa_core.hpp"

namespace fp8idx {

constexpr int kPage = 64;
constexpr int kPagedWaves = 4;
constexpr int kPagesPerWave = 16;                 // consecutive pages of the chunk per wave
constexpr int kKeysPerWG = kPagedWaves * kPagesPerWave * kPage;
constexpr int kFragsPerPage = kPage / 16;         // 16-key MFMA fragments per page

// One page's four B-operands (lane l: key l % 16 of each 16-key fragment,
// bytes 32 * (l / 16) .. +32) and kv scales; an invalid page id reads nothing.
struct PageFrags {
  v8i b[kFragsPerPage];
  float s[kFragsPerPage];
};

__device__ __forceinline__ void load_page(const PagedLogitsArgs& a, int32_t page, int lane, PageFrags& pf) {
  const bool ok = page >= 0 && page < a.num_pages;
  const int64_t pidx = ok ? page : 0;
#pragma unroll
  for (int f = 0; f < kFragsPerPage; ++f) {
    const int64_t slot = pidx * kPage + f * 16 + (lane & 15);
    const v4i* ptr = reinterpret_cast<const v4i*>(a.kv_pool + slot * kDim + 32 * (lane >> 4));
    v4i x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
    float sc = 0.f;
    if (ok) {
      x = ptr[0];
      y = ptr[1];
      sc = a.scale_pool[slot];
    }
    pf.b[f] = v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    pf.s[f] = sc;
  }
}

__global__ __launch_bounds__(64 * kPagedWaves, 2) void logits_paged_kernel(PagedLogitsArgs a, int qgroups) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b = blockIdx.x / qgroups;
  const int qg = blockIdx.x - b * qgroups;
  const int nn = a.next_n;
  const int r_base = b * nn + 4 * qg;
  const int nq = min(4, nn - 4 * qg);

  // q and the weights do not depend on the lengths: their loads go first.
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
  // this wave's pages: [wave * kPagesPerWave, + np) of the chunk's covered pages
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int chunk_pages = (covered - c_lo + kPage - 1) / kPage;
  const int np = min(max(chunk_pages - wave_u * kPagesPerWave, 0), kPagesPerWave);
  if (np == 0) return;   // no barriers below: waves finish independently
  const int wpage0 = c_lo / kPage + wave_u * kPagesPerWave;   // first logical page of the wave
  const int32_t* __restrict__ bt = a.block_table + (int64_t)b * a.max_pages;
  int32_t pid[kPagesPerWave];   // wave-uniform page ids, read up front
#pragma unroll
  for (int i = 0; i < kPagesPerWave; ++i) pid[i] = i < np ? bt[wpage0 + i] : -1;

  PageFrags buf[2];
  load_page(a, pid[0], lane, buf[0]);
  const int my_q = reduce_rows4_qsel(lane);
  const bool row_ok = my_q < nq;
  const int my_len = len[my_q];
  float* __restrict__ out_row = a.logits + (int64_t)(row_ok ? r_base + my_q : 0) * a.ld;
  const bool clean = a.clean != 0;

  auto score_page = [&](int i, const PageFrags& pf) {
    const bool ok = pid[i] >= 0 && pid[i] < a.num_pages;
#pragma unroll
    for (int f = 0; f < kFragsPerPage; ++f) {
      const float v = fragment_logit(qf, pf.b[f]) * pf.s[f];
      const int j = (wpage0 + i) * kPage + f * 16 + (lane & 15);
      if (row_ok && j < covered) {
        if (ok && j < my_len) {
          out_row[j] = v;
        } else if (clean) {
          out_row[j] = -INFINITY;
        }
      }
    }
  };
  // Double buffer: the next page's loads are in flight while a page is scored.
#pragma unroll
  for (int i = 0; i < kPagesPerWave; i += 2) {
    if (i < np) {
      if (i + 1 < np) load_page(a, pid[i + 1], lane, buf[1]);
      score_page(i, buf[0]);
      if (i + 1 < np) {
        if (i + 2 < np) load_page(a, pid[i + 2], lane, buf[0]);
        score_page(i + 1, buf[1]);
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
