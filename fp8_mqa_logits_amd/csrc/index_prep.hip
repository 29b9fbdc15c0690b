// Index preparation for the indexer: the `gen_nsa_ks_ke` step on the
// lightllm "parallel NSA ragged index copies" PR page (ks/ke of every query
// token plus the ragged memory-index buffer), and its decode / MTP form
// (per-row key counts and the requests' block-table rows).
//
// Ragged: request b holds seq_len[b] tokens, the last q_len[b] of which are
// queries; the keys of all requests lie back to back, request b's first at
// cu_seq[b].  Query t of request b sees keys [cu_seq[b], cu_seq[b] +
// seq_len[b] - q_len[b] + t + 1), and ragged key cu_seq[b] + p is kv slot
// table[req_idx[b], p].
//
// One launch, no host synchronisation: every workgroup scans the (at most
// kPrepMaxReq) request lengths into LDS, then grid-strides over the query
// tokens and over the ragged keys up to the caller's capacities, locating
// each element's request by binary search in the LDS prefix sums.  A thread
// copies four consecutive keys, so the table reads and the buffer writes are
// coalesced.

#include "device_common.hpp"
#include "launch.hpp"

#include <algorithm>

namespace fp8idx {

constexpr int kPrepThreads = 256;

// Largest b in [0, B) with cum[b] <= x (cum is non-decreasing, cum[0] = 0 <= x < cum[B]).
__device__ __forceinline__ int find_request(const int32_t* cum, int B, int64_t x) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cum[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(kPrepThreads) void prep_ragged_kernel(PrepRaggedArgs a) {
  __shared__ int32_t cs[kPrepMaxReq + 1];
  __shared__ int32_t cq[kPrepMaxReq + 1];
  __shared__ int32_t wsum[2][kPrepThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = a.B;
  const int per = (B + kPrepThreads - 1) / kPrepThreads;

  // per-thread sums over a contiguous run of requests
  int32_t s_loc = 0, q_loc = 0;
  for (int i = 0; i < per; ++i) {
    const int b = tid * per + i;
    if (b < B) {
      const int32_t s = max(a.seq_len[b], 0);
      s_loc += s;
      q_loc += min(max(a.q_len[b], 0), s);
    }
  }
  // exclusive scan over the workgroup
  int32_t s_inc = s_loc, q_inc = q_loc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t ts = __shfl_up(s_inc, o), tq = __shfl_up(q_inc, o);
    if (lane >= o) {
      s_inc += ts;
      q_inc += tq;
    }
  }
  if (lane == 63) {
    wsum[0][wave] = s_inc;
    wsum[1][wave] = q_inc;
  }
  __syncthreads();
  int32_t s_run = s_inc - s_loc, q_run = q_inc - q_loc;
  for (int w = 0; w < wave; ++w) {
    s_run += wsum[0][w];
    q_run += wsum[1][w];
  }
  for (int i = 0; i < per; ++i) {
    const int b = tid * per + i;
    if (b < B) {
      const int32_t s = max(a.seq_len[b], 0);
      cs[b] = s_run;
      cq[b] = q_run;
      s_run += s;
      q_run += min(max(a.q_len[b], 0), s);
    }
  }
  if (tid == kPrepThreads - 1) {
    cs[B] = s_run;
    cq[B] = q_run;
  }
  __syncthreads();
  const int64_t total_s = cs[B], total_q = cq[B];

  if (blockIdx.x == 0) {
    for (int b = tid; b <= B; b += kPrepThreads) {
      a.cu_seq[b] = cs[b];
      a.cu_q[b] = cq[b];
    }
  }
  const int64_t gtid = (int64_t)blockIdx.x * kPrepThreads + tid;
  const int64_t gstride = (int64_t)gridDim.x * kPrepThreads;

  // query windows
  const int64_t nq = min(total_q, a.max_q);
  for (int64_t i = gtid; i < nq; i += gstride) {
    const int b = find_request(cq, B, i);
    const int32_t t = (int32_t)(i - cq[b]);
    const int32_t s_b = cs[b + 1] - cs[b], q_b = cq[b + 1] - cq[b];
    a.ks[i] = cs[b];
    a.ke[i] = cs[b] + s_b - q_b + t + 1;
  }

  // ragged memory indices, four consecutive keys per thread
  if (a.ragged_mem) {
    const int64_t nk = min(total_s, a.max_keys);
    for (int64_t u = gtid; u * 4 < nk; u += gstride) {
      const int64_t j0 = u * 4;
      int b = find_request(cs, B, j0);
      const int32_t r0 = a.req_idx[b];
      const int64_t p0 = j0 - cs[b];
      if (j0 + 4 <= min(nk, (int64_t)cs[b + 1]) && r0 >= 0 && r0 < a.num_rows && p0 + 4 <= a.ld_table) {
        // common case: the four keys are one request's, inside its table row
        const int32_t* src = a.table + (int64_t)r0 * a.ld_table + p0;
        const v4i v = {src[0], src[1], src[2], src[3]};
        *reinterpret_cast<v4i*>(a.ragged_mem + j0) = v;
        continue;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t j = j0 + e;
        if (j < nk) {
          while (j >= cs[b + 1]) ++b;   // empty requests have cs[b] == cs[b + 1]
          const int64_t p = j - cs[b];
          const int32_t r = a.req_idx[b];
          int32_t v = -1;
          if (r >= 0 && r < a.num_rows && p < a.ld_table) v = a.table[(int64_t)r * a.ld_table + p];
          a.ragged_mem[j] = v;
        }
      }
    }
  }
}

// Grid: (request, slice of kPrepDecodePages pages of its block-table row).
constexpr int kPrepDecodePages = 1024;

__global__ __launch_bounds__(kPrepThreads) void prep_decode_kernel(PrepDecodeArgs a) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  if (blockIdx.y == 0) {
    const int32_t s = a.seq_len[b];
    for (int t = tid; t < a.next_n; t += kPrepThreads)
      a.row_len[(int64_t)b * a.next_n + t] = max(0, s - a.next_n + t + 1);
  }
  const int32_t r = a.req_idx[b];
  const bool ok = r >= 0 && r < a.num_rows;
  const int32_t* src = a.req_to_page + (int64_t)(ok ? r : 0) * a.ld_r2p;
  int32_t* dst = a.block_table + (int64_t)b * a.ld_bt;
  const int p_hi = min(a.max_pages, (int)(blockIdx.y + 1) * kPrepDecodePages);
  for (int p = blockIdx.y * kPrepDecodePages + tid; p < p_hi; p += kPrepThreads) dst[p] = ok ? src[p] : -1;
}

hipError_t launch_prep_ragged(const PrepRaggedArgs& a, const DeviceInfo& dev, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  const int64_t work = std::max<int64_t>(a.max_q, a.ragged_mem ? (a.max_keys + 3) / 4 : 0);
  int64_t blocks = std::max<int64_t>(1, (work + kPrepThreads - 1) / kPrepThreads);
  // enough workgroups to fill the device a few times over; each one rescans the lengths
  blocks = std::min<int64_t>(blocks, (int64_t)(dev.cu_count > 0 ? dev.cu_count : 256) * 8);
  hipLaunchKernelGGL(prep_ragged_kernel, dim3((unsigned)blocks), dim3(kPrepThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prep_decode(const PrepDecodeArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  const int slices = std::max(1, (a.max_pages + kPrepDecodePages - 1) / kPrepDecodePages);
  if (slices > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prep_decode_kernel, dim3((unsigned)a.B, (unsigned)slices), dim3(kPrepThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace fp8idx
