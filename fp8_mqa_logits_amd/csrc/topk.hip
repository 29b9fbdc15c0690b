// Per-row top-k over float32 logits with an index map, for gfx950
// (the `fast_topk_transform_fused(score, lengths, page_table_size_1,
// cu_seqlens_q, topk, row_starts)` step of the indexer loop on the
// bench_mqa_logits_chunking.py page).
//
// Selection rule: the k largest logits of the row's window [ks, ke), ties at
// the k-th value going to the lower key index, so the selected set is unique.
//
// Algorithm (exact radix select on order-preserving keys):
// - Each workgroup owns one segment of one row: up to THREADS * VPT elements,
//   loaded once with coalesced loads and kept in VGPRs as uint32 keys that
//   sort like the floats (-0.0 folded onto +0.0; key 0 marks padding).
//   Wave w holds positions [w * 64 * VPT, (w + 1) * 64 * VPT), so
//   (wave, register, lane) order is position order.
// - Candidate threshold: one key register in 16 forms a strided sample; the
//   sample key of rank ~1.25 * k * (sample / segment) + 16 becomes a lower
//   threshold T.  A popcount pass counts the keys >= T; when they number at
//   least k (and fit the LDS list) a second pass compacts them into LDS in
//   position order, using wave ballots and per-wave offsets.  Segments that
//   fit the list whole skip the sample (T = every key).
// - Exact selection on the candidates: the bits shared by T and the maximum
//   are fixed; the rest are resolved 11 at a time, most significant first,
//   with an LDS histogram and a suffix scan per digit.  This yields the exact
//   k-th key tau and the number of elements equal to tau still to take.
// - Emission: each thread walks a contiguous run of the ordered candidates;
//   an exclusive scan over threads gives output slots, so elements above
//   tau plus the lowest-positioned elements equal to tau are written in
//   ascending position order and the output is deterministic.
// - If the sample misjudges (fewer than k candidates, or too many for LDS),
//   the same exact selection runs over every key in registers instead.
// - Rows longer than one segment are split: each segment emits its local
//   top-k (key, index) candidates in position order, and further levels of
//   the same kernel select from the concatenated candidates.  Because the
//   rule is a total order (value desc, index asc), a row's top-k is always
//   contained in the union of its segments' top-k.
// - The last level maps each selected key index through the token table
//   (page size 1: table[req(i), j - ks[i]]) or the block table
//   (table[b, j / page] * page + j % page), or writes j itself.

#include "device_common.hpp"
#include "launch.hpp"

#include <fp8idx.h>

#include <algorithm>

namespace fp8idx {

struct TopkKernelArgs {
  const float* logits;
  int64_t ld;
  const int32_t* ks;
  const int32_t* ke;
  int32_t width;
  const uint32_t* in_keys;
  const int32_t* in_idx;
  int64_t in_len;
  int32_t seg_len;
  int32_t nseg;
  int32_t k;
  int32_t* out;
  int64_t ld_out;
  uint32_t* out_keys;
  int32_t* out_idx;
  int32_t row0;
  TopkMap map;
};

constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;
constexpr int kCandCap = 8192;      // capacity of the LDS candidate list
constexpr int kSampleStride = 16;   // one key register in 16 feeds the threshold sample

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += (uint32_t)__shfl_xor((int)v, o);
  return v;
}

__device__ __forceinline__ int32_t map_index(const TopkMap& m, int req, int row_ks, int32_t j) {
  if (m.kind == FP8IDX_MAP_TOKEN_TABLE) {
    const int64_t pos = (int64_t)j - row_ks;
    if (req < 0 || pos < 0 || pos >= m.ld) return -1;
    return m.table[(int64_t)req * m.ld + pos];
  }
  if (m.kind == FP8IDX_MAP_BLOCK_TABLE) {
    const int64_t p = j / m.page_size;
    if (req < 0 || p >= m.ld) return -1;
    const int32_t page = m.table[(int64_t)req * m.ld + p];
    if (page < 0) return -1;
    return page * m.page_size + (j - (int32_t)p * m.page_size);
  }
  return j;
}

// Request of a global row under the map (uniform per workgroup).
__device__ __forceinline__ int map_request(const TopkMap& m, int grow) {
  if (m.kind == FP8IDX_MAP_TOKEN_TABLE) {
    if (m.cu_rows == nullptr) return 0;
    // largest r in [0, num_req) with cu_rows[r] <= grow
    int lo = 0, hi = m.num_req - 1;
    if (grow < m.cu_rows[0] || grow >= m.cu_rows[m.num_req]) return -1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (m.cu_rows[mid] <= grow) lo = mid; else hi = mid - 1;
    }
    return lo;
  }
  if (m.kind == FP8IDX_MAP_BLOCK_TABLE) {
    const int b = grow / m.rows_per_req;
    return b < m.num_req ? b : -1;
  }
  return 0;
}

// LDS of one workgroup: digit histogram, the ordered candidate list and
// small per-wave scratch for reductions and scans.
template <int NW>
struct TopkShared {
  uint32_t hist[kBins];
  uint32_t ck[kCandCap];   // candidate keys, in position order
  uint32_t cp[kCandCap];   // candidate positions within the segment
  uint32_t w0[NW];
  uint32_t w1[NW];
  uint32_t w2[NW];
  uint32_t digit;
  uint32_t above;
};

// Exact rank-th largest key (1 <= rank <= count) of a multiset of keys spread
// over the workgroup, all inside [lo, hi].  for_each(visit) calls visit(key)
// on each of the calling thread's keys.  On return `need` holds how many
// elements equal to the result belong to the rank largest.  The bits shared
// by lo and hi are fixed up front; the rest are resolved 11 at a time, most
// significant first, with an LDS histogram and a suffix scan per digit.
template <int THREADS, typename ForEach>
__device__ uint32_t radix_select(ForEach for_each, uint32_t lo, uint32_t hi, uint32_t rank, uint32_t& need,
                                 TopkShared<THREADS / 64>& sh) {
  constexpr int NW = THREADS / 64;
  constexpr int DPT = kBins / THREADS;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  need = rank;
  if (lo == hi) return hi;
  const int hb = 31 - __builtin_clz(lo ^ hi);
  uint32_t pmask = hb == 31 ? 0u : ~((2u << hb) - 1u);
  uint32_t prefix = hi & pmask;
  int top = hb;
  while (top >= 0) {
    const int shift = max(0, top - (kDigitBits - 1));
    const uint32_t dmask = (2u << (top - shift)) - 1u;
#pragma unroll
    for (int i = 0; i < DPT; ++i) sh.hist[tid * DPT + i] = 0u;
    __syncthreads();
    for_each([&](uint32_t v) {
      if ((v & pmask) == prefix) atomicAdd(&sh.hist[(v >> shift) & dmask], 1u);
    });
    __syncthreads();
    uint32_t mine[DPT];
    uint32_t st = 0u;
#pragma unroll
    for (int i = 0; i < DPT; ++i) {
      mine[i] = sh.hist[tid * DPT + i];
      st += mine[i];
    }
    uint32_t incl = st;   // suffix sum over this and higher lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t v = (uint32_t)__shfl_down((int)incl, o);
      if (lane + o < 64) incl += v;
    }
    if (lane == 0) sh.w0[wave] = incl;
    __syncthreads();
    uint32_t above = incl - st;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (w > wave) above += sh.w0[w];
    if (above < need && need <= above + st) {
      uint32_t acc = above;
#pragma unroll
      for (int i = DPT - 1; i >= 0; --i) {
        if (acc < need && acc + mine[i] >= need) {
          sh.digit = (uint32_t)(tid * DPT + i);
          sh.above = acc;
        }
        acc += mine[i];
      }
    }
    __syncthreads();
    need -= sh.above;
    prefix |= sh.digit << shift;
    pmask |= dmask << shift;
    top = shift - 1;
  }
  return prefix;
}

// Block-wide reduction of (max, min, sum) over the workgroup.
template <int NW>
__device__ void block_max_min_sum(uint32_t& mx, uint32_t& mn, uint32_t& sm, TopkShared<NW>& sh) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  mx = wave_max_u32(mx);
  mn = wave_min_u32(mn);
  sm = wave_sum_u32(sm);
  __syncthreads();   // earlier readers of w0..w2 are done
  if (lane == 0) {
    sh.w0[wave] = mx;
    sh.w1[wave] = mn;
    sh.w2[wave] = sm;
  }
  __syncthreads();
  mx = 0u;
  mn = 0xffffffffu;
  sm = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mx = max(mx, sh.w0[w]);
    mn = min(mn, sh.w1[w]);
    sm += sh.w2[w];
  }
}

// Exclusive prefix sums over threads (thread order) of two per-thread counts.
template <int NW>
__device__ void block_excl_scan2(uint32_t a, uint32_t b, uint32_t& a_before, uint32_t& b_before,
                                 TopkShared<NW>& sh) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t ia = a, ib = b;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t ta = (uint32_t)__shfl_up((int)ia, o);
    const uint32_t tb = (uint32_t)__shfl_up((int)ib, o);
    if (lane >= o) {
      ia += ta;
      ib += tb;
    }
  }
  __syncthreads();
  if (lane == 63) {
    sh.w0[wave] = ia;
    sh.w1[wave] = ib;
  }
  __syncthreads();
  a_before = ia - a;
  b_before = ib - b;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w < wave) {
      a_before += sh.w0[w];
      b_before += sh.w1[w];
    }
  }
}

template <bool LEVEL0, bool FINAL>
struct Emitter {
  const TopkKernelArgs& a;
  int64_t sa;
  int64_t row;
  int64_t out_base;
  int req;
  int row_ks;
  __device__ __forceinline__ void operator()(uint32_t o, uint32_t pos, uint32_t key) const {
    int32_t j;
    if (LEVEL0) j = (int32_t)(sa + pos);
    else j = a.in_idx[row * a.in_len + sa + pos];
    if (FINAL) {
      a.out[out_base + o] = map_index(a.map, req, row_ks, j);
    } else {
      a.out_keys[out_base + o] = key;
      a.out_idx[out_base + o] = j;
    }
  }
};

template <int THREADS, int VPT, bool LEVEL0, bool FINAL>
__global__ __launch_bounds__(THREADS) void topk_kernel(TopkKernelArgs a) {
  constexpr int NW = THREADS / 64;
  static_assert(kBins % THREADS == 0, "bins per thread");
  __shared__ TopkShared<NW> sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row = blockIdx.x / a.nseg;
  const int seg = blockIdx.x - row * a.nseg;

  // ---- segment window -------------------------------------------------------
  int row_ks = 0;
  int64_t sa = 0;
  int len = 0;
  if (LEVEL0 || FINAL) {
    const int e = min(max(a.ke[row], 0), a.width);
    row_ks = a.ks ? min(max(a.ks[row], 0), e) : 0;
    if (LEVEL0) {
      sa = (int64_t)row_ks + (int64_t)seg * a.seg_len;
      len = (int)max((int64_t)0, min((int64_t)a.seg_len, (int64_t)e - sa));
    }
  }
  if (!LEVEL0) {
    sa = (int64_t)seg * a.seg_len;
    len = (int)max((int64_t)0, min((int64_t)a.seg_len, a.in_len - sa));
  }

  // ---- load keys into VGPRs -------------------------------------------------
  // Loads are unconditional from a clamped in-bounds position (len >= 1);
  // positions past the segment are then replaced by the padding key 0.
  uint32_t key[VPT];
  const int base = wave * (64 * VPT) + lane;
  const int last = max(len - 1, 0);
  if (len == 0) {
#pragma unroll
    for (int p = 0; p < VPT; ++p) key[p] = 0u;
  } else if (LEVEL0) {
    const float* src = a.logits + (int64_t)row * a.ld + sa;
    // all VPT loads are issued before any is consumed: the padding mask is
    // applied arithmetically so no load sits under a branch
#pragma unroll
    for (int p = 0; p < VPT; ++p) key[p] = __float_as_uint(__builtin_nontemporal_load(src + min(base + p * 64, last)));
#pragma unroll
    for (int p = 0; p < VPT; ++p) {
      const uint32_t keep = 0u - (uint32_t)(base + p * 64 < len);
      key[p] = max(float_to_ordered(__uint_as_float(key[p])), 1u) & keep;
    }
  } else {
    const uint32_t* src = a.in_keys + (int64_t)row * a.in_len + sa;
#pragma unroll
    for (int p = 0; p < VPT; ++p) key[p] = src[min(base + p * 64, last)];
#pragma unroll
    for (int p = 0; p < VPT; ++p) key[p] &= 0u - (uint32_t)(base + p * 64 < len);
  }

  // ---- valid count, min and max ---------------------------------------------
  uint32_t kmax = 0u, kmin = 0xffffffffu, cnt = 0u;
#pragma unroll
  for (int p = 0; p < VPT; ++p) {
    const uint32_t v = key[p];
    if (v != 0u) {
      kmax = max(kmax, v);
      kmin = min(kmin, v);
      ++cnt;
    }
  }
  block_max_min_sum<NW>(kmax, kmin, cnt, sh);
  const uint32_t kk = min((uint32_t)a.k, cnt);

  const int64_t out_base = FINAL ? (int64_t)row * a.ld_out : ((int64_t)row * a.nseg + seg) * (int64_t)a.k;
  Emitter<LEVEL0, FINAL> emit{a, sa, row, out_base, FINAL ? map_request(a.map, a.row0 + row) : 0, row_ks};

  if (kk > 0u) {
    // ---- candidate threshold T from a strided sample ---------------------------
    // Target: about 1.25 * kk + 16 sample-strides of elements at or above T, so
    // that the exact k-th key is almost always among the candidates.
    uint32_t T = 1u;   // 1 = every valid key
    if (cnt > (uint32_t)kCandCap) {
      uint32_t smax = 0u, smin = 0xffffffffu, ns = 0u;
#pragma unroll
      for (int p = 0; p < VPT; p += kSampleStride) {
        const uint32_t v = key[p];
        if (v != 0u) {
          smax = max(smax, v);
          smin = min(smin, v);
          ++ns;
        }
      }
      block_max_min_sum<NW>(smax, smin, ns, sh);
      const uint64_t want = ((uint64_t)kk * ns * 5u + 4ull * cnt - 1u) / (4ull * cnt) + 16u;
      if (ns > 0u && want < ns) {
        uint32_t unused;
        T = radix_select<THREADS>(
            [&](auto&& visit) {
#pragma unroll
              for (int p = 0; p < VPT; p += kSampleStride)
                if (key[p] != 0u) visit(key[p]);
            },
            smin, smax, (uint32_t)want, unused, sh);
      }
    }

    // ---- count candidates (keys >= T) per wave --------------------------------
    uint32_t cw = 0u;
#pragma unroll
    for (int p = 0; p < VPT; ++p) cw += (uint32_t)__popcll(ballot64(key[p] >= T));
    __syncthreads();
    if (lane == 0) sh.w2[wave] = cw;
    __syncthreads();
    uint32_t C = 0u, woff = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t x = sh.w2[w];
      if (w < wave) woff += x;
      C += x;
    }

    if (C >= kk && C <= (uint32_t)kCandCap) {
      // ---- ordered compaction of the candidates into LDS -----------------------
      uint32_t off = woff;
#pragma unroll
      for (int p = 0; p < VPT; ++p) {
        const bool c = key[p] >= T;
        const uint64_t b = ballot64(c);
        if (c) {
          const uint32_t o = off + mbcnt64(b);
          sh.ck[o] = key[p];
          sh.cp[o] = (uint32_t)(base + p * 64);
        }
        off += (uint32_t)__popcll(b);
      }
      __syncthreads();
      // ---- exact threshold among the candidates --------------------------------
      uint32_t need;
      const uint32_t tau = radix_select<THREADS>(
          [&](auto&& visit) {
            for (uint32_t i = tid; i < C; i += THREADS) visit(sh.ck[i]);
          },
          T, kmax, kk, need, sh);
      // ---- emission in position order ------------------------------------------
      const uint32_t per = (C + THREADS - 1) / THREADS;
      const uint32_t c0 = min(C, (uint32_t)tid * per);
      const uint32_t c1 = min(C, c0 + per);
      uint32_t gt = 0u, eq = 0u;
      for (uint32_t i = c0; i < c1; ++i) {
        const uint32_t v = sh.ck[i];
        gt += v > tau;
        eq += v == tau;
      }
      uint32_t gt_before, eq_before;
      block_excl_scan2<NW>(gt, eq, gt_before, eq_before, sh);
      uint32_t run_eq = eq_before;
      uint32_t run_sel = gt_before + min(eq_before, need);
      for (uint32_t i = c0; i < c1; ++i) {
        const uint32_t v = sh.ck[i];
        bool sel = v > tau;
        if (v == tau) {
          sel = run_eq < need;
          ++run_eq;
        }
        if (sel) {
          emit(run_sel, sh.cp[i], v);
          ++run_sel;
        }
      }
    } else {
      // ---- fallback: exact select over every key in registers -------------------
      uint32_t need;
      const uint32_t tau = radix_select<THREADS>(
          [&](auto&& visit) {
#pragma unroll
            for (int p = 0; p < VPT; ++p)
              if (key[p] != 0u) visit(key[p]);
          },
          kmin, kmax, kk, need, sh);
      uint32_t gt = 0u, eq = 0u;
#pragma unroll
      for (int p = 0; p < VPT; ++p) {
        gt += (uint32_t)__popcll(ballot64(key[p] > tau));
        eq += (uint32_t)__popcll(ballot64(key[p] == tau));
      }
      __syncthreads();
      if (lane == 0) {
        sh.w0[wave] = gt;
        sh.w1[wave] = eq;
      }
      __syncthreads();
      uint32_t gt_before = 0u, eq_before = 0u;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        if (w < wave) {
          gt_before += sh.w0[w];
          eq_before += sh.w1[w];
        }
      }
      uint32_t run_eq = eq_before;
      uint32_t run_sel = gt_before + min(eq_before, need);
#pragma unroll
      for (int p = 0; p < VPT; ++p) {
        const uint32_t v = key[p];
        const bool is_gt = v > tau;
        const bool is_eq = v == tau;
        const uint64_t beq = ballot64(is_eq);
        const bool sel = is_gt || (is_eq && (run_eq + mbcnt64(beq)) < need);
        const uint64_t bsel = ballot64(sel);
        if (sel) emit(run_sel + mbcnt64(bsel), (uint32_t)(base + p * 64), v);
        run_eq += (uint32_t)__popcll(beq);
        run_sel += (uint32_t)__popcll(bsel);
      }
    }
  }
  // padding after the kk selected entries
  for (int o = (int)kk + tid; o < a.k; o += THREADS) {
    if (FINAL) {
      a.out[out_base + o] = -1;
    } else {
      a.out_keys[out_base + o] = 0u;
      a.out_idx[out_base + o] = -1;
    }
  }
}

// ---- host-side plan and launch ----------------------------------------------

struct TopkCfg {
  int threads;
  int vpt;
  int cap;
};
constexpr TopkCfg kTopkCfgs[] = {{256, 16, 4096}, {512, 32, 16384}, {512, 64, 32768}, {512, 128, 65536}};
constexpr int kNumTopkCfgs = 4;
constexpr int64_t kMaxSeg = 65536;

static int pick_cfg(int64_t seg_len) {
  for (int c = 0; c < kNumTopkCfgs; ++c)
    if (seg_len <= kTopkCfgs[c].cap) return c;
  return kNumTopkCfgs - 1;
}

TopkPlan plan_topk(int32_t rows, int64_t width, int32_t k) {
  TopkPlan p{};
  p.buf_bytes[0] = p.buf_bytes[1] = 0;
  int64_t in_len = width > 0 ? width : 1;
  const int64_t target_wgs = 1024;
  const int64_t min_seg = std::max<int64_t>(4 * (int64_t)k, 4096);
  for (int lvl = 0; lvl < kMaxTopkLevels; ++lvl) {
    int64_t nseg = (in_len + kMaxSeg - 1) / kMaxSeg;
    if (lvl == 0 && in_len > min_seg && rows > 0 && rows < target_wgs) {
      const int64_t want = std::min<int64_t>((target_wgs + rows - 1) / rows, in_len / min_seg);
      nseg = std::max<int64_t>(nseg, want);
    }
    int64_t seg_len = (in_len + nseg - 1) / nseg;
    seg_len = std::min<int64_t>(seg_len, kMaxSeg);
    nseg = (in_len + seg_len - 1) / seg_len;
    TopkLevel& L = p.level[lvl];
    L.in_len = in_len;
    L.seg_len = (int32_t)seg_len;
    L.nseg = (int32_t)nseg;
    L.cfg = pick_cfg(seg_len);
    p.nlevels = lvl + 1;
    if (nseg == 1) break;
    const int64_t out_len = nseg * (int64_t)k;
    const size_t bytes = (size_t)rows * (size_t)out_len * 8u;
    p.buf_bytes[lvl & 1] = std::max(p.buf_bytes[lvl & 1], bytes);
    in_len = out_len;
  }
  return p;
}

static size_t align256(size_t x) { return (x + 255u) & ~(size_t)255u; }

size_t topk_workspace_bytes(const TopkPlan& p) {
  size_t total = 0;
  for (int b = 0; b < 2; ++b)
    if (p.buf_bytes[b]) total += align256(p.buf_bytes[b]);
  return total;
}

template <int THREADS, int VPT>
static void launch_cfg(bool level0, bool final_level, unsigned grid, const TopkKernelArgs& a, hipStream_t s) {
  if (level0 && final_level)
    hipLaunchKernelGGL((topk_kernel<THREADS, VPT, true, true>), dim3(grid), dim3(THREADS), 0, s, a);
  else if (level0)
    hipLaunchKernelGGL((topk_kernel<THREADS, VPT, true, false>), dim3(grid), dim3(THREADS), 0, s, a);
  else if (final_level)
    hipLaunchKernelGGL((topk_kernel<THREADS, VPT, false, true>), dim3(grid), dim3(THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((topk_kernel<THREADS, VPT, false, false>), dim3(grid), dim3(THREADS), 0, s, a);
}

hipError_t launch_topk(const TopkArgs& ta, const TopkPlan& plan, void* ws, hipStream_t s) {
  if (ta.rows <= 0) return hipSuccess;
  uint8_t* bufs[2] = {nullptr, nullptr};
  {
    uint8_t* w = static_cast<uint8_t*>(ws);
    size_t off = 0;
    for (int b = 0; b < 2; ++b) {
      if (plan.buf_bytes[b]) {
        bufs[b] = w + off;
        off += align256(plan.buf_bytes[b]);
      }
    }
  }
  for (int lvl = 0; lvl < plan.nlevels; ++lvl) {
    const TopkLevel& L = plan.level[lvl];
    const bool level0 = lvl == 0;
    const bool final_level = lvl == plan.nlevels - 1;
    TopkKernelArgs a{};
    a.logits = ta.logits;
    a.ld = ta.ld;
    a.ks = ta.ks;
    a.ke = ta.ke;
    a.width = ta.width;
    a.seg_len = L.seg_len;
    a.nseg = L.nseg;
    a.k = ta.k;
    a.row0 = ta.row0;
    a.map = ta.map;
    if (!level0) {
      const uint8_t* src = bufs[(lvl - 1) & 1];
      const int64_t n_in = (int64_t)ta.rows * L.in_len;
      a.in_keys = reinterpret_cast<const uint32_t*>(src);
      a.in_idx = reinterpret_cast<const int32_t*>(src + (size_t)n_in * 4u);
      a.in_len = L.in_len;
    }
    if (final_level) {
      a.out = ta.out;
      a.ld_out = ta.ld_out;
    } else {
      uint8_t* dst = bufs[lvl & 1];
      const int64_t n_out = (int64_t)ta.rows * L.nseg * ta.k;
      a.out_keys = reinterpret_cast<uint32_t*>(dst);
      a.out_idx = reinterpret_cast<int32_t*>(dst + (size_t)n_out * 4u);
    }
    const int64_t grid = (int64_t)ta.rows * L.nseg;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    switch (L.cfg) {
      case 0: launch_cfg<256, 16>(level0, final_level, (unsigned)grid, a, s); break;
      case 1: launch_cfg<512, 32>(level0, final_level, (unsigned)grid, a, s); break;
      case 2: launch_cfg<512, 64>(level0, final_level, (unsigned)grid, a, s); break;
      default: launch_cfg<512, 128>(level0, final_level, (unsigned)grid, a, s); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace fp8idx
