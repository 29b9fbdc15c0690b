// Per-row top-k over float32 logits with an index map, for gfx950
// (the `fast_topk_transform_fused(score, lengths, page_table_size_1,
// cu_seqlens_q, topk, row_starts)` step of the indexer loop on the
// bench_mqa_logits_chunking.py page).
//
// Selection rule: the k largest logits of the row's window [ks, ke), ties at
// the k-th value going to the lower key index, so the selected set is unique.
// Keys are compared as order-preserving uint32 codes of the floats (-0.0 is
// folded onto +0.0; code 0 marks padding).
//
// Algorithm: one workgroup of 256 threads per (row, segment of at most 70016
// keys), streaming the segment from memory; nothing is held per key in
// registers, so several workgroups share a CU and their loads overlap each
// other's selection work.
// 1. Threshold: 16 runs of 256 consecutive keys, spread evenly over the
//    segment, form a sample; a radix search over the sample, stopped once
//    the bin in question holds at most 16 sample keys, gives a lower
//    threshold T near the sample rank 1.3 * k * (sample / segment) + 16 (a
//    segment that fits the LDS candidate list whole takes every key).
// 2. Compaction: one streaming pass with 16-byte loads appends every key >= T
//    (about 1.3 k of them) as a (code, position) pair to an LDS list; each
//    wave claims its slots with one LDS atomic per 32 keys a lane examined,
//    while the next 32 keys per lane are already loading.  The list order
//    depends on timing.
// 3. Boundary bin: a 2048-bin histogram of the list between T and the sample
//    maximum locates the bin of the k-th largest code; every candidate in a
//    higher bin is selected, and the few in that bin are ranked pairwise by
//    (value desc, position asc), which settles the k-th value and its ties
//    in one step.  (If that bin holds more than 256 candidates, e.g. under
//    heavy ties, an exact radix search over the list finds the k-th code
//    tau, and the ties at tau are ranked by position through an LDS bitmap
//    with per-word prefix popcounts.)
// 4. Order: the positions of the selected keys are set in an LDS bitmap, and
//    each key's output slot is its rank by position (prefix popcount).  The
//    output row is the selected keys in ascending position order, identical
//    on every run.
// If the sample misjudges (fewer than k candidates, or more than fit), the
// same exact selection and ordering run over every key of the segment,
// streamed from memory once per step.
// Few long rows (at most 512 rows of at most 131072 keys, k up to about
// 2300: paged decode) take one 512-thread workgroup per whole row instead:
// twice the loads in flight of a 256-thread segment, a single launch and no
// merge level (position bitmaps sized for 131072 keys, one workgroup per CU).
// In the fused paged entry the logits kernel also hands over each row's
// largest key code per 16-key fragment.  The kk-th largest fragment maximum T
// is at most the kk-th largest key (at least kk fragments, hence kk keys,
// reach it), and every key >= T sits in a fragment whose maximum reaches T:
// so a row of at least 1.5 kk fragments lists the fragments >= T, reads only
// those (four lanes per 64-byte fragment), and keeps their keys >= T.  On the
// decode rows that is about a quarter of the fragments and 1.15-1.75 kk
// candidates; a list that would overflow falls back to the sampled path.
// Other rows longer than one segment, or few rows that need more parallelism, are
// split: each segment emits its local top-k (code, index) pairs in index
// order, and further levels of the same kernel select from the concatenated
// pairs (still in index order, so position order is index order).  Because
// the rule is a total order (value desc, index asc), a row's top-k is always
// contained in the union of its segments' top-k.  The last level maps each
// selected key index through the token table (page size 1:
// table[req(i), j - ks[i]]) or the block table (table[b, j / page] * page +
// j % page), or writes j itself.

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
  const uint32_t* frag_max;   // per (row, 16-key fragment) largest key code, or null
  FragLayout frag;            // its layout (launch.hpp)
  int32_t frag_next_n;        // rows per request of the logits launch that wrote it
};

constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;
// Keys per segment: the largest whose bitmaps keep the workgroup's LDS at three per CU (52 KB).
constexpr int64_t kMaxSeg = 70016;
// Position bitmap words of a segment of up to `seg` keys (positions count from the 16-byte load base).
constexpr int bitmap_words(int64_t seg) { return (int)((seg + 4 + 31) / 32) + 1; }
constexpr int kBitmapWords = bitmap_words(kMaxSeg);
constexpr int kTopkThreads = 256;
constexpr int kSampleRuns = 16;
// Few long rows: one wide workgroup per whole row (no merge level).
constexpr int kWideThreads = 512;
constexpr int64_t kWideSeg = 131072;
constexpr int kWideRowsMax = 512;
constexpr int kElemsPerPass = 32;   // keys a thread loads per streaming pass
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

// Candidate-list capacity for k: the expected list (1.3 k + 24 sample units
// of keys, at most 384 keys) must stay under 7/8 of it.
constexpr int kSmallCap = 4096;
constexpr int kBigCap = 16384;
inline bool topk_needs_big_cap(int64_t k) { return k * 13 / 10 + 512 > (int64_t)kSmallCap * 7 / 8; }

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

__device__ __forceinline__ int32_t map_index(const TopkMap m, int req, int row_ks, int32_t j) {
  if (m.kind == FP8IDX_MAP_TOKEN_TABLE) {
    const int64_t pos = (int64_t)j - row_ks;
    if (req < 0 || pos < 0 || pos >= m.ld) return -1;
    return m.table[(int64_t)req * m.ld + pos];
  }
  if (m.kind == FP8IDX_MAP_BLOCK_TABLE) {
    const int64_t p = j / m.page_size;
    if (req < 0 || p >= m.ld) return -1;
    const int32_t page = m.table[(int64_t)req * m.ld + p];
    if (page < 0 || page >= m.num_pages) return -1;
    return page * m.page_size + (j - (int32_t)p * m.page_size);
  }
  return j;
}

// Request of a global row under the map (uniform per workgroup).
__device__ __forceinline__ int map_request(const TopkMap m, int grow) {
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

// LDS of one workgroup of NW waves with a CAP-entry candidate list and WORDS-word position bitmaps.
// A boundary bin of up to NW * 64 candidates (one per thread) is ranked pairwise.
template <int NW, int CAP, int WORDS>
struct TopkShared {
  static constexpr int kWords = WORDS;
  static constexpr int kBoundaryMax = NW * 64;
  v2u cand[(CAP > WORDS ? CAP : WORDS) + 1];   // candidates (code, position); bitmaps in the fallback;
                                               // [CAP] absorbs appends past the end (the count grows)
  uint32_t hist[WORDS];             // digit histogram, later per-word prefix popcounts
  uint32_t bits[WORDS];             // position bitmap
  uint32_t bk[kBoundaryMax];        // codes of the candidates in the boundary bin
  uint32_t bp[kBoundaryMax];        // and their positions
  uint32_t w0[NW];
  uint32_t w1[NW];
  uint32_t w2[NW];
  uint32_t cnt;
  uint32_t nfrag_listed;            // fragments reaching the threshold (fragment-maximum path)
  uint32_t nb;
  uint32_t digit;
  uint32_t above;
  uint32_t dcount;
};

// Bin of sh.hist[0, kBins) that holds the need-th largest element (1 <= need
// <= total), with the number of elements in higher bins (above) and in the
// bin itself (count).  Ends with a barrier.
template <int THREADS, typename Shared>
__device__ __forceinline__ void pick_bin(uint32_t need, uint32_t& bin, uint32_t& above, uint32_t& count,
                         Shared& sh) {
  constexpr int NW = THREADS / 64;
  constexpr int DPT = kBins / THREADS;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
  uint32_t ab = incl - st;
#pragma unroll
  for (int w = 0; w < NW; ++w)
    if (w > wave) ab += sh.w0[w];
  if (ab < need && need <= ab + st) {
    uint32_t acc = ab;
#pragma unroll
    for (int i = DPT - 1; i >= 0; --i) {
      if (acc < need && acc + mine[i] >= need) {
        sh.digit = (uint32_t)(tid * DPT + i);
        sh.above = acc;
        sh.dcount = mine[i];
      }
      acc += mine[i];
    }
  }
  __syncthreads();
  bin = sh.digit;
  above = sh.above;
  count = sh.dcount;
}

// The rank-th largest code (1 <= rank <= count) of a multiset spread over the
// workgroup, all inside [lo, hi]; for_each(visit) calls visit(code) on each of
// the calling thread's codes.  Bits are resolved 11 at a time from the most
// significant bit where lo and hi differ.  With slack = 0 the result is exact
// and `need` returns how many elements equal to it belong to the rank
// largest.  With slack > 0 the search may stop once the bin holding the rank
// has at most slack elements and return that bin's lowest code: then between
// rank and rank + slack - 1 elements are >= the result (`need` is not set).
template <int THREADS, typename Shared, typename ForEach>
__device__ __forceinline__ uint32_t radix_select(ForEach for_each, uint32_t lo, uint32_t hi, uint32_t rank, uint32_t slack,
                                 uint32_t& need, Shared& sh) {
  constexpr int DPT = kBins / THREADS;
  const int tid = threadIdx.x;
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
    uint32_t digit, above, count;
    pick_bin<THREADS>(need, digit, above, count, sh);
    need -= above;
    prefix |= digit << shift;
    pmask |= dmask << shift;
    top = shift - 1;
    if (count <= slack) break;
  }
  return prefix;
}

template <int NW>
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* w) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_u32(v);
  __syncthreads();
  if (lane == 0) w[wave] = v;
  __syncthreads();
  uint32_t s = 0u;
#pragma unroll
  for (int i = 0; i < NW; ++i) s += w[i];
  return s;
}

// Workgroup min, max and sum in one exchange.
template <int NW>
__device__ __forceinline__ void block_min_max_sum(uint32_t& mn, uint32_t& mx, uint32_t& sm, uint32_t* w0,
                                                  uint32_t* w1, uint32_t* w2) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  sm = wave_sum_u32(sm);
  __syncthreads();
  if (lane == 0) {
    w0[wave] = mn;
    w1[wave] = mx;
    w2[wave] = sm;
  }
  __syncthreads();
  mn = 0xffffffffu;
  mx = 0u;
  sm = 0u;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    mn = min(mn, w0[i]);
    mx = max(mx, w1[i]);
    sm += w2[i];
  }
}

// Exclusive prefix popcounts of bitmap words [0, nwords) into pre[].
template <int THREADS, int WORDS>
__device__ __forceinline__ void bitmap_prefix(const uint32_t* bits, uint32_t* pre, int nwords, uint32_t* w) {
  constexpr int NW = THREADS / 64;
  constexpr int WPT = (WORDS + THREADS - 1) / THREADS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t local[WPT];
  uint32_t sum = 0u;
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int wi = tid * WPT + i;
    local[i] = wi < nwords ? (uint32_t)__popc(bits[wi]) : 0u;
    sum += local[i];
  }
  uint32_t incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t v = (uint32_t)__shfl_up((int)incl, o);
    if (lane >= o) incl += v;
  }
  __syncthreads();
  if (lane == 63) w[wave] = incl;
  __syncthreads();
  uint32_t run = incl - sum;
#pragma unroll
  for (int i = 0; i < NW; ++i)
    if (i < wave) run += w[i];
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int wi = tid * WPT + i;
    if (wi < nwords) pre[wi] = run;
    run += local[i];
  }
  __syncthreads();
}

__device__ __forceinline__ uint32_t bitmap_rank(const uint32_t* bits, const uint32_t* pre, uint32_t pos) {
  const uint32_t w = pos >> 5;
  return pre[w] + (uint32_t)__popc(bits[w] & ((1u << (pos & 31)) - 1u));
}

// The keys of one segment as codes, addressed by position from a load base
// rounded down to VEC elements; valid positions are [off, span).
template <bool LEVEL0, int VEC>
struct SegmentSource {
  const float* f;       // level 0: logits at the load base
  const uint32_t* u;    // other levels: codes at the load base
  int off;
  int span;

  __device__ __forceinline__ static uint32_t float_code(float x) { return max(float_to_ordered(x), 1u); }

  // codes of positions [v * VEC, v * VEC + VEC)
  __device__ __forceinline__ void load(int v, uint32_t* c) const {
    if (LEVEL0) {
      if (VEC == 4) {
        const v4f t = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(f) + v);
#pragma unroll
        for (int i = 0; i < VEC; ++i) c[i] = float_code(t[i]);
      } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) c[i] = float_code(__builtin_nontemporal_load(f + v * VEC + i));
      }
    } else {
      if (VEC == 4) {
        const v4i t = *(reinterpret_cast<const v4i*>(u) + v);
#pragma unroll
        for (int i = 0; i < VEC; ++i) c[i] = (uint32_t)t[i];
      } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) c[i] = u[v * VEC + i];
      }
    }
  }
  // raw keys of positions [v * VEC, v * VEC + VEC): level 0 float bits, other levels codes
  __device__ __forceinline__ void load_raw(int v, uint32_t* c) const {
    if (LEVEL0) {
      if (VEC == 4) {
        const v4i t = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(f) + v);
#pragma unroll
        for (int i = 0; i < VEC; ++i) c[i] = (uint32_t)t[i];
      } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) c[i] = __float_as_uint(__builtin_nontemporal_load(f + v * VEC + i));
      }
    } else {
      load(v, c);
    }
  }
  __device__ __forceinline__ static uint32_t raw_code(uint32_t r) { return LEVEL0 ? float_code(__uint_as_float(r)) : r; }
  __device__ __forceinline__ uint32_t code_at(int pos) const { return LEVEL0 ? float_code(f[pos]) : u[pos]; }
  __device__ __forceinline__ bool valid(int pos) const { return pos >= off && pos < span; }
};

// Appends this lane's candidates among one streaming pass's keys c (raw keys,
// vector v of slot u at v0 + u * THREADS) to the LDS list, at slots claimed
// wave-wide with one LDS atomic.  FAST: every vector lies in the window and a
// key is a candidate when its bits, read as a signed int, reach Ti (level 0
// with the threshold above +0.0); otherwise the general test on codes.
template <bool FAST, int THREADS, int CAP, int UNR, int VEC, bool LEVEL0, typename Shared>
__device__ __forceinline__ void append_candidates(const uint32_t (&c)[UNR][VEC], int v0, int nvec,
                                                  const SegmentSource<LEVEL0, VEC>& src, uint32_t T, int Ti,
                                                  int lane, Shared& sh) {
  auto is_cand = [&](int u, int i) -> bool {
    if (FAST) return (int)c[u][i] >= Ti;
    const int v = v0 + u * THREADS;
    return v < nvec && src.valid(v * VEC + i) && SegmentSource<LEVEL0, VEC>::raw_code(c[u][i]) >= T;
  };
  auto code_of = [](uint32_t r) -> uint32_t {
    return FAST ? (r | 0x80000000u) : SegmentSource<LEVEL0, VEC>::raw_code(r);
  };
  uint32_t mine = 0u;
#pragma unroll
  for (int u = 0; u < UNR; ++u)
#pragma unroll
    for (int i = 0; i < VEC; ++i) mine += is_cand(u, i) ? 1u : 0u;
  uint32_t incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = (uint32_t)__shfl_up((int)incl, o);
    if (lane >= o) incl += t;
  }
  const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
  if (total == 0u) return;
  uint32_t base = 0u;
  if (lane == 63) base = atomicAdd(&sh.cnt, total);
  base = __builtin_amdgcn_readlane(base, 63);
  uint32_t slot = base + incl - mine;
#pragma unroll
  for (int u = 0; u < UNR; ++u)
#pragma unroll
    for (int i = 0; i < VEC; ++i)
      if (is_cand(u, i)) {
        sh.cand[min(slot, (uint32_t)CAP)] = v2u{code_of(c[u][i]), (uint32_t)((v0 + u * THREADS) * VEC + i)};
        ++slot;
      }
}

template <int THREADS, int CAP, int SEG, bool LEVEL0, bool FINAL, int VEC, bool FM = false>
__global__ __launch_bounds__(THREADS) void topk_kernel(TopkKernelArgs a) {
  static_assert(!FM || (LEVEL0 && VEC == 4 && (SEG + 15) / 16 <= kSampleRuns * THREADS),
                "fragment maxima: a window's fragments fit the per-thread sample registers");
  constexpr int NW = THREADS / 64;
  constexpr int UNR = kElemsPerPass / VEC;   // vectors per thread per pass
  static_assert(kBins % THREADS == 0, "bins per thread");
  constexpr int WORDS = bitmap_words(SEG);
  constexpr int kSampleSize = kSampleRuns * THREADS;   // sample runs are one workgroup wide
  constexpr int kBoundaryMax = TopkShared<NW, CAP, WORDS>::kBoundaryMax;
  __shared__ TopkShared<NW, CAP, WORDS> sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int row = blockIdx.x / a.nseg;
  const int seg = blockIdx.x - row * a.nseg;
  // The row's fragment maxima (fragment b * THREADS + tid) load first, beside the window bounds.
  uint32_t fc[FM ? kSampleRuns : 1];
  if constexpr (FM) {
    if (a.frag_max != nullptr) {
      // this row's unit and row slot in the chunk-major layout of the paged logits kernel
      const int nn = a.frag_next_n;
      const int rb = row / nn, rt = row - rb * nn;
      const int64_t base = ((int64_t)rb * ((nn + 3) / 4) + rt / 4) * a.frag.unit_stride + (rt & 3) * a.frag.fpc;
      const int64_t blk = (int64_t)a.frag.rows * a.frag.fpc;
      const int64_t per_row = a.frag.unit_stride / a.frag.rows;   // fragments of a row in the layout
#pragma unroll
      for (int b = 0; b < kSampleRuns; ++b) {
        const int f = b * THREADS + tid;
        const int c = f / a.frag.fpc;
        const int64_t idx = base + c * blk + (f - c * a.frag.fpc);
        fc[b] = f < per_row && idx < a.frag.elems ? a.frag_max[idx] : 0u;
      }
    }
  }

  // ---- segment window --------------------------------------------------------
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
  const int64_t lb = sa & ~(int64_t)(VEC - 1);
  SegmentSource<LEVEL0, VEC> src;
  src.f = LEVEL0 ? a.logits + (int64_t)row * a.ld + lb : nullptr;
  src.u = LEVEL0 ? nullptr : a.in_keys + (int64_t)row * a.in_len + lb;
  src.off = (int)(sa - lb);
  src.span = src.off + len;
  const int nvec = (src.span + VEC - 1) / VEC;

  const int64_t out_base = FINAL ? (int64_t)row * a.ld_out : ((int64_t)row * a.nseg + seg) * (int64_t)a.k;
  const TopkMap map = a.map;
  const int req = FINAL ? map_request(map, a.row0 + row) : 0;
  auto emit = [&](uint32_t slot, uint32_t pos, uint32_t code) {
    int32_t j;
    if (LEVEL0) j = (int32_t)(lb + pos);
    else j = a.in_idx[(int64_t)row * a.in_len + lb + pos];
    if (FINAL) {
      a.out[out_base + slot] = map_index(map, req, row_ks, j);
    } else {
      a.out_keys[out_base + slot] = code;
      a.out_idx[out_base + slot] = j;
    }
  };
  // One pass over the segment: visit(pos, code) for every valid non-padding key.
  auto stream = [&](auto&& visit) {
    for (int vb = 0; vb < nvec; vb += THREADS * UNR) {
      const int v0 = vb + tid;
      uint32_t c[UNR][VEC];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int v = min(v0 + u * THREADS, nvec - 1);
        src.load(v, c[u]);
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int v = v0 + u * THREADS;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const int pos = v * VEC + i;
          if (v < nvec && src.valid(pos) && c[u][i] != 0u) visit(pos, c[u][i]);
        }
      }
    }
  };

  // ---- LDS state of the candidate list ---------------------------------------
  const int nwords = (src.span + 31) / 32;
  for (int wi = tid; wi < nwords; wi += THREADS) sh.bits[wi] = 0u;
  if (tid == 0) {
    sh.cnt = 0u;
    sh.nb = 0u;
    sh.nfrag_listed = 0u;
  }

  // Streaming passes of the compaction below: pass 0 is loaded as soon as the
  // sample's loads are issued, so it arrives while the threshold is chosen.
  constexpr int kPass = THREADS * UNR;
  auto load_pass = [&](int vb, uint32_t (&dst)[UNR][VEC]) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) src.load_raw(min(vb + tid + u * THREADS, nvec - 1), dst[u]);
  };
  uint32_t c[UNR][VEC];
  bool c_loaded = false;

  // ---- 1. candidate threshold ------------------------------------------------
  uint32_t T = 1u;          // lowest candidate code; 1 takes every key
  bool sampled = false;     // T came from the sample
  bool try_list = true;     // false: the list cannot hold the candidates
  uint32_t bshift = 0u;     // candidate bins: min((code - T) >> bshift, kBins - 1)
  uint32_t kk = (uint32_t)min(a.k, len);   // level 0: every position of the window is a key
  // Fragment maxima (when the logits kernel wrote them): fragment f holds keys [16 f, 16 f + 16) of a
  // window that starts at key 0.  At least kk fragments have a maximum >= the kk-th largest
  // fragment maximum, so at least kk keys do: that value bounds the kk-th largest key from below,
  // and every key at or above it lies in a fragment whose maximum reaches it.  With at least 1.5 kk
  // fragments the bound sits high enough that the keys reaching it fit the list (1.15 to 1.75 kk on
  // the decode rows); if they do not (ties, values crowding into few fragments), the sampled
  // threshold and the streamed compaction below run instead.
  const int nfrag = (len + 15) / 16;
  uint32_t C = 0xffffffffu;
  bool listed = false;   // the candidate list came from the fragment maxima
  auto cand_bin = [&](uint32_t code) { return min((code - T) >> bshift, (uint32_t)(kBins - 1)); };
  if (FM && a.frag_max != nullptr && len > CAP && 2 * nfrag >= 3 * (int)kk && sa == 0) {
#pragma unroll
    for (int b = 0; b < kSampleRuns; ++b) fc[b] = b * THREADS + tid < nfrag ? max(fc[b], 1u) : 0u;   // 0: none
    uint32_t fmin = 0xffffffffu, fmax = 0u, nf = 0u;
#pragma unroll
    for (int b = 0; b < kSampleRuns; ++b) {
      if (fc[b] != 0u) {
        fmin = min(fmin, fc[b]);
        fmax = max(fmax, fc[b]);
        ++nf;
      }
    }
    block_min_max_sum<NW>(fmin, fmax, nf, sh.w0, sh.w1, sh.w2);
    uint32_t unused;
    // slack 16: T is the lowest code of a bin holding the kk-th largest maximum, so at least kk
    // (and fewer than kk + 16, bar ties) fragments reach it
    uint32_t Tf = radix_select<THREADS>(
        [&](auto&& visit) {
#pragma unroll
          for (int b = 0; b < kSampleRuns; ++b)
            if (fc[b] != 0u) visit(fc[b]);
        },
        fmin, fmax, kk, 16u, unused, sh);
    Tf = max(Tf, 1u);
    // The fragments whose maximum reaches Tf, listed in LDS (the histogram array is free until the
    // selection), then read 16 keys at a time; their keys >= Tf form the candidate list.
    uint32_t* flist = sh.hist;
    constexpr int kFragListCap = WORDS;
    uint32_t mine = 0u;
#pragma unroll
    for (int b = 0; b < kSampleRuns; ++b) mine += fc[b] >= Tf ? 1u : 0u;
    uint32_t incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t t = (uint32_t)__shfl_up((int)incl, o);
      if (lane >= o) incl += t;
    }
    uint32_t fbase = 0u;
    if (lane == 63 && incl > 0u) fbase = atomicAdd(&sh.nfrag_listed, incl);
    fbase = __builtin_amdgcn_readlane(fbase, 63);
    uint32_t fslot = fbase + incl - mine;
#pragma unroll
    for (int b = 0; b < kSampleRuns; ++b)
      if (fc[b] >= Tf) {
        if (fslot < (uint32_t)kFragListCap) flist[fslot] = (uint32_t)(b * THREADS + tid);
        ++fslot;
      }
    __syncthreads();
    const uint32_t nq = sh.nfrag_listed;
    if (nq <= (uint32_t)kFragListCap) {
      // Four consecutive lanes read one fragment (16 bytes each), so a load instruction covers 16
      // fragments; kQ loads per thread cover THREADS * kQ / 4 listed fragments per round trip.
      constexpr int kQ = 18;
      const float* rowp = src.f;   // window start (key 0) at a 16-byte boundary
      const int64_t last4 = a.ld - 4;   // last 16-byte load inside the row
      const int quarter = tid & 3;
      for (uint32_t q0 = 0; q0 < nq; q0 += THREADS * kQ / 4) {
        v4f d[kQ];
        int key0[kQ];   // position of d[j][0]
#pragma unroll
        for (int j = 0; j < kQ; ++j) {
          const uint32_t qi = q0 + (uint32_t)(j * (THREADS / 4) + (tid >> 2));
          key0[j] = (int)flist[min(qi, nq - 1u)] * 16 + 4 * quarter;
          d[j] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(rowp + min((int64_t)key0[j], last4)));
        }
        auto take = [&](int j, int e) -> bool {
          return q0 + (uint32_t)(j * (THREADS / 4) + (tid >> 2)) < nq && key0[j] + e < len &&
                 SegmentSource<LEVEL0, VEC>::float_code(d[j][e]) >= Tf;
        };
        uint32_t cm = 0u;
#pragma unroll
        for (int j = 0; j < kQ; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) cm += take(j, e) ? 1u : 0u;
        uint32_t ci = cm;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t t = (uint32_t)__shfl_up((int)ci, o);
          if (lane >= o) ci += t;
        }
        uint32_t cbase = 0u;
        if (lane == 63 && ci > 0u) cbase = atomicAdd(&sh.cnt, ci);
        cbase = __builtin_amdgcn_readlane(cbase, 63);
        uint32_t cslot = cbase + ci - cm;
#pragma unroll
        for (int j = 0; j < kQ; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (take(j, e)) {
              sh.cand[min(cslot, (uint32_t)CAP)] =
                  v2u{SegmentSource<LEVEL0, VEC>::float_code(d[j][e]), (uint32_t)(key0[j] + e)};
              ++cslot;
            }
      }
    }
    __syncthreads();
    const uint32_t cf = sh.nfrag_listed <= (uint32_t)WORDS ? sh.cnt : 0xffffffffu;
    __syncthreads();   // every thread has read the counts
    if (cf >= kk && cf <= (uint32_t)CAP) {
      listed = true;
      C = cf;
      T = Tf;
      sampled = true;
      const uint32_t range = fmax - min(T, fmax);
      bshift = range >> kDigitBits ? (uint32_t)(32 - __builtin_clz(range) - kDigitBits) : 0u;
#pragma unroll
      for (int i = 0; i < kBins / THREADS; ++i) sh.hist[tid * (kBins / THREADS) + i] = 0u;
    } else if (tid == 0) {
      sh.cnt = 0u;
    }
    __syncthreads();
  }
  if (!listed) {
    if (len > CAP) {
      uint32_t sc[kSampleRuns];
#pragma unroll
      for (int b = 0; b < kSampleRuns; ++b) {
        const int start = src.off + (int)((int64_t)b * (len - THREADS) / (kSampleRuns - 1));
        sc[b] = src.code_at(start + tid);
      }
      if (nvec > 0) {
        load_pass(0, c);
        c_loaded = true;
        __builtin_amdgcn_sched_barrier(0);   // keep these loads ahead of the threshold work
      }
      uint32_t smin = 0xffffffffu, smax = 0u, ns = 0u;
#pragma unroll
      for (int b = 0; b < kSampleRuns; ++b) {
        if (sc[b] != 0u) {
          smin = min(smin, sc[b]);
          smax = max(smax, sc[b]);
          ++ns;
        }
      }
      block_min_max_sum<NW>(smin, smax, ns, sh.w0, sh.w1, sh.w2);
      // sample rank whose code should leave ~1.3 k keys at or above it
      const uint64_t want = ((uint64_t)kk * kSampleSize * 13u + 10ull * len - 1u) / (10ull * len) + 16u;
      if (ns > 0u && want < ns && want * (uint64_t)len <= (uint64_t)CAP * kSampleSize * 7u / 8u) {
        uint32_t unused;
        T = radix_select<THREADS>(
            [&](auto&& visit) {
#pragma unroll
              for (int b = 0; b < kSampleRuns; ++b)
                if (sc[b] != 0u) visit(sc[b]);
            },
            smin, smax, (uint32_t)want, 16u, unused, sh);
        T = max(T, 1u);
        sampled = true;
        const uint32_t range = smax - min(T, smax);
        bshift = range >> kDigitBits ? (uint32_t)(32 - __builtin_clz(range) - kDigitBits) : 0u;
      } else if (LEVEL0) {
        try_list = false;   // every key would be a candidate, more than the list holds
      }
    }
    if (sampled) {
#pragma unroll
      for (int i = 0; i < kBins / THREADS; ++i) sh.hist[tid * (kBins / THREADS) + i] = 0u;
    }
    __syncthreads();

    // ---- 2. compaction of the codes >= T ----------------------------------------
    if (try_list) {
      // Every lane runs every pass (the slot scan below is wave-wide); the next
      // pass's loads are in flight while this pass's keys are appended.  Keys are
      // loaded raw.  With the threshold above +0.0, a level-0 key is a candidate
      // exactly when its bits, read as a signed int, reach T - 2^31: negative
      // floats, -0.0 and negative NaNs are negative ints, and the code of a
      // non-negative float is its bits with the sign bit set.  A pass whose
      // vectors all lie in the window then costs one compare per key; other
      // passes take the general test on codes.
      const bool raw_cmp = LEVEL0 && T > 0x80000000u;
      const int Ti = (int)(T - 0x80000000u);
      if (nvec > 0 && !c_loaded) load_pass(0, c);
      for (int vb = 0; vb < nvec; vb += kPass) {
        uint32_t nx[UNR][VEC];
        const bool more = vb + kPass < nvec;
        if (more) load_pass(vb + kPass, nx);
        const int v0 = vb + tid;
        if (raw_cmp && vb * VEC >= src.off && (vb + kPass) * VEC <= src.span)
          append_candidates<true, THREADS, CAP, UNR, VEC>(c, v0, nvec, src, T, Ti, lane, sh);
        else
          append_candidates<false, THREADS, CAP, UNR, VEC>(c, v0, nvec, src, T, Ti, lane, sh);
        if (more) {
#pragma unroll
          for (int u = 0; u < UNR; ++u)
#pragma unroll
            for (int i = 0; i < VEC; ++i) c[u][i] = nx[u][i];
        }
      }
      __syncthreads();
      C = sh.cnt;
      if (!LEVEL0 && !sampled) kk = min((uint32_t)a.k, C);   // C counted every key
    }
  }

  bool done = false;
  bool row_written = false;   // output row including padding already stored
  if (kk > 0u && C >= kk && C <= (uint32_t)CAP) {
    bool binned = sampled;
    if (!sampled && C > kk) {
      // An unsampled list (every key of a short segment, or a merge level's candidates) is binned
      // between its own smallest and largest code, as a sampled list is between T and the sample
      // maximum: one histogram pass instead of a radix select.
      uint32_t cmin = 0xffffffffu, cmax = 0u, unused = 0u;
      for (uint32_t i = tid; i < C; i += THREADS) {
        cmin = min(cmin, sh.cand[i].x);
        cmax = max(cmax, sh.cand[i].x);
      }
      block_min_max_sum<NW>(cmin, cmax, unused, sh.w0, sh.w1, sh.w2);
      T = cmin;   // >= 1: every listed code is
      const uint32_t range = cmax - cmin;
      bshift = range >> kDigitBits ? (uint32_t)(32 - __builtin_clz(range) - kDigitBits) : 0u;
#pragma unroll
      for (int i = 0; i < kBins / THREADS; ++i) sh.hist[tid * (kBins / THREADS) + i] = 0u;
      __syncthreads();
      binned = true;
    }
    if (binned) {
      // ---- 3. the bin of the k-th candidate ------------------------------------
      // Each thread handles list entries tid + THREADS * j in chunks of kRegPairs
      // held in registers (one chunk, read once, when the list is small).
      constexpr int kLpt = CAP / THREADS;
      constexpr int kRegPairs = kLpt < 16 ? kLpt : 16;
      constexpr int kChunks = kLpt / kRegPairs;
      v2u reg[kRegPairs];
      auto load_chunk = [&](int ch) {
#pragma unroll
        for (int j = 0; j < kRegPairs; ++j) {
          const uint32_t i = (uint32_t)((ch * kRegPairs + j) * THREADS + tid);
          reg[j] = i < C ? sh.cand[i] : v2u{0u, 0u};   // code 0: no entry (all candidates are >= T >= 1)
        }
      };
      if (kChunks == 1) load_chunk(0);
      for (int ch = 0; ch < kChunks; ++ch) {
        if (kChunks > 1) load_chunk(ch);
#pragma unroll
        for (int j = 0; j < kRegPairs; ++j)
          if (reg[j].x != 0u) atomicAdd(&sh.hist[cand_bin(reg[j].x)], 1u);
      }
      __syncthreads();
      uint32_t b, above, m;
      pick_bin<THREADS>(kk, b, above, m, sh);
      if (m <= (uint32_t)kBoundaryMax) {
        const uint32_t need = kk - above;   // taken from the boundary bin, 1 <= need <= m
        for (int ch = 0; ch < kChunks; ++ch) {
          if (kChunks > 1) load_chunk(ch);
#pragma unroll
          for (int j = 0; j < kRegPairs; ++j) {
            if (reg[j].x == 0u) continue;
            const uint32_t bn = cand_bin(reg[j].x);
            const uint32_t pos = reg[j].y;
            if (bn > b) {
              atomicOr(&sh.bits[pos >> 5], 1u << (pos & 31));
            } else if (bn == b) {
              const uint32_t o = atomicAdd(&sh.nb, 1u);
              sh.bk[o] = reg[j].x;
              sh.bp[o] = pos;
            }
          }
        }
        __syncthreads();
        // ---- 4. rank the boundary bin pairwise: value desc, then position asc ----
        if (tid < (int)m) {
          const uint32_t mc = sh.bk[tid], mp = sh.bp[tid];
          uint32_t r = 0u;
          for (uint32_t j = 0; j < m; ++j) {
            const uint32_t c2 = sh.bk[j], p2 = sh.bp[j];
            r += (c2 > mc) || (c2 == mc && p2 < mp);
          }
          if (r < need) atomicOr(&sh.bits[mp >> 5], 1u << (mp & 31));
        }
        __syncthreads();
        // ---- 5. output slots by position --------------------------------------
        bitmap_prefix<THREADS, WORDS>(sh.bits, sh.hist, nwords, sh.w0);
        if (kChunks == 1) {
          // The list lives in registers now: stage the output row in its LDS
          // and store the row with coalesced writes.
          v2u* stage = sh.cand;
#pragma unroll
          for (int j = 0; j < kRegPairs; ++j) {
            const uint32_t pos = reg[j].y;
            if (reg[j].x != 0u && ((sh.bits[pos >> 5] >> (pos & 31)) & 1u))
              stage[bitmap_rank(sh.bits, sh.hist, pos)] = reg[j];
          }
          __syncthreads();
          // A thread's outputs in batches: every source-index load of a batch, then every map
          // load, then the stores, so the loads of a batch are in flight together.
          constexpr int kOutBatch = 8;
          for (int o0 = 0; o0 < a.k; o0 += THREADS * kOutBatch) {
            int32_t jv[kOutBatch];
            uint32_t cv[kOutBatch];
#pragma unroll
            for (int b = 0; b < kOutBatch; ++b) {
              const int o = o0 + b * THREADS + tid;
              const v2u e = o < (int)kk ? stage[o] : v2u{0u, 0u};
              cv[b] = e.x;
              jv[b] = -1;
              if (o < (int)kk) jv[b] = LEVEL0 ? (int32_t)(lb + e.y) : a.in_idx[(int64_t)row * a.in_len + lb + e.y];
            }
            if (FINAL) {
#pragma unroll
              for (int b = 0; b < kOutBatch; ++b) {
                const int o = o0 + b * THREADS + tid;
                jv[b] = o < (int)kk ? map_index(map, req, row_ks, jv[b]) : -1;
              }
            }
#pragma unroll
            for (int b = 0; b < kOutBatch; ++b) {
              const int o = o0 + b * THREADS + tid;
              if (o < a.k) {
                if (FINAL) {
                  a.out[out_base + o] = jv[b];
                } else {
                  a.out_keys[out_base + o] = o < (int)kk ? cv[b] : 0u;
                  a.out_idx[out_base + o] = jv[b];
                }
              }
            }
          }
          row_written = true;
        } else {
          for (int ch = 0; ch < kChunks; ++ch) {
            load_chunk(ch);
#pragma unroll
            for (int j = 0; j < kRegPairs; ++j) {
              const uint32_t pos = reg[j].y;
              if (reg[j].x != 0u && ((sh.bits[pos >> 5] >> (pos & 31)) & 1u))
                emit(bitmap_rank(sh.bits, sh.hist, pos), pos, reg[j].x);
            }
          }
        }
        done = true;
      }
    }
    if (!done) {
      // ---- exact selection on the whole list (dense ties, or an unsampled list) ----
      // A list of at most kk entries is taken whole: tau = 0 lies below every
      // listed code (codes are >= 1), so no entry ties with it.
      uint32_t need = 0u;
      uint32_t tau = 0u;
      if (C > kk) {
        uint32_t cmin = 0xffffffffu, cmax = 0u, unused = 0u;
        for (uint32_t i = tid; i < C; i += THREADS) {
          cmin = min(cmin, sh.cand[i].x);
          cmax = max(cmax, sh.cand[i].x);
        }
        block_min_max_sum<NW>(cmin, cmax, unused, sh.w0, sh.w1, sh.w2);
        tau = radix_select<THREADS>(
            [&](auto&& visit) {
              for (uint32_t i = tid; i < C; i += THREADS) visit(sh.cand[i].x);
            },
            cmin, cmax, kk, 0u, need, sh);
      }
      uint32_t eq = 0u;
      for (uint32_t i = tid; i < C; i += THREADS) eq += sh.cand[i].x == tau;
      const uint32_t E = block_sum<NW>(eq, sh.w0);
      if (need < E) {
        for (int wi = tid; wi < nwords; wi += THREADS) sh.bits[wi] = 0u;
        __syncthreads();
        for (uint32_t i = tid; i < C; i += THREADS)
          if (sh.cand[i].x == tau) atomicOr(&sh.bits[sh.cand[i].y >> 5], 1u << (sh.cand[i].y & 31));
        __syncthreads();
        bitmap_prefix<THREADS, WORDS>(sh.bits, sh.hist, nwords, sh.w0);
        // ties past the first `need` by position drop out: code 0 is below tau
        for (uint32_t i = tid; i < C; i += THREADS)
          if (sh.cand[i].x == tau && bitmap_rank(sh.bits, sh.hist, sh.cand[i].y) >= need) sh.cand[i].x = 0u;
        __syncthreads();
      }
      for (int wi = tid; wi < nwords; wi += THREADS) sh.bits[wi] = 0u;
      __syncthreads();
      for (uint32_t i = tid; i < C; i += THREADS)
        if (sh.cand[i].x >= tau) atomicOr(&sh.bits[sh.cand[i].y >> 5], 1u << (sh.cand[i].y & 31));
      __syncthreads();
      bitmap_prefix<THREADS, WORDS>(sh.bits, sh.hist, nwords, sh.w0);
      for (uint32_t i = tid; i < C; i += THREADS) {
        const v2u e = sh.cand[i];
        if (e.x >= tau) emit(bitmap_rank(sh.bits, sh.hist, e.y), e.y, e.x);
      }
      done = true;
    }
  }
  if (!done && len > 0) {
    // ---- fallback: exact selection over every key of the segment, streamed --------
    if (!LEVEL0) {
      uint32_t nv = 0u;
      stream([&](int, uint32_t) { ++nv; });
      kk = min((uint32_t)a.k, block_sum<NW>(nv, sh.w0));
    }
    if (kk > 0u) {
      uint32_t need;
      const uint32_t tau = radix_select<THREADS>(
          [&](auto&& visit) { stream([&](int, uint32_t code) { visit(code); }); }, 1u, 0xffffffffu, kk, 0u,
          need, sh);
      uint32_t* tie_bits = reinterpret_cast<uint32_t*>(sh.cand);   // the candidate list is free here
      uint32_t* tie_pre = tie_bits + WORDS;
      uint32_t eq = 0u;
      stream([&](int, uint32_t code) { eq += code == tau; });
      const uint32_t E = block_sum<NW>(eq, sh.w0);
      const bool rank_ties = need < E;
      if (rank_ties) {
        for (int wi = tid; wi < nwords; wi += THREADS) tie_bits[wi] = 0u;
        __syncthreads();
        stream([&](int pos, uint32_t code) {
          if (code == tau) atomicOr(&tie_bits[pos >> 5], 1u << (pos & 31));
        });
        __syncthreads();
        bitmap_prefix<THREADS, WORDS>(tie_bits, tie_pre, nwords, sh.w0);
      }
      auto selected = [&](int pos, uint32_t code) {
        return code > tau || (code == tau && (!rank_ties || bitmap_rank(tie_bits, tie_pre, pos) < need));
      };
      for (int wi = tid; wi < nwords; wi += THREADS) sh.bits[wi] = 0u;
      __syncthreads();
      stream([&](int pos, uint32_t code) {
        if (selected(pos, code)) atomicOr(&sh.bits[pos >> 5], 1u << (pos & 31));
      });
      __syncthreads();
      bitmap_prefix<THREADS, WORDS>(sh.bits, sh.hist, nwords, sh.w0);
      stream([&](int pos, uint32_t code) {
        if (selected(pos, code)) emit(bitmap_rank(sh.bits, sh.hist, (uint32_t)pos), (uint32_t)pos, code);
      });
    }
  }
  // padding after the kk selected entries
  if (!row_written) {
    for (int o = (int)kk + tid; o < a.k; o += THREADS) {
      if (FINAL) {
        a.out[out_base + o] = -1;
      } else {
        a.out_keys[out_base + o] = 0u;
        a.out_idx[out_base + o] = -1;
      }
    }
  }
}

// ---- host-side plan and launch ----------------------------------------------

TopkPlan plan_topk(int32_t rows, int64_t width, int32_t k) {
  TopkPlan p{};
  p.supported = true;
  p.buf_bytes[0] = p.buf_bytes[1] = 0;
  int64_t in_len = width > 0 ? width : 1;
  const int64_t min_seg = std::max<int64_t>(8 * (int64_t)k, 16384);
  // Few long rows (decode): one 512-thread workgroup takes a whole row of up to 131072 keys, twice the
  // loads in flight of a 256-thread segment, in a single launch without a merge level.
  if (rows > 0 && rows <= kWideRowsMax && in_len > min_seg && in_len <= kWideSeg && !topk_needs_big_cap(k)) {
    TopkLevel& L = p.level[0];
    L.in_len = in_len;
    L.seg_len = (int32_t)in_len;
    L.nseg = 1;
    L.cfg = 2;
    p.nlevels = 1;
    return p;
  }
  // few rows: split long windows so about this many workgroups run.  Every extra segment sends k
  // more candidates to the next level, so the target stays low: on 256 decode rows of up to 131072
  // keys, 2 segments per row ran 11% faster than 4.
  const int64_t target_wgs = 512;
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
    L.cfg = topk_needs_big_cap(k) ? 1 : 0;
    p.nlevels = lvl + 1;
    if (nseg == 1) break;
    const int64_t out_len = nseg * (int64_t)k;
    const size_t bytes = (size_t)rows * (size_t)out_len * 8u;
    p.buf_bytes[lvl & 1] = std::max(p.buf_bytes[lvl & 1], bytes);
    in_len = out_len;
  }
  // the last level writes the output row, so it must hold one segment per row
  if (p.level[p.nlevels - 1].nseg > 1) p.supported = false;
  return p;
}

static size_t align256(size_t x) { return (x + 255u) & ~(size_t)255u; }

bool topk_plan_takes_frag_max(const TopkPlan& p) { return p.supported && p.nlevels == 1 && p.level[0].cfg == 2; }

size_t topk_workspace_bytes(const TopkPlan& p) {
  size_t total = 0;
  for (int b = 0; b < 2; ++b)
    if (p.buf_bytes[b]) total += align256(p.buf_bytes[b]);
  return total;
}

template <int THREADS, int CAP, int SEG, bool LEVEL0, bool FINAL>
static void launch_vec(bool vec4, unsigned grid, const TopkKernelArgs& a, hipStream_t s) {
  if (vec4)
    hipLaunchKernelGGL((topk_kernel<THREADS, CAP, SEG, LEVEL0, FINAL, 4>), dim3(grid), dim3(THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((topk_kernel<THREADS, CAP, SEG, LEVEL0, FINAL, 1>), dim3(grid), dim3(THREADS), 0, s, a);
}

static void launch_wide_frag_max(unsigned grid, const TopkKernelArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((topk_kernel<kWideThreads, kSmallCap, (int)kWideSeg, true, true, 4, true>), dim3(grid),
                     dim3(kWideThreads), 0, s, a);
}

template <int CAP>
static void launch_cap(bool level0, bool final_level, bool vec4, unsigned grid, const TopkKernelArgs& a,
                       hipStream_t s) {
  constexpr int kSeg = (int)kMaxSeg;
  if (level0 && final_level) launch_vec<kTopkThreads, CAP, kSeg, true, true>(vec4, grid, a, s);
  else if (level0) launch_vec<kTopkThreads, CAP, kSeg, true, false>(vec4, grid, a, s);
  else if (final_level) launch_vec<kTopkThreads, CAP, kSeg, false, true>(vec4, grid, a, s);
  else launch_vec<kTopkThreads, CAP, kSeg, false, false>(vec4, grid, a, s);
}

hipError_t launch_topk(const TopkArgs& ta, const TopkPlan& plan, void* ws, hipStream_t s) {
  if (ta.rows <= 0) return hipSuccess;
  if (!plan.supported) return hipErrorInvalidValue;
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
    bool vec4;
    if (!level0) {
      const uint8_t* src = bufs[(lvl - 1) & 1];
      const int64_t n_in = (int64_t)ta.rows * L.in_len;
      a.in_keys = reinterpret_cast<const uint32_t*>(src);
      a.in_idx = reinterpret_cast<const int32_t*>(src + (size_t)n_in * 4u);
      a.in_len = L.in_len;
      vec4 = (L.in_len % 4) == 0;
    } else {
      // 16-byte loads need every row start 16-byte aligned
      vec4 = (ta.ld % 4) == 0 && (reinterpret_cast<uintptr_t>(ta.logits) & 15u) == 0;
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
    if (L.cfg == 2 && ta.frag_max != nullptr && vec4 && ta.ks == nullptr) {
      a.frag_max = ta.frag_max;
      a.frag = ta.frag;
      a.frag_next_n = ta.frag_next_n;
      launch_wide_frag_max((unsigned)grid, a, s);
    } else if (L.cfg == 2) {
      launch_vec<kWideThreads, kSmallCap, (int)kWideSeg, true, true>(vec4, (unsigned)grid, a, s);
    } else if (L.cfg == 1) {
      launch_cap<kBigCap>(level0, final_level, vec4, (unsigned)grid, a, s);
    } else {
      launch_cap<kSmallCap>(level0, final_level, vec4, (unsigned)grid, a, s);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace fp8idx
