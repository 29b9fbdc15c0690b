// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8idx {

struct RaggedLogitsArgs {
  const uint8_t* q;
  const uint8_t* kv;
  const float* kv_scale;
  const float* weights;
  const int32_t* ks;
  const int32_t* ke;
  int32_t m;
  int32_t n;
  float* logits;
  int64_t ld;
  int32_t clean;
  unsigned int* queue;   // kRaggedQueueWords work-queue counters (device), cleared by each launch
  int32_t wgs_per_cu;    // resident workgroups to launch per CU; 0: as many as fit (leaves none for
                         // kernels on other streams)
};

// Work-queue counters of one ragged logits launch: one claim counter per XCD queue, padded to
// 256 bytes so that the counters of a workspace never share a cache line with other data.
constexpr int kRaggedQueueWords = 8;
constexpr size_t kRaggedQueueBytes = 256;

// Layout of the paged logits kernel's per-fragment maxima (the fused paged entry hands them to its
// top-k).  Chunk-major, so that each claimed chunk's maxima leave as one contiguous block: the
// maxima of unit u's chunk c are frag_max[u * unit_stride + c * rows * fpc + r * fpc + j] for the
// unit's row r < rows and the chunk's 16-key fragment j < fpc; fragment f of a row is chunk f / fpc,
// j = f % fpc.  A row's request b and index t (of next_n) give u = b * ceil(next_n / 4) + t / 4,
// r = t % 4.
struct FragLayout {
  int32_t rows;          // row slots per block: min(4, next_n)
  int32_t fpc;           // fragments per row and chunk: 4 x the chunk's pages
  int64_t unit_stride;   // elements per unit: blocks for every chunk of the width
  int64_t elems;         // capacity of frag_max (elements), checked by every store
};

struct PagedLogitsArgs {
  const uint8_t* q;
  const uint8_t* kv_pool;
  const float* scale_pool;
  const float* weights;
  const int32_t* row_len;
  const int32_t* block_table;
  int32_t B;
  int32_t next_n;
  int32_t max_pages;
  int64_t num_pages;
  float* logits;
  int64_t ld;
  int32_t width;
  int32_t clean;
  // Optional (null: not written): per (row, 16-key fragment f) the largest order code
  // (float_to_ordered) of the row's logits at keys [16 f, 16 f + 16) inside its window (0 for none),
  // laid out as `frag` says (take it from paged_frag_layout for the same B, next_n, max_pages and
  // width); only with 16-byte aligned logits rows and frag_max.
  uint32_t* frag_max;
  FragLayout frag;
};

struct TopkMap {
  int32_t kind;
  const int32_t* table;
  int64_t ld;
  int32_t num_req;
  const int32_t* cu_rows;
  int32_t rows_per_req;
  int32_t page_size;
  int64_t num_pages;   // block table: page ids outside [0, num_pages) map to -1
};

struct TopkArgs {
  const float* logits;
  int64_t ld;
  int32_t rows;
  int32_t width;
  const int32_t* ks;  // may be null
  const int32_t* ke;
  int32_t k;
  int32_t row0;
  TopkMap map;
  int32_t* out;
  int64_t ld_out;
  // Optional: the fragment maxima the paged logits kernel wrote for these logits (see
  // PagedLogitsArgs::frag_max), row i of the call being row i of that launch, whose requests have
  // frag_next_n rows; used by the one-workgroup-per-row configuration when ks is null.
  const uint32_t* frag_max;
  FragLayout frag;
  int32_t frag_next_n;
};

// Host-side plan of the multi-level top-k: level 0 splits each row into
// segments; each further level merges the previous level's per-segment
// candidates until one segment per row remains.
struct TopkLevel {
  int64_t in_len;   // elements per row entering this level
  int32_t seg_len;  // elements per segment (<= capacity of the chosen config)
  int32_t nseg;     // segments per row
  int32_t cfg;      // kernel configuration id
};

constexpr int kMaxTopkLevels = 8;
constexpr size_t kQRowBytesHost = 32 * 128;   // q bytes per query row (H * D)
constexpr int kMaxK = 16384;

struct TopkPlan {
  int nlevels;
  bool supported;       // false: the merge would need more than kMaxTopkLevels levels
  TopkLevel level[kMaxTopkLevels];
  size_t buf_bytes[2];  // ping-pong candidate buffers (bytes each)
};

// Device properties the launchers need, cached per device.
struct DeviceInfo {
  int cu_count;
  int ragged_wgs_per_cu;   // resident workgroups of the ragged logits kernel per CU
  int paged_wgs_per_cu;    // resident workgroups of the paged logits kernel per CU
};

// Fills the occupancy fields of `d` (called once per device).
void query_ragged_occupancy(DeviceInfo& d);
void query_paged_occupancy(DeviceInfo& d);

TopkPlan plan_topk(int32_t rows, int64_t width, int32_t k);
size_t topk_workspace_bytes(const TopkPlan& p);
// True when launch_topk under this plan takes fragment maxima (one workgroup per whole row).
bool topk_plan_takes_frag_max(const TopkPlan& p);

hipError_t launch_logits_ragged(const RaggedLogitsArgs& a, const DeviceInfo& dev, hipStream_t s);
// Device address of the current device's static work-queue counters (logits_ragged.hip), looked up
// once per device; used by the entry point that allocates nothing.
hipError_t ragged_noalloc_queue(unsigned int** out);
hipError_t launch_logits_paged(const PagedLogitsArgs& a, const DeviceInfo& dev, hipStream_t s);
// The fragment-maxima layout a paged logits launch over B requests of next_n rows uses (elems = 0:
// the caller sets the capacity).
FragLayout paged_frag_layout(int32_t B, int32_t next_n, int32_t max_pages, int32_t width);
constexpr int kPrepMaxReq = 4096;   // requests per index-preparation call
struct PrepRaggedArgs {
  const int32_t* seq_len;
  const int32_t* q_len;
  const int32_t* req_idx;
  const int32_t* table;
  int64_t ld_table;
  int32_t num_rows;
  int32_t B;
  int32_t* cu_seq;
  int32_t* cu_q;
  int32_t* ks;
  int32_t* ke;
  int64_t max_q;
  int32_t* ragged_mem;
  int64_t max_keys;
};
struct PrepDecodeArgs {
  const int32_t* seq_len;
  const int32_t* req_idx;
  const int32_t* req_to_page;
  int64_t ld_r2p;
  int32_t num_rows;
  int32_t B;
  int32_t next_n;
  int32_t* row_len;
  int32_t* block_table;
  int64_t ld_bt;
  int32_t max_pages;
};
hipError_t launch_prep_ragged(const PrepRaggedArgs& a, const DeviceInfo& dev, hipStream_t s);
hipError_t launch_prep_decode(const PrepDecodeArgs& a, hipStream_t s);

struct QuantArgs {
  const float* x;
  int64_t ld_x;
  int64_t rows;
  int32_t D;
  uint8_t* codes;
  int64_t ld_codes;
  float* scale;
};
hipError_t launch_quant_fp8(const QuantArgs& a, hipStream_t s);
hipError_t launch_topk(const TopkArgs& a, const TopkPlan& plan, void* ws, hipStream_t s);

// Sparse MLA attention over top-k slots (sparse_mla.hip).
constexpr int kMlaDqk = 576;   // KV row: 512 latent + 64 rotary values
constexpr int kMlaDv = 512;    // value: the latent part
constexpr int kMlaBlock = 64;  // keys staged per step
struct SparseMlaArgs {
  const uint16_t* q;        // bf16 [T, H, 576]
  const uint8_t* kv;        // e4m3fn [S, 576]
  const float* kv_scale;    // [S]
  int64_t num_slots;
  const int32_t* indices;   // [T, ld_idx]
  int64_t ld_idx;
  int32_t T;
  int32_t H;
  int32_t topk;
  float sm_scale;
  float* out;               // [T, H, 512]
  float* lse;               // [T, H] or null
};
struct SparseMlaPlan {
  int32_t nsplit;           // key ranges per (token, head block)
  int32_t keys_per_split;   // a multiple of kMlaBlock
  size_t ws_bytes;          // partial outputs when nsplit > 1
};
SparseMlaPlan plan_sparse_mla(int32_t T, int32_t H, int32_t topk);
hipError_t launch_sparse_mla(const SparseMlaArgs& a, const SparseMlaPlan& plan, void* ws, hipStream_t s);

// fp8 MFMA throughput probe: blocks x kProbeThreads threads, each wave iters x kProbeChains MFMAs;
// one float per thread to out (keeps the work live).
constexpr int kProbeChains = 4;
constexpr int kProbeThreads = 256;
hipError_t launch_mfma_probe(int blocks, int iters, float* out, hipStream_t s);
// Logits-core probe: blocks x kProbeThreads threads, each wave iters x (8 MFMAs + the exact
// epilogue of one 16-key fragment) on register operands; one float per thread to out.
hipError_t launch_logits_core_probe(int blocks, int iters, float* out, hipStream_t s);

}  // namespace fp8idx
