// C ABI of the fp8 MQA indexer library: argument validation, device checks,
// workspace arithmetic and the row-chunked fused loop.  Every kernel launch
// goes on the caller's stream; nothing here allocates or synchronises.

#include <fp8idx.h>

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>

#include "launch.hpp"

namespace {

using fp8idx::DeviceInfo;

thread_local int32_t g_last_hip_error = 0;

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
DeviceInfo g_dev_info[kMaxDevices];
int g_dev_ok[kMaxDevices];

fp8idx_status hip_fail(hipError_t e) {
  g_last_hip_error = (int32_t)e;
  return FP8IDX_EHIP;
}

// Current device must be a gfx950; properties are read once per device.
fp8idx_status current_device(DeviceInfo* out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8IDX_EDEVICE;
  std::call_once(g_dev_once[dev], [dev]() {
    hipDeviceProp_t p;
    std::memset(&p, 0, sizeof(p));
    if (hipGetDeviceProperties(&p, dev) == hipSuccess) {
      g_dev_ok[dev] = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
      g_dev_info[dev].cu_count = p.multiProcessorCount;
      if (g_dev_ok[dev]) {
        fp8idx::query_ragged_occupancy(g_dev_info[dev]);
        fp8idx::query_paged_occupancy(g_dev_info[dev]);
      }
    } else {
      g_dev_ok[dev] = 0;
    }
  });
  if (!g_dev_ok[dev]) return FP8IDX_EDEVICE;
  *out = g_dev_info[dev];
  return FP8IDX_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t align256(size_t x) { return (x + 255u) & ~(size_t)255u; }

// Leading dimension of the float32 logits the fused entries keep in the
// workspace: the key count rounded up to 4 floats (16-byte rows).
int64_t ws_logits_ld(int64_t width) { return (width + 3) / 4 * 4; }

int32_t rows_per_chunk(size_t cap, int64_t ld, int32_t rows) {
  if (rows <= 0) return 0;
  if (cap == 0) return rows;
  const int64_t r = (int64_t)(cap / ((size_t)std::max<int64_t>(ld, 1) * 4u));
  return (int32_t)std::max<int64_t>(1, std::min<int64_t>(rows, r));
}

fp8idx_status check_shape(int32_t H, int32_t D) {
  if (H != 32 || D != 128) return FP8IDX_EUNSUPPORTED;
  return FP8IDX_OK;
}

fp8idx_status check_map(const fp8idx_map* map) {
  if (map == nullptr) return FP8IDX_OK;
  switch (map->kind) {
    case FP8IDX_MAP_NONE:
      return FP8IDX_OK;
    case FP8IDX_MAP_TOKEN_TABLE:
      if (!map->table || map->ld < 1 || map->num_req < 1) return FP8IDX_EINVAL;
      if (!aligned(map->table, 4) || (map->cu_rows && !aligned(map->cu_rows, 4))) return FP8IDX_EINVAL;
      return FP8IDX_OK;
    case FP8IDX_MAP_BLOCK_TABLE:
      if (!map->table || map->ld < 1 || map->num_req < 1 || map->rows_per_req < 1 || map->page_size < 1 ||
          map->num_pages < 1)
        return FP8IDX_EINVAL;
      if (!aligned(map->table, 4)) return FP8IDX_EINVAL;
      return FP8IDX_OK;
    default:
      return FP8IDX_EINVAL;
  }
}

fp8idx::TopkMap to_kernel_map(const fp8idx_map* map) {
  fp8idx::TopkMap m{};
  if (map == nullptr) {
    m.kind = FP8IDX_MAP_NONE;
    return m;
  }
  m.kind = map->kind;
  m.table = map->table;
  m.ld = map->ld;
  m.num_req = map->num_req;
  m.cu_rows = map->cu_rows;
  m.rows_per_req = map->rows_per_req;
  m.page_size = map->page_size;
  m.num_pages = map->num_pages;
  return m;
}

fp8idx_status check_ragged(const uint8_t* q, const uint8_t* kv, const float* kv_scale, const float* weights,
                           const int32_t* ks, const int32_t* ke, int32_t m, int32_t n, int32_t H, int32_t D) {
  if (fp8idx_status s = check_shape(H, D)) return s;
  if (m < 0 || n < 1) return FP8IDX_EINVAL;
  if (m == 0) return FP8IDX_OK;
  if (!q || !kv || !kv_scale || !weights || !ks || !ke) return FP8IDX_EINVAL;
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(weights, 16)) return FP8IDX_EINVAL;
  if (!aligned(kv_scale, 4) || !aligned(ks, 4) || !aligned(ke, 4)) return FP8IDX_EINVAL;
  return FP8IDX_OK;
}

fp8idx_status check_paged(const uint8_t* q, const uint8_t* kv_pool, const float* scale_pool,
                          const float* weights, const int32_t* row_len, const int32_t* block_table,
                          int32_t B, int32_t next_n, int32_t H, int32_t D, int32_t page_size,
                          int32_t max_pages, int64_t num_pages, int32_t width) {
  if (fp8idx_status s = check_shape(H, D)) return s;
  if (page_size != 64) return FP8IDX_EUNSUPPORTED;
  if (B < 0 || next_n < 1 || max_pages < 1 || num_pages < 1 || width < 0) return FP8IDX_EINVAL;
  if ((int64_t)width > (int64_t)max_pages * page_size) return FP8IDX_EINVAL;
  if (num_pages > (int64_t)(INT32_MAX / page_size)) return FP8IDX_EUNSUPPORTED;   // slot ids are int32
  if ((int64_t)B * next_n > INT32_MAX) return FP8IDX_EINVAL;
  if (B == 0) return FP8IDX_OK;
  if (!q || !kv_pool || !scale_pool || !weights || !row_len || !block_table) return FP8IDX_EINVAL;
  if (!aligned(q, 16) || !aligned(kv_pool, 16) || !aligned(weights, 16)) return FP8IDX_EINVAL;
  if (!aligned(scale_pool, 4) || !aligned(row_len, 4) || !aligned(block_table, 4)) return FP8IDX_EINVAL;
  return FP8IDX_OK;
}

fp8idx_status check_topk_args(int32_t rows, int32_t width, int64_t ld, int32_t k, int64_t ld_out) {
  if (k < 1 || k > fp8idx::kMaxK) return FP8IDX_EUNSUPPORTED;
  if (rows < 0 || width < 0 || ld < width || ld < 1 || ld_out < k) return FP8IDX_EINVAL;
  return FP8IDX_OK;
}

fp8idx_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return FP8IDX_OK;
  if (ws == nullptr || ws_bytes < need) return FP8IDX_EWORKSPACE;
  if (!aligned(ws, 256)) return FP8IDX_EINVAL;
  return FP8IDX_OK;
}

// Layout of the fused entries' workspace: [queue counters (ragged only)] [chunk logits x buffers]
// [fragment maxima (paged, when the top-k takes them)] [top-k candidates].  ok is false when the
// arguments are rejected (an unsupported top-k plan).
struct FusedLayout {
  bool ok;
  int32_t rpc;          // rows per chunk
  size_t queue_bytes;   // work-queue counters of the ragged logits launches
  size_t buf_bytes;     // one chunk of logits
  int32_t buffers;      // chunk logits buffers (2 when the overlap entry alternates them)
  int64_t frag_elems;   // fragment maxima of one chunk's requests (any chunk size of the paged kernel)
  size_t frag_bytes;    // one chunk's fragment maxima (paged, one-workgroup-per-row top-k), else 0
  size_t topk_bytes;    // candidates of the largest chunk's top-k
  size_t total;
};

FusedLayout fused_layout(int32_t rows, int64_t width, int32_t k, size_t cap, int32_t granule, bool ragged,
                         int32_t logit_buffers = 1) {
  FusedLayout L{};
  const int64_t ld = ws_logits_ld(width);
  int32_t rpc = rows_per_chunk(cap, ld, rows);
  if (granule > 1 && rpc < rows) rpc = std::max<int32_t>(granule, rpc / granule * granule);
  rpc = std::min(rpc, rows);
  if (rpc <= 0) return L;
  // As many chunks as the cap-derived size gives, with the rows spread evenly over them (in whole
  // granules): a short last chunk would run its launches at a fraction of their rate.
  const int32_t nch = (rows + rpc - 1) / rpc;
  int32_t even = (rows + nch - 1) / nch;
  if (granule > 1) even = (even + granule - 1) / granule * granule;
  rpc = std::min(rpc, even);
  const int32_t last = rows % rpc == 0 ? rpc : rows % rpc;
  const fp8idx::TopkPlan p0 = fp8idx::plan_topk(rpc, width, k);
  const fp8idx::TopkPlan p1 = fp8idx::plan_topk(last, width, k);
  if (!p0.supported || !p1.supported) return L;
  L.ok = true;
  L.rpc = rpc;
  L.queue_bytes = ragged ? fp8idx::kRaggedQueueBytes : 0;
  L.buf_bytes = align256((size_t)rpc * (size_t)ld * 4u);
  L.buffers = rpc < rows ? logit_buffers : 1;
  // the paged kernel's chunk-major maxima: per 4-row unit, min(4, next_n) rows of every 16-key
  // fragment of the width, rounded up to whole chunks of the larger chunk size (16 pages)
  const int32_t nn = std::max(granule, 1);
  const int64_t units = (int64_t)(rpc / nn) * ((nn + 3) / 4);
  L.frag_elems = units * ((width + 1023) / 1024) * (int64_t)std::min(4, nn) * 64;
  const bool frag = !ragged && (fp8idx::topk_plan_takes_frag_max(p0) || fp8idx::topk_plan_takes_frag_max(p1));
  L.frag_bytes = frag ? align256((size_t)L.frag_elems * 4u) : 0;
  L.topk_bytes = std::max(fp8idx::topk_workspace_bytes(p0), fp8idx::topk_workspace_bytes(p1));
  L.total = L.queue_bytes + L.buf_bytes * (size_t)L.buffers + L.frag_bytes + L.topk_bytes;
  return L;
}

// ---- argument validation, shared by the entry points and fp8idx_validate_only ----------------

// Everything but the workspace (the allocation-free variant has none).
fp8idx_status validate_logits_ragged_io(const fp8idx_call_args& c) {
  if (fp8idx_status s = check_ragged(c.q, c.kv, c.kv_scale, c.weights, c.ks, c.ke, c.m, c.n, c.H, c.D)) return s;
  if (c.m == 0) return FP8IDX_OK;
  if (!c.logits || !aligned(c.logits, 4) || c.ld_logits < c.n) return FP8IDX_EINVAL;
  return FP8IDX_OK;
}

fp8idx_status validate_logits_ragged(const fp8idx_call_args& c) {
  if (fp8idx_status s = validate_logits_ragged_io(c)) return s;
  if (c.m == 0) return FP8IDX_OK;
  return check_ws(c.ws, c.ws_bytes, fp8idx::kRaggedQueueBytes);
}

fp8idx_status validate_logits_paged(const fp8idx_call_args& c) {
  if (fp8idx_status s = check_paged(c.q, c.kv, c.kv_scale, c.weights, c.row_len, c.block_table, c.B, c.next_n,
                                    c.H, c.D, c.page_size, c.max_pages, c.num_pages, c.width))
    return s;
  if (c.B > 0 && (!c.logits || !aligned(c.logits, 4) || c.ld_logits < c.width || c.ld_logits < 1))
    return FP8IDX_EINVAL;
  return FP8IDX_OK;
}

fp8idx_status validate_topk(const fp8idx_call_args& c) {
  if (fp8idx_status s = check_topk_args(c.rows, c.width, c.ld_logits, c.k, c.ld_out)) return s;
  if (fp8idx_status s = check_map(c.map)) return s;
  if (c.rows == 0) return FP8IDX_OK;
  if (!c.scores || !c.ke || !c.out || c.row0 < 0) return FP8IDX_EINVAL;
  if (!aligned(c.scores, 4) || !aligned(c.ke, 4) || !aligned(c.out, 4) || (c.ks && !aligned(c.ks, 4)))
    return FP8IDX_EINVAL;
  const fp8idx::TopkPlan plan = fp8idx::plan_topk(c.rows, c.width, c.k);
  if (!plan.supported) return FP8IDX_EUNSUPPORTED;
  return check_ws(c.ws, c.ws_bytes, fp8idx::topk_workspace_bytes(plan));
}

fp8idx_status validate_fused_ragged(const fp8idx_call_args& c, bool overlap) {
  if (fp8idx_status s = check_ragged(c.q, c.kv, c.kv_scale, c.weights, c.ks, c.ke, c.m, c.n, c.H, c.D)) return s;
  if (fp8idx_status s = check_topk_args(c.m, c.n, c.n, c.k, c.ld_out)) return s;
  if (fp8idx_status s = check_map(c.map)) return s;
  if (c.m == 0) return FP8IDX_OK;
  if (!c.out || !aligned(c.out, 4)) return FP8IDX_EINVAL;
  if (overlap && (c.side_stream == nullptr || c.side_stream == c.stream)) return FP8IDX_EINVAL;
  const FusedLayout L = fused_layout(c.m, c.n, c.k, c.logits_cap_bytes, 1, true, overlap ? 2 : 1);
  if (!L.ok) return FP8IDX_EUNSUPPORTED;
  return check_ws(c.ws, c.ws_bytes, L.total);
}

fp8idx_status validate_fused_paged(const fp8idx_call_args& c) {
  if (fp8idx_status s = check_paged(c.q, c.kv, c.kv_scale, c.weights, c.row_len, c.block_table, c.B, c.next_n,
                                    c.H, c.D, c.page_size, c.max_pages, c.num_pages, c.width))
    return s;
  const int32_t rows = (int32_t)((int64_t)c.B * c.next_n);
  if (fp8idx_status s = check_topk_args(rows, c.width, std::max<int64_t>(c.width, 1), c.k, c.ld_out)) return s;
  if (rows == 0) return FP8IDX_OK;
  if (!c.out || !aligned(c.out, 4)) return FP8IDX_EINVAL;
  const FusedLayout L = fused_layout(rows, c.width, c.k, c.logits_cap_bytes, c.next_n, false);
  if (!L.ok) return FP8IDX_EUNSUPPORTED;
  return check_ws(c.ws, c.ws_bytes, L.total);
}

fp8idx_call_args ragged_call(const uint8_t* q, const uint8_t* kv, const float* kv_scale, const float* weights,
                             const int32_t* ks, const int32_t* ke, int32_t m, int32_t n, int32_t H, int32_t D) {
  fp8idx_call_args c{};
  c.q = q;
  c.kv = kv;
  c.kv_scale = kv_scale;
  c.weights = weights;
  c.ks = ks;
  c.ke = ke;
  c.m = m;
  c.n = n;
  c.H = H;
  c.D = D;
  return c;
}

fp8idx_call_args paged_call(const uint8_t* q, const uint8_t* kv_pool, const float* scale_pool,
                            const float* weights, const int32_t* row_len, const int32_t* block_table, int32_t B,
                            int32_t next_n, int32_t H, int32_t D, int32_t page_size, int32_t max_pages,
                            int64_t num_pages, int32_t width) {
  fp8idx_call_args c{};
  c.q = q;
  c.kv = kv_pool;
  c.kv_scale = scale_pool;
  c.weights = weights;
  c.row_len = row_len;
  c.block_table = block_table;
  c.B = B;
  c.next_n = next_n;
  c.H = H;
  c.D = D;
  c.page_size = page_size;
  c.max_pages = max_pages;
  c.num_pages = num_pages;
  c.width = width;
  return c;
}

// The four ordering events of one overlapped call, created for the call and destroyed at its end.
// A wait enqueued on a stream keeps the event state at the time it was enqueued, and destroying an
// event whose recorded work is still pending is allowed (its resources go once that work ends), so
// nothing here outlives the call.
struct CallEvents {
  hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
  hipError_t create() {
    for (auto& e : ev) {
      const hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
      if (r != hipSuccess) {
        e = nullptr;
        return r;
      }
    }
    return hipSuccess;
  }
  ~CallEvents() {
    for (auto& e : ev)
      if (e) (void)hipEventDestroy(e);
  }
};

}  // namespace

extern "C" {

const char* fp8idx_status_string(int32_t status) {
  switch (status) {
    case FP8IDX_OK: return "FP8IDX_OK";
    case FP8IDX_EINVAL: return "FP8IDX_EINVAL: invalid argument (null pointer, size, stride or alignment)";
    case FP8IDX_EUNSUPPORTED: return "FP8IDX_EUNSUPPORTED: unsupported shape (H must be 32, D 128, page size 64, 1 <= k <= 16384)";
    case FP8IDX_EWORKSPACE: return "FP8IDX_EWORKSPACE: workspace smaller than fp8idx_workspace_bytes()";
    case FP8IDX_EDEVICE: return "FP8IDX_EDEVICE: no gfx950 device is current";
    case FP8IDX_EHIP: return "FP8IDX_EHIP: a HIP call failed (see fp8idx_last_hip_error)";
    default: return "FP8IDX: unknown status";
  }
}

int32_t fp8idx_last_hip_error(void) { return g_last_hip_error; }

const char* fp8idx_version(void) { return "fp8idx 0.1.0 gfx950"; }

int32_t fp8idx_rows_per_chunk(size_t logits_cap_bytes, int64_t width, int32_t rows) {
  return rows_per_chunk(logits_cap_bytes, ws_logits_ld(width), rows);
}

size_t fp8idx_sparse_mla_workspace_bytes(int32_t T, int32_t H, int32_t topk) {
  if (T <= 0 || H <= 0 || topk < 1) return 0;
  return fp8idx::plan_sparse_mla(T, H, topk).ws_bytes;
}

fp8idx_status indexer_sparse_mla(const uint16_t* q, const uint8_t* kv, const float* kv_scale, int64_t num_slots,
                                 const int32_t* indices, int64_t ld_indices, int32_t T, int32_t H, int32_t D,
                                 int32_t Dv, int32_t topk, float sm_scale, float* out, float* lse, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (D != fp8idx::kMlaDqk || Dv != fp8idx::kMlaDv || H <= 0 || H % 16 != 0) return FP8IDX_EUNSUPPORTED;
  if (T < 0 || topk < 1 || ld_indices < topk || num_slots < 1) return FP8IDX_EINVAL;
  if ((int64_t)T * H > INT32_MAX) return FP8IDX_EINVAL;
  if (T == 0) return FP8IDX_OK;
  if (!q || !kv || !kv_scale || !indices || !out) return FP8IDX_EINVAL;
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(out, 16) || !aligned(kv_scale, 4) || !aligned(indices, 4) ||
      (lse && !aligned(lse, 4)))
    return FP8IDX_EINVAL;
  const fp8idx::SparseMlaPlan plan = fp8idx::plan_sparse_mla(T, H, topk);
  if (plan.ws_bytes > 0 && (ws == nullptr || ws_bytes < plan.ws_bytes)) return FP8IDX_EWORKSPACE;
  if (plan.ws_bytes > 0 && !aligned(ws, 256)) return FP8IDX_EINVAL;
  DeviceInfo dev;
  if (fp8idx_status s = current_device(&dev)) return s;
  fp8idx::SparseMlaArgs a{q, kv, kv_scale, num_slots, indices, ld_indices, T, H, topk, sm_scale, out, lse};
  const hipError_t e = fp8idx::launch_sparse_mla(a, plan, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8IDX_OK : hip_fail(e);
}

size_t fp8idx_workspace_bytes(int32_t op, int32_t rows, int64_t width, int32_t k, size_t logits_cap_bytes) {
  if (op == FP8IDX_OP_LOGITS_RAGGED) return rows > 0 && width > 0 ? fp8idx::kRaggedQueueBytes : 0;
  if (rows <= 0 || width < 0 || k < 1 || k > fp8idx::kMaxK) return 0;
  switch (op) {
    case FP8IDX_OP_TOPK: {
      const fp8idx::TopkPlan p = fp8idx::plan_topk(rows, width, k);
      return p.supported ? fp8idx::topk_workspace_bytes(p) : 0;
    }
    case FP8IDX_OP_LOGITS_TOPK_RAGGED:
      return fused_layout(rows, width, k, logits_cap_bytes, 1, true).total;
    case FP8IDX_OP_LOGITS_TOPK_RAGGED_OVERLAP:
      return fused_layout(rows, width, k, logits_cap_bytes, 1, true, 2).total;
    default:
      return 0;
  }
}

fp8idx_status fp8idx_validate_only(int32_t entry, const fp8idx_call_args* args) {
  if (args == nullptr) return FP8IDX_EINVAL;
  switch (entry) {
    case FP8IDX_ENTRY_LOGITS_RAGGED: return validate_logits_ragged(*args);
    case FP8IDX_ENTRY_LOGITS_PAGED: return validate_logits_paged(*args);
    case FP8IDX_ENTRY_TOPK: return validate_topk(*args);
    case FP8IDX_ENTRY_LOGITS_TOPK_RAGGED: return validate_fused_ragged(*args, false);
    case FP8IDX_ENTRY_LOGITS_TOPK_RAGGED_OVERLAP: return validate_fused_ragged(*args, true);
    case FP8IDX_ENTRY_LOGITS_TOPK_PAGED: return validate_fused_paged(*args);
    default: return FP8IDX_EINVAL;
  }
}

fp8idx_status indexer_prepare_ragged(const int32_t* seq_len, const int32_t* q_len, const int32_t* req_idx,
                                     const int32_t* table, int64_t ld_table, int32_t num_table_rows, int32_t B,
                                     int32_t* cu_seq, int32_t* cu_q, int32_t* ks, int32_t* ke, int64_t max_q,
                                     int32_t* ragged_mem, int64_t max_keys, void* stream) {
  if (B < 0 || max_q < 0 || max_keys < 0 || num_table_rows < 0) return FP8IDX_EINVAL;
  if (B > fp8idx::kPrepMaxReq) return FP8IDX_EUNSUPPORTED;
  if (B == 0) return FP8IDX_OK;
  if (!seq_len || !q_len || !req_idx || !cu_seq || !cu_q) return FP8IDX_EINVAL;
  if (max_q > 0 && (!ks || !ke)) return FP8IDX_EINVAL;
  if (ragged_mem && (!table || ld_table < 1)) return FP8IDX_EINVAL;
  for (const void* p : {(const void*)seq_len, (const void*)q_len, (const void*)req_idx, (const void*)cu_seq,
                        (const void*)cu_q, (const void*)ks, (const void*)ke, (const void*)table,
                        (const void*)ragged_mem})
    if (p && !aligned(p, 4)) return FP8IDX_EINVAL;
  DeviceInfo dev;
  if (fp8idx_status s = current_device(&dev)) return s;
  fp8idx::PrepRaggedArgs a{seq_len, q_len, req_idx, table, ld_table, num_table_rows, B, cu_seq, cu_q,
                           ks, ke, max_q, ragged_mem, ragged_mem ? max_keys : 0};
  const hipError_t e = fp8idx::launch_prep_ragged(a, dev, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8IDX_OK : hip_fail(e);
}

fp8idx_status indexer_prepare_decode(const int32_t* seq_len, const int32_t* req_idx, const int32_t* req_to_page,
                                     int64_t ld_req_to_page, int32_t num_table_rows, int32_t B, int32_t next_n,
                                     int32_t* row_len, int32_t* block_table, int32_t max_pages, void* stream) {
  if (B < 0 || next_n < 1 || max_pages < 0 || num_table_rows < 0 || ld_req_to_page < max_pages)
    return FP8IDX_EINVAL;
  if ((int64_t)B * next_n > 0x7fffffffLL) return FP8IDX_EUNSUPPORTED;
  if (B == 0) return FP8IDX_OK;
  if (!seq_len || !req_idx || !row_len || (max_pages > 0 && (!req_to_page || !block_table))) return FP8IDX_EINVAL;
  for (const void* p : {(const void*)seq_len, (const void*)req_idx, (const void*)req_to_page, (const void*)row_len,
                        (const void*)block_table})
    if (p && !aligned(p, 4)) return FP8IDX_EINVAL;
  DeviceInfo dev;
  if (fp8idx_status s = current_device(&dev)) return s;
  fp8idx::PrepDecodeArgs a{seq_len, req_idx, req_to_page, ld_req_to_page, num_table_rows, B, next_n,
                           row_len, block_table, max_pages, max_pages};
  const hipError_t e = fp8idx::launch_prep_decode(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8IDX_OK : hip_fail(e);
}

fp8idx_status fp8idx_probe_mfma_fp8(int32_t blocks, int32_t iters, float* out, double* flops, void* stream) {
  if (blocks <= 0 || iters <= 0 || !out || !aligned(out, 4)) return FP8IDX_EINVAL;
  DeviceInfo dev;
  if (fp8idx_status s = current_device(&dev)) return s;
  if (flops) *flops = (double)blocks * (fp8idx::kProbeThreads / 64) * (double)iters * fp8idx::kProbeChains * 65536.0;
  const hipError_t e = fp8idx::launch_mfma_probe(blocks, iters, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8IDX_OK : hip_fail(e);
}

fp8idx_status fp8idx_probe_logits_core(int32_t blocks, int32_t iters, float* out, double* flops, void* stream) {
  if (blocks <= 0 || iters <= 0 || !out || !aligned(out, 4)) return FP8IDX_EINVAL;
  DeviceInfo dev;
  if (fp8idx_status s = current_device(&dev)) return s;
  if (flops) *flops = (double)blocks * (fp8idx::kProbeThreads / 64) * (double)iters * 8.0 * 65536.0;
  const hipError_t e = fp8idx::launch_logits_core_probe(blocks, iters, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8IDX_OK : hip_fail(e);
}

fp8idx_status indexer_quant_fp8(const float* x, int64_t ld_x, int64_t rows, int32_t D, uint8_t* codes,
                                int64_t ld_codes, float* scale, void* stream) {
  if (D < 4 || D > 2048 || D % 4 != 0) return FP8IDX_EUNSUPPORTED;
  if (rows < 0) return FP8IDX_EINVAL;
  if (rows == 0) return FP8IDX_OK;
  if (!x || !codes || !scale) return FP8IDX_EINVAL;
  if (!aligned(x, 16) || ld_x < D || ld_x % 4 != 0) return FP8IDX_EINVAL;
  if (!aligned(codes, 4) || ld_codes < D || ld_codes % 4 != 0 || !aligned(scale, 4)) return FP8IDX_EINVAL;
  DeviceInfo dev;
  if (fp8idx_status s = current_device(&dev)) return s;
  fp8idx::QuantArgs a{x, ld_x, rows, D, codes, ld_codes, scale};
  const hipError_t e = fp8idx::launch_quant_fp8(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8IDX_OK : hip_fail(e);
}

fp8idx_status indexer_logits_ragged(const uint8_t* q, const uint8_t* kv, const float* kv_scale,
                                    const float* weights, const int32_t* ks, const int32_t* ke,
                                    int32_t m, int32_t n, int32_t H, int32_t D,
                                    float* logits, int64_t ld_logits, int32_t clean, void* ws, size_t ws_bytes,
                                    void* stream) {
  fp8idx_call_args c = ragged_call(q, kv, kv_scale, weights, ks, ke, m, n, H, D);
  c.logits = logits;
  c.ld_logits = ld_logits;
  c.clean = clean;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  if (fp8idx_status s = validate_logits_ragged(c)) return s;
  if (m == 0) return FP8IDX_OK;
  DeviceInfo dev;
  if (fp8idx_status s = current_device(&dev)) return s;
  fp8idx::RaggedLogitsArgs a{q, kv, kv_scale, weights, ks, ke, m, n, logits, ld_logits, clean,
                             static_cast<unsigned int*>(ws)};
  const hipError_t e = fp8idx::launch_logits_ragged(a, dev, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8IDX_OK : hip_fail(e);
}

fp8idx_status indexer_logits_ragged_noalloc(const uint8_t* q, const uint8_t* kv, const float* kv_scale,
                                            const float* weights, const int32_t* ks, const int32_t* ke, int32_t m,
                                            int32_t n, int32_t H, int32_t D, float* logits, int64_t ld_logits,
                                            int32_t clean, void* stream) {
  fp8idx_call_args c = ragged_call(q, kv, kv_scale, weights, ks, ke, m, n, H, D);
  c.logits = logits;
  c.ld_logits = ld_logits;
  c.clean = clean;
  if (fp8idx_status s = validate_logits_ragged_io(c)) return s;
  if (m == 0) return FP8IDX_OK;
  DeviceInfo dev;
  if (fp8idx_status s = current_device(&dev)) return s;
  unsigned int* queue = nullptr;
  if (hipError_t e = fp8idx::ragged_noalloc_queue(&queue)) return hip_fail(e);
  fp8idx::RaggedLogitsArgs a{q, kv, kv_scale, weights, ks, ke, m, n, logits, ld_logits, clean, queue};
  const hipError_t e = fp8idx::launch_logits_ragged(a, dev, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8IDX_OK : hip_fail(e);
}

fp8idx_status indexer_logits_paged(const uint8_t* q, const uint8_t* kv_pool, const float* scale_pool,
                                   const float* weights, const int32_t* row_len, const int32_t* block_table,
                                   int32_t B, int32_t next_n, int32_t H, int32_t D, int32_t page_size,
                                   int32_t max_pages, int64_t num_pages, float* logits, int64_t ld_logits,
                                   int32_t width, int32_t clean, void* stream) {
  fp8idx_call_args c = paged_call(q, kv_pool, scale_pool, weights, row_len, block_table, B, next_n, H, D,
                                  page_size, max_pages, num_pages, width);
  c.logits = logits;
  c.ld_logits = ld_logits;
  c.clean = clean;
  if (fp8idx_status s = validate_logits_paged(c)) return s;
  if (B == 0 || width == 0) return FP8IDX_OK;
  DeviceInfo dev;
  if (fp8idx_status s = current_device(&dev)) return s;
  fp8idx::PagedLogitsArgs a{q, kv_pool, scale_pool, weights, row_len, block_table, B, next_n, max_pages,
                            num_pages, logits, ld_logits, width, clean};
  const hipError_t e = fp8idx::launch_logits_paged(a, dev, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8IDX_OK : hip_fail(e);
}

fp8idx_status indexer_topk(const float* logits, int64_t ld, int32_t rows, int32_t width, const int32_t* ks,
                           const int32_t* ke, int32_t k, int32_t row0, const fp8idx_map* map, int32_t* out,
                           int64_t ld_out, void* ws, size_t ws_bytes, void* stream) {
  fp8idx_call_args c{};
  c.scores = logits;
  c.ld_logits = ld;
  c.rows = rows;
  c.width = width;
  c.ks = ks;
  c.ke = ke;
  c.k = k;
  c.row0 = row0;
  c.map = map;
  c.out = out;
  c.ld_out = ld_out;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  if (fp8idx_status s = validate_topk(c)) return s;
  if (rows == 0) return FP8IDX_OK;
  DeviceInfo dev;
  if (fp8idx_status s = current_device(&dev)) return s;
  const fp8idx::TopkPlan plan = fp8idx::plan_topk(rows, width, k);
  fp8idx::TopkArgs a{logits, ld, rows, width, ks, ke, k, row0, to_kernel_map(map), out, ld_out};
  const hipError_t e = fp8idx::launch_topk(a, plan, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8IDX_OK : hip_fail(e);
}

fp8idx_status indexer_logits_topk_ragged(const uint8_t* q, const uint8_t* kv, const float* kv_scale,
                                         const float* weights, const int32_t* ks, const int32_t* ke, int32_t m,
                                         int32_t n, int32_t H, int32_t D, int32_t k, const fp8idx_map* map,
                                         int32_t* out, int64_t ld_out, size_t logits_cap_bytes, void* ws,
                                         size_t ws_bytes, void* stream) {
  fp8idx_call_args c = ragged_call(q, kv, kv_scale, weights, ks, ke, m, n, H, D);
  c.k = k;
  c.map = map;
  c.out = out;
  c.ld_out = ld_out;
  c.logits_cap_bytes = logits_cap_bytes;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  if (fp8idx_status s = validate_fused_ragged(c, false)) return s;
  if (m == 0) return FP8IDX_OK;
  DeviceInfo dev;
  if (fp8idx_status s = current_device(&dev)) return s;

  const hipStream_t st = static_cast<hipStream_t>(stream);
  const FusedLayout L = fused_layout(m, n, k, logits_cap_bytes, 1, true);
  const int64_t ld = ws_logits_ld(n);
  const int32_t rpc = L.rpc;
  uint8_t* w = static_cast<uint8_t*>(ws);
  unsigned int* queue = reinterpret_cast<unsigned int*>(w);
  float* chunk_logits = reinterpret_cast<float*>(w + L.queue_bytes);
  void* topk_ws = w + L.queue_bytes + L.buf_bytes;
  const fp8idx::TopkMap kmap = to_kernel_map(map);
  for (int32_t s0 = 0; s0 < m; s0 += rpc) {
    const int32_t rows = std::min(rpc, m - s0);
    fp8idx::RaggedLogitsArgs la{q + (size_t)s0 * fp8idx::kQRowBytesHost, kv, kv_scale,
                                weights + (size_t)s0 * 32, ks + s0, ke + s0, rows, n, chunk_logits, ld, 0, queue};
    hipError_t e = fp8idx::launch_logits_ragged(la, dev, st);
    if (e != hipSuccess) return hip_fail(e);
    const fp8idx::TopkPlan plan = fp8idx::plan_topk(rows, n, k);
    fp8idx::TopkArgs ta{chunk_logits, ld, rows, n, ks + s0, ke + s0, k, s0, kmap, out + (int64_t)s0 * ld_out, ld_out};
    e = fp8idx::launch_topk(ta, plan, topk_ws, st);
    if (e != hipSuccess) return hip_fail(e);
  }
  return FP8IDX_OK;
}

fp8idx_status indexer_logits_topk_ragged_overlap(const uint8_t* q, const uint8_t* kv, const float* kv_scale,
                                                 const float* weights, const int32_t* ks, const int32_t* ke,
                                                 int32_t m, int32_t n, int32_t H, int32_t D, int32_t k,
                                                 const fp8idx_map* map, int32_t* out, int64_t ld_out,
                                                 size_t logits_cap_bytes, void* ws, size_t ws_bytes, void* stream,
                                                 void* side_stream) {
  fp8idx_call_args c = ragged_call(q, kv, kv_scale, weights, ks, ke, m, n, H, D);
  c.k = k;
  c.map = map;
  c.out = out;
  c.ld_out = ld_out;
  c.logits_cap_bytes = logits_cap_bytes;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  c.stream = stream;
  c.side_stream = side_stream;
  if (fp8idx_status s = validate_fused_ragged(c, true)) return s;
  if (m == 0) return FP8IDX_OK;
  DeviceInfo dev;
  if (fp8idx_status s = current_device(&dev)) return s;
  CallEvents events;
  if (hipError_t e = events.create()) return hip_fail(e);
  hipEvent_t* ev = events.ev;

  const hipStream_t main_st = static_cast<hipStream_t>(stream);
  const hipStream_t side = static_cast<hipStream_t>(side_stream);
  const FusedLayout L = fused_layout(m, n, k, logits_cap_bytes, 1, true, 2);
  const int64_t ld = ws_logits_ld(n);
  const int32_t rpc = L.rpc;
  const int32_t nchunks = (m + rpc - 1) / rpc;
  uint8_t* w = static_cast<uint8_t*>(ws);
  unsigned int* queue = reinterpret_cast<unsigned int*>(w);
  float* bufs[2] = {reinterpret_cast<float*>(w + L.queue_bytes),
                    reinterpret_cast<float*>(w + L.queue_bytes + (L.buffers > 1 ? L.buf_bytes : 0))};
  void* topk_ws = w + L.queue_bytes + L.buf_bytes * (size_t)L.buffers;
  const fp8idx::TopkMap kmap = to_kernel_map(map);
  hipError_t e = hipSuccess;
  for (int32_t ci = 0; ci < nchunks; ++ci) {
    const int32_t s0 = ci * rpc;
    const int32_t rows = std::min(rpc, m - s0);
    const int b = ci & 1;
    // the top-k of chunk ci - 2 must have read this buffer before it is rewritten
    if (ci >= 2 && (e = hipStreamWaitEvent(main_st, ev[2 + b], 0)) != hipSuccess) return hip_fail(e);
    // the logits launches all run on the main stream, one after another, so they share one counter set;
    // after the first chunk, one workgroup slot per CU is left to the previous chunk's top-k
    fp8idx::RaggedLogitsArgs la{q + (size_t)s0 * fp8idx::kQRowBytesHost, kv, kv_scale,
                                weights + (size_t)s0 * 32, ks + s0, ke + s0, rows, n, bufs[b], ld, 0, queue,
                                ci > 0 ? std::max(1, dev.ragged_wgs_per_cu - 1) : 0};
    if ((e = fp8idx::launch_logits_ragged(la, dev, main_st)) != hipSuccess) return hip_fail(e);
    if ((e = hipEventRecord(ev[b], main_st)) != hipSuccess) return hip_fail(e);
    if ((e = hipStreamWaitEvent(side, ev[b], 0)) != hipSuccess) return hip_fail(e);
    const fp8idx::TopkPlan plan = fp8idx::plan_topk(rows, n, k);
    fp8idx::TopkArgs ta{bufs[b], ld, rows, n, ks + s0, ke + s0, k, s0, kmap, out + (int64_t)s0 * ld_out, ld_out};
    if ((e = fp8idx::launch_topk(ta, plan, topk_ws, side)) != hipSuccess) return hip_fail(e);
    if ((e = hipEventRecord(ev[2 + b], side)) != hipSuccess) return hip_fail(e);
  }
  // join: the side stream runs the top-ks in order, so the last one implies all
  if ((e = hipStreamWaitEvent(main_st, ev[2 + ((nchunks - 1) & 1)], 0)) != hipSuccess) return hip_fail(e);
  return FP8IDX_OK;
}

fp8idx_status indexer_logits_topk_paged(const uint8_t* q, const uint8_t* kv_pool, const float* scale_pool,
                                        const float* weights, const int32_t* row_len, const int32_t* block_table,
                                        int32_t B, int32_t next_n, int32_t H, int32_t D, int32_t page_size,
                                        int32_t max_pages, int64_t num_pages, int32_t width, int32_t k,
                                        int32_t map_to_slots, int32_t* out, int64_t ld_out,
                                        size_t logits_cap_bytes, void* ws, size_t ws_bytes, void* stream) {
  fp8idx_call_args c = paged_call(q, kv_pool, scale_pool, weights, row_len, block_table, B, next_n, H, D,
                                  page_size, max_pages, num_pages, width);
  c.k = k;
  c.map_to_slots = map_to_slots;
  c.out = out;
  c.ld_out = ld_out;
  c.logits_cap_bytes = logits_cap_bytes;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  if (fp8idx_status s = validate_fused_paged(c)) return s;
  const int32_t rows = (int32_t)((int64_t)B * next_n);
  if (rows == 0) return FP8IDX_OK;
  DeviceInfo dev;
  if (fp8idx_status s = current_device(&dev)) return s;

  const hipStream_t st = static_cast<hipStream_t>(stream);
  const FusedLayout L = fused_layout(rows, width, k, logits_cap_bytes, next_n, false);
  const int64_t ld = ws_logits_ld(width);
  const int32_t rpc = L.rpc;
  const int32_t req_per_chunk = std::max<int32_t>(1, rpc / next_n);
  float* chunk_logits = static_cast<float*>(ws);
  uint32_t* frag_max = L.frag_bytes ? reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + L.buf_bytes) : nullptr;
  void* topk_ws = static_cast<uint8_t*>(ws) + L.buf_bytes + L.frag_bytes;
  fp8idx::TopkMap kmap{};
  if (map_to_slots) {
    kmap.kind = FP8IDX_MAP_BLOCK_TABLE;
    kmap.table = block_table;
    kmap.ld = max_pages;
    kmap.num_req = B;
    kmap.rows_per_req = next_n;
    kmap.page_size = page_size;
    kmap.num_pages = num_pages;
  } else {
    kmap.kind = FP8IDX_MAP_NONE;
  }
  for (int32_t b0 = 0; b0 < B; b0 += req_per_chunk) {
    const int32_t nb = std::min(req_per_chunk, B - b0);
    const int32_t r0 = b0 * next_n;
    const int32_t nr = nb * next_n;
    // the top-k of a chunk whose rows each take one workgroup starts from the logits kernel's
    // per-fragment maxima
    const fp8idx::TopkPlan plan = fp8idx::plan_topk(nr, width, k);
    uint32_t* fm = fp8idx::topk_plan_takes_frag_max(plan) ? frag_max : nullptr;
    fp8idx::FragLayout fl = fp8idx::paged_frag_layout(nb, next_n, max_pages, width);
    fl.elems = L.frag_elems;
    fp8idx::PagedLogitsArgs la{q + (size_t)r0 * fp8idx::kQRowBytesHost, kv_pool, scale_pool,
                               weights + (size_t)r0 * 32, row_len + r0, block_table + (int64_t)b0 * max_pages,
                               nb, next_n, max_pages, num_pages, chunk_logits, ld, width, 0, fm, fl};
    hipError_t e = fp8idx::launch_logits_paged(la, dev, st);
    if (e != hipSuccess) return hip_fail(e);
    fp8idx::TopkArgs ta{chunk_logits, ld, nr, width, nullptr, row_len + r0, k, r0, kmap,
                        out + (int64_t)r0 * ld_out, ld_out, fm, fl, next_n};
    e = fp8idx::launch_topk(ta, plan, topk_ws, st);
    if (e != hipSuccess) return hip_fail(e);
  }
  return FP8IDX_OK;
}

size_t fp8idx_workspace_bytes_paged(int32_t B, int32_t next_n, int32_t width, int32_t k, size_t logits_cap_bytes) {
  if (B <= 0 || next_n <= 0 || width < 0 || k < 1 || k > fp8idx::kMaxK) return 0;
  if ((int64_t)B * next_n > INT32_MAX) return 0;   // the entry rejects such a call
  return fused_layout(B * next_n, width, k, logits_cap_bytes, next_n, false).total;
}

}  // extern "C"
