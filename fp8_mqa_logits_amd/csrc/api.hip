// C ABI of the fp8 MQA indexer library: argument validation, device checks,
// workspace arithmetic and the row-chunked fused loop.  Every kernel launch
// goes on the caller's stream; nothing here allocates or synchronises.

#include <fp8idx.h>

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
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
      if (!map->table || map->ld < 1 || map->num_req < 1 || map->rows_per_req < 1 || map->page_size < 1)
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

// Events of the overlapped fused entry, created once per device: [0..1] a
// chunk buffer's logits are written, [2..3] its top-k has read them.
std::once_flag g_ev_once[kMaxDevices];
hipEvent_t g_ev[kMaxDevices][4];
int g_ev_ok[kMaxDevices];

fp8idx_status overlap_events(hipEvent_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8IDX_EDEVICE;
  std::call_once(g_ev_once[dev], [dev]() {
    g_ev_ok[dev] = 1;
    for (int i = 0; i < 4; ++i)
      if (hipEventCreateWithFlags(&g_ev[dev][i], hipEventDisableTiming) != hipSuccess) g_ev_ok[dev] = 0;
  });
  if (!g_ev_ok[dev]) return FP8IDX_EHIP;
  *out = g_ev[dev];
  return FP8IDX_OK;
}

size_t fused_ws_bytes(int32_t rows, int64_t width, int32_t k, size_t cap, int32_t granule,
                      int32_t logit_buffers = 1) {
  const int64_t ld = ws_logits_ld(width);
  int32_t rpc = rows_per_chunk(cap, ld, rows);
  if (granule > 1 && rpc < rows) rpc = std::max<int32_t>(granule, rpc / granule * granule);
  rpc = std::min(rpc, rows);
  if (rpc <= 0) return 0;
  const int32_t last = rows % rpc == 0 ? rpc : rows % rpc;
  const size_t logits = align256((size_t)rpc * (size_t)ld * 4u) * (size_t)(rpc < rows ? logit_buffers : 1);
  const size_t t0 = fp8idx::topk_workspace_bytes(fp8idx::plan_topk(rpc, width, k));
  const size_t t1 = fp8idx::topk_workspace_bytes(fp8idx::plan_topk(last, width, k));
  return logits + std::max(t0, t1);
}

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
  if (rows <= 0 || width < 0 || k < 1 || k > fp8idx::kMaxK) return 0;
  switch (op) {
    case FP8IDX_OP_TOPK:
      return fp8idx::topk_workspace_bytes(fp8idx::plan_topk(rows, width, k));
    case FP8IDX_OP_LOGITS_TOPK_RAGGED:
      return fused_ws_bytes(rows, width, k, logits_cap_bytes, 1);
    case FP8IDX_OP_LOGITS_TOPK_RAGGED_OVERLAP:
      return fused_ws_bytes(rows, width, k, logits_cap_bytes, 1, 2);
    default:
      return 0;
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
                                    float* logits, int64_t ld_logits, int32_t clean, void* stream) {
  if (fp8idx_status s = check_ragged(q, kv, kv_scale, weights, ks, ke, m, n, H, D)) return s;
  if (m > 0 && (!logits || !aligned(logits, 4) || ld_logits < n)) return FP8IDX_EINVAL;
  if (m == 0) return FP8IDX_OK;
  DeviceInfo dev;
  if (fp8idx_status s = current_device(&dev)) return s;
  fp8idx::RaggedLogitsArgs a{q, kv, kv_scale, weights, ks, ke, m, n, logits, ld_logits, clean};
  const hipError_t e = fp8idx::launch_logits_ragged(a, dev, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8IDX_OK : hip_fail(e);
}

fp8idx_status indexer_logits_paged(const uint8_t* q, const uint8_t* kv_pool, const float* scale_pool,
                                   const float* weights, const int32_t* row_len, const int32_t* block_table,
                                   int32_t B, int32_t next_n, int32_t H, int32_t D, int32_t page_size,
                                   int32_t max_pages, int64_t num_pages, float* logits, int64_t ld_logits,
                                   int32_t width, int32_t clean, void* stream) {
  if (fp8idx_status s = check_paged(q, kv_pool, scale_pool, weights, row_len, block_table, B, next_n, H, D,
                                    page_size, max_pages, num_pages, width))
    return s;
  if (B > 0 && (!logits || !aligned(logits, 4) || ld_logits < width || ld_logits < 1)) return FP8IDX_EINVAL;
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
  if (fp8idx_status s = check_topk_args(rows, width, ld, k, ld_out)) return s;
  if (fp8idx_status s = check_map(map)) return s;
  if (rows == 0) return FP8IDX_OK;
  if (!logits || !ke || !out || row0 < 0) return FP8IDX_EINVAL;
  if (!aligned(logits, 4) || !aligned(ke, 4) || !aligned(out, 4) || (ks && !aligned(ks, 4))) return FP8IDX_EINVAL;
  const fp8idx::TopkPlan plan = fp8idx::plan_topk(rows, width, k);
  const size_t need = fp8idx::topk_workspace_bytes(plan);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return FP8IDX_EWORKSPACE;
  if (need > 0 && !aligned(ws, 256)) return FP8IDX_EINVAL;
  DeviceInfo dev;
  if (fp8idx_status s = current_device(&dev)) return s;
  fp8idx::TopkArgs a{logits, ld, rows, width, ks, ke, k, row0, to_kernel_map(map), out, ld_out};
  const hipError_t e = fp8idx::launch_topk(a, plan, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8IDX_OK : hip_fail(e);
}

fp8idx_status indexer_logits_topk_ragged(const uint8_t* q, const uint8_t* kv, const float* kv_scale,
                                         const float* weights, const int32_t* ks, const int32_t* ke, int32_t m,
                                         int32_t n, int32_t H, int32_t D, int32_t k, const fp8idx_map* map,
                                         int32_t* out, int64_t ld_out, size_t logits_cap_bytes, void* ws,
                                         size_t ws_bytes, void* stream) {
  if (fp8idx_status s = check_ragged(q, kv, kv_scale, weights, ks, ke, m, n, H, D)) return s;
  if (fp8idx_status s = check_topk_args(m, n, n, k, ld_out)) return s;
  if (fp8idx_status s = check_map(map)) return s;
  if (m == 0) return FP8IDX_OK;
  if (!out || !aligned(out, 4)) return FP8IDX_EINVAL;
  const size_t need = fused_ws_bytes(m, n, k, logits_cap_bytes, 1);
  if (ws == nullptr || ws_bytes < need) return FP8IDX_EWORKSPACE;
  if (!aligned(ws, 256)) return FP8IDX_EINVAL;
  DeviceInfo dev;
  if (fp8idx_status s = current_device(&dev)) return s;

  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t ld = ws_logits_ld(n);
  const int32_t rpc = rows_per_chunk(logits_cap_bytes, ld, m);
  float* chunk_logits = static_cast<float*>(ws);
  void* topk_ws = static_cast<uint8_t*>(ws) + align256((size_t)rpc * (size_t)ld * 4u);
  const fp8idx::TopkMap kmap = to_kernel_map(map);
  for (int32_t s0 = 0; s0 < m; s0 += rpc) {
    const int32_t rows = std::min(rpc, m - s0);
    fp8idx::RaggedLogitsArgs la{q + (size_t)s0 * fp8idx::kQRowBytesHost, kv, kv_scale,
                                weights + (size_t)s0 * 32, ks + s0, ke + s0, rows, n, chunk_logits, ld, 0};
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
  if (fp8idx_status s = check_ragged(q, kv, kv_scale, weights, ks, ke, m, n, H, D)) return s;
  if (fp8idx_status s = check_topk_args(m, n, n, k, ld_out)) return s;
  if (fp8idx_status s = check_map(map)) return s;
  if (m == 0) return FP8IDX_OK;
  if (!out || !aligned(out, 4)) return FP8IDX_EINVAL;
  if (side_stream == nullptr || side_stream == stream) return FP8IDX_EINVAL;
  const size_t need = fused_ws_bytes(m, n, k, logits_cap_bytes, 1, 2);
  if (ws == nullptr || ws_bytes < need) return FP8IDX_EWORKSPACE;
  if (!aligned(ws, 256)) return FP8IDX_EINVAL;
  DeviceInfo dev;
  if (fp8idx_status s = current_device(&dev)) return s;
  hipEvent_t* ev = nullptr;
  if (fp8idx_status s = overlap_events(&ev)) return s;

  const hipStream_t main_st = static_cast<hipStream_t>(stream);
  const hipStream_t side = static_cast<hipStream_t>(side_stream);
  const int64_t ld = ws_logits_ld(n);
  const int32_t rpc = rows_per_chunk(logits_cap_bytes, ld, m);
  const int32_t nchunks = (m + rpc - 1) / rpc;
  const size_t buf_bytes = align256((size_t)rpc * (size_t)ld * 4u);
  float* bufs[2] = {static_cast<float*>(ws),
                    reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + (nchunks > 1 ? buf_bytes : 0))};
  void* topk_ws = static_cast<uint8_t*>(ws) + buf_bytes * (nchunks > 1 ? 2 : 1);
  const fp8idx::TopkMap kmap = to_kernel_map(map);
  hipError_t e = hipSuccess;
  for (int32_t c = 0; c < nchunks; ++c) {
    const int32_t s0 = c * rpc;
    const int32_t rows = std::min(rpc, m - s0);
    const int b = c & 1;
    // the top-k of chunk c - 2 must have read this buffer before it is rewritten
    if (c >= 2 && (e = hipStreamWaitEvent(main_st, ev[2 + b], 0)) != hipSuccess) return hip_fail(e);
    fp8idx::RaggedLogitsArgs la{q + (size_t)s0 * fp8idx::kQRowBytesHost, kv, kv_scale,
                                weights + (size_t)s0 * 32, ks + s0, ke + s0, rows, n, bufs[b], ld, 0};
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
  if (fp8idx_status s = check_paged(q, kv_pool, scale_pool, weights, row_len, block_table, B, next_n, H, D,
                                    page_size, max_pages, num_pages, width))
    return s;
  const int64_t rows64 = (int64_t)B * next_n;
  const int32_t rows = (int32_t)rows64;
  if (fp8idx_status s = check_topk_args(rows, width, std::max<int64_t>(width, 1), k, ld_out)) return s;
  if (rows == 0) return FP8IDX_OK;
  if (!out || !aligned(out, 4)) return FP8IDX_EINVAL;
  const size_t need = fused_ws_bytes(rows, width, k, logits_cap_bytes, next_n);
  if (ws == nullptr || ws_bytes < need) return FP8IDX_EWORKSPACE;
  if (!aligned(ws, 256)) return FP8IDX_EINVAL;
  DeviceInfo dev;
  if (fp8idx_status s = current_device(&dev)) return s;

  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t ld = ws_logits_ld(width);
  int32_t rpc = rows_per_chunk(logits_cap_bytes, ld, rows);
  if (rpc < rows) rpc = std::max<int32_t>(next_n, rpc / next_n * next_n);
  rpc = std::min(rpc, rows);
  const int32_t req_per_chunk = std::max<int32_t>(1, rpc / next_n);
  float* chunk_logits = static_cast<float*>(ws);
  void* topk_ws = static_cast<uint8_t*>(ws) + align256((size_t)rpc * (size_t)ld * 4u);
  fp8idx::TopkMap kmap{};
  if (map_to_slots) {
    kmap.kind = FP8IDX_MAP_BLOCK_TABLE;
    kmap.table = block_table;
    kmap.ld = max_pages;
    kmap.num_req = B;
    kmap.rows_per_req = next_n;
    kmap.page_size = page_size;
  } else {
    kmap.kind = FP8IDX_MAP_NONE;
  }
  for (int32_t b0 = 0; b0 < B; b0 += req_per_chunk) {
    const int32_t nb = std::min(req_per_chunk, B - b0);
    const int32_t r0 = b0 * next_n;
    const int32_t nr = nb * next_n;
    fp8idx::PagedLogitsArgs la{q + (size_t)r0 * fp8idx::kQRowBytesHost, kv_pool, scale_pool,
                               weights + (size_t)r0 * 32, row_len + r0, block_table + (int64_t)b0 * max_pages,
                               nb, next_n, max_pages, num_pages, chunk_logits, ld, width, 0};
    hipError_t e = fp8idx::launch_logits_paged(la, dev, st);
    if (e != hipSuccess) return hip_fail(e);
    const fp8idx::TopkPlan plan = fp8idx::plan_topk(nr, width, k);
    fp8idx::TopkArgs ta{chunk_logits, ld, nr, width, nullptr, row_len + r0, k, r0, kmap,
                        out + (int64_t)r0 * ld_out, ld_out};
    e = fp8idx::launch_topk(ta, plan, topk_ws, st);
    if (e != hipSuccess) return hip_fail(e);
  }
  return FP8IDX_OK;
}

size_t fp8idx_workspace_bytes_paged(int32_t B, int32_t next_n, int32_t width, int32_t k, size_t logits_cap_bytes) {
  if (B <= 0 || next_n <= 0 || width < 0 || k < 1 || k > fp8idx::kMaxK) return 0;
  return fused_ws_bytes(B * next_n, width, k, logits_cap_bytes, next_n);
}

}  // extern "C"
