"""ctypes binding of libfp8idx.so, the C ABI declared in include/fp8idx.h.

Argument marshalling only: each function checks the dtype, shape (or
element count), contiguity and device of every torch tensor against the
sizes the call implies (the C ABI takes bare pointers and cannot see how
large a buffer is), raising ``ValueError`` before anything is launched; it
then takes their device pointers and the current HIP stream, calls the C
entry point of the same name and raises ``Fp8idxError`` on a non-OK status.  Output and workspace tensors the caller
does not pass are allocated here with torch (device memory is the only thing
torch provides); every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library is not built, or the device
is not a gfx950, the call raises.
"""

from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8idx.so")

H = 32
D = 128

STATUS_NAMES = {0: "OK", 1: "EINVAL", 2: "EUNSUPPORTED", 3: "EWORKSPACE", 4: "EDEVICE", 5: "EHIP"}
MAP_NONE, MAP_TOKEN_TABLE, MAP_BLOCK_TABLE = 0, 1, 2
OP_TOPK, OP_LOGITS_TOPK_RAGGED, OP_LOGITS_TOPK_RAGGED_OVERLAP, OP_LOGITS_RAGGED = 0, 1, 2, 3
(ENTRY_LOGITS_RAGGED, ENTRY_LOGITS_PAGED, ENTRY_TOPK, ENTRY_LOGITS_TOPK_RAGGED,
 ENTRY_LOGITS_TOPK_RAGGED_OVERLAP, ENTRY_LOGITS_TOPK_PAGED) = range(6)

EXPORTED = (
    "indexer_logits_ragged", "indexer_logits_paged", "indexer_topk",
    "indexer_logits_topk_ragged", "indexer_logits_topk_paged",
    "fp8idx_workspace_bytes", "fp8idx_workspace_bytes_paged", "fp8idx_rows_per_chunk",
    "fp8idx_status_string", "fp8idx_last_hip_error", "fp8idx_version",
    "indexer_quant_fp8", "indexer_logits_topk_ragged_overlap",
    "indexer_prepare_ragged", "indexer_prepare_decode",
    "indexer_sparse_mla", "fp8idx_sparse_mla_workspace_bytes", "fp8idx_probe_mfma_fp8", "fp8idx_probe_logits_core",
    "fp8idx_validate_only", "indexer_logits_ragged_noalloc",
)

MLA_DQK = 576   # sparse MLA KV row: 512 latent + 64 rotary values
MLA_DV = 512


class Fp8idxError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg}")
        self.status = status


class _CMap(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("table", ctypes.c_void_p),
        ("ld", ctypes.c_int64),
        ("num_req", ctypes.c_int32),
        ("cu_rows", ctypes.c_void_p),
        ("rows_per_req", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
    ]


class CallArgs(ctypes.Structure):
    """fp8idx_call_args: the arguments of one indexer call, for fp8idx_validate_only()."""

    _fields_ = [
        ("q", ctypes.c_void_p), ("kv", ctypes.c_void_p), ("kv_scale", ctypes.c_void_p),
        ("weights", ctypes.c_void_p), ("ks", ctypes.c_void_p), ("ke", ctypes.c_void_p),
        ("row_len", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
        ("m", ctypes.c_int32), ("n", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
        ("B", ctypes.c_int32), ("next_n", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("max_pages", ctypes.c_int32), ("num_pages", ctypes.c_int64), ("width", ctypes.c_int32),
        ("logits", ctypes.c_void_p), ("scores", ctypes.c_void_p), ("ld_logits", ctypes.c_int64),
        ("clean", ctypes.c_int32), ("rows", ctypes.c_int32), ("k", ctypes.c_int32), ("row0", ctypes.c_int32),
        ("map_to_slots", ctypes.c_int32), ("map", ctypes.c_void_p), ("out", ctypes.c_void_p),
        ("ld_out", ctypes.c_int64), ("logits_cap_bytes", ctypes.c_size_t), ("ws", ctypes.c_void_p),
        ("ws_bytes", ctypes.c_size_t), ("stream", ctypes.c_void_p), ("side_stream", ctypes.c_void_p),
    ]


_LIB = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfp8idx.so and declare its signatures (raises if it is missing)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built: run `python -m fp8_mqa_logits_amd.build` "
            "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(path)
    sig = {
        "indexer_logits_ragged": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _I64, _I32,
                                         _P, _SZ, _P]),
        "indexer_logits_paged": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I64,
                                        _P, _I64, _I32, _I32, _P]),
        "indexer_topk": (_I32, [_P, _I64, _I32, _I32, _P, _P, _I32, _I32, ctypes.POINTER(_CMap), _P, _I64,
                                _P, _SZ, _P]),
        "indexer_logits_topk_ragged": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                              ctypes.POINTER(_CMap), _P, _I64, _SZ, _P, _SZ, _P]),
        "indexer_logits_topk_paged": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I64,
                                             _I32, _I32, _I32, _P, _I64, _SZ, _P, _SZ, _P]),
        "fp8idx_workspace_bytes": (_SZ, [_I32, _I32, _I64, _I32, _SZ]),
        "fp8idx_workspace_bytes_paged": (_SZ, [_I32, _I32, _I32, _I32, _SZ]),
        "fp8idx_rows_per_chunk": (_I32, [_SZ, _I64, _I32]),
        "fp8idx_status_string": (ctypes.c_char_p, [_I32]),
        "fp8idx_last_hip_error": (_I32, []),
        "fp8idx_version": (ctypes.c_char_p, []),
        "indexer_quant_fp8": (_I32, [_P, _I64, _I64, _I32, _P, _I64, _P, _P]),
        "indexer_prepare_ragged": (_I32, [_P, _P, _P, _P, _I64, _I32, _I32, _P, _P, _P, _P, _I64, _P, _I64, _P]),
        "indexer_prepare_decode": (_I32, [_P, _P, _P, _I64, _I32, _I32, _I32, _P, _P, _I32, _P]),
        "indexer_logits_topk_ragged_overlap": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                                      ctypes.POINTER(_CMap), _P, _I64, _SZ, _P, _SZ, _P, _P]),
        "indexer_sparse_mla": (_I32, [_P, _P, _P, _I64, _P, _I64, _I32, _I32, _I32, _I32, _I32, ctypes.c_float,
                                      _P, _P, _P, _SZ, _P]),
        "fp8idx_sparse_mla_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
        "fp8idx_probe_mfma_fp8": (_I32, [_I32, _I32, _P, ctypes.POINTER(ctypes.c_double), _P]),
        "fp8idx_probe_logits_core": (_I32, [_I32, _I32, _P, ctypes.POINTER(ctypes.c_double), _P]),
        "fp8idx_validate_only": (_I32, [_I32, ctypes.POINTER(CallArgs)]),
        "indexer_logits_ragged_noalloc": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _I64, _I32,
                                                 _P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = L
    return L


def _check(fn: str, status: int) -> None:
    if status != 0:
        L = load_library()
        msg = L.fp8idx_status_string(status).decode()
        if status == 5:
            msg += f" (hipError {L.fp8idx_last_hip_error()})"
        raise Fp8idxError(fn, status, msg)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device, stream) -> int:
    if stream is None:
        return torch.cuda.current_stream(dev).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, name: str) -> torch.device:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t.device


def _same_device(dev: torch.device, **tensors) -> None:
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _need(t: torch.Tensor, name: str, dtypes, dev: Optional[torch.device] = None) -> torch.Tensor:
    """dtype and contiguity (and, with dev, the device) of one tensor."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _fp8(t: torch.Tensor, name: str, dev: Optional[torch.device] = None) -> torch.Tensor:
    _need(t, name, (torch.uint8, torch.float8_e4m3fn), dev)
    return t.view(torch.uint8) if t.dtype != torch.uint8 else t


def _shape(t: torch.Tensor, name: str, shape) -> None:
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _numel(t: torch.Tensor, name: str, n: int) -> None:
    if t.dim() != 1 or t.numel() != n:
        raise ValueError(f"{name} must be 1-D with {n} elements, got shape {tuple(t.shape)}")


_F32 = (torch.float32,)
_I32T = (torch.int32,)


@dataclasses.dataclass
class TopkMap:
    """Index map of the top-k stage (fp8idx_map): kind, table [num_req, ld] int32 and extras.

    Block table: ``num_pages`` is the pool's page count (page ids outside [0, num_pages) map to -1).
    """

    kind: int = MAP_NONE
    table: Optional[torch.Tensor] = None
    cu_rows: Optional[torch.Tensor] = None
    rows_per_req: int = 1
    page_size: int = 1
    num_pages: int = 0

    def check(self) -> None:
        """Shapes and dtypes of the map's tensors (raises ValueError)."""
        if self.kind not in (MAP_NONE, MAP_TOKEN_TABLE, MAP_BLOCK_TABLE):
            raise ValueError(f"unknown map kind {self.kind}")
        if self.kind == MAP_NONE:
            return
        if self.table is None:
            raise ValueError("a token or block table map needs a table")
        if self.table.dtype != torch.int32 or not self.table.is_contiguous() or self.table.dim() != 2:
            raise ValueError("map table must be a contiguous 2-D int32 tensor")
        if self.cu_rows is not None:
            if self.cu_rows.dtype != torch.int32 or not self.cu_rows.is_contiguous():
                raise ValueError("cu_rows must be a contiguous int32 tensor")
            _numel(self.cu_rows, "cu_rows", self.table.shape[0] + 1)
        if self.kind == MAP_BLOCK_TABLE:
            if self.rows_per_req < 1 or self.page_size < 1:
                raise ValueError("block table map needs rows_per_req >= 1 and page_size >= 1")
            if self.num_pages < 1:
                raise ValueError("block table map needs num_pages (pages in the pool) >= 1")

    def to_c(self) -> _CMap:
        self.check()
        m = _CMap()
        m.kind = self.kind
        if self.table is not None:
            m.table = self.table.data_ptr()
            m.ld = self.table.shape[1]
            m.num_req = self.table.shape[0]
        if self.cu_rows is not None:
            m.cu_rows = self.cu_rows.data_ptr()
        m.rows_per_req = self.rows_per_req
        m.page_size = self.page_size
        m.num_pages = self.num_pages
        return m


def _cmap(map_: Optional[TopkMap]):
    if map_ is None:
        return None
    return ctypes.byref(map_.to_c())


def _map_devices(map_: Optional[TopkMap], dev: torch.device) -> None:
    if map_ is not None:
        _same_device(dev, table=map_.table, cu_rows=map_.cu_rows)


# ---------------------------------------------------------------------------
# Pure host helpers
# ---------------------------------------------------------------------------

def fp8idx_workspace_bytes(op: int, rows: int, width: int, k: int, logits_cap_bytes: int = 0) -> int:
    return int(load_library().fp8idx_workspace_bytes(op, rows, width, k, logits_cap_bytes))


def fp8idx_workspace_bytes_paged(B: int, next_n: int, width: int, k: int, logits_cap_bytes: int = 0) -> int:
    return int(load_library().fp8idx_workspace_bytes_paged(B, next_n, width, k, logits_cap_bytes))


def fp8idx_rows_per_chunk(logits_cap_bytes: int, width: int, rows: int) -> int:
    return int(load_library().fp8idx_rows_per_chunk(logits_cap_bytes, width, rows))


def fp8idx_version() -> str:
    return load_library().fp8idx_version().decode()


def fp8idx_validate_only(entry: int, args: CallArgs) -> int:
    """Status the entry would return for these arguments before looking for a device (host only)."""
    return int(load_library().fp8idx_validate_only(int(entry), ctypes.byref(args)))


def _workspace(nbytes: int, dev: torch.device, ws: Optional[torch.Tensor]):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
    if ws.dtype != torch.uint8 or ws.device != dev or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 device tensor")
    off = (-ws.data_ptr()) % 256
    avail = ws.numel() - off
    if avail < nbytes:
        raise ValueError(f"workspace too small: {max(0, avail)} usable bytes after 256-byte alignment, "
                         f"{nbytes} needed")
    return ws.data_ptr() + off, avail


def _ragged_inputs(q, kv, kv_scale, weights, ks, ke):
    """Checks of the ragged logits inputs; returns (q8, kv8, m, n)."""
    q8 = _fp8(q, "q")
    kv8 = _fp8(kv, "kv")
    if q8.dim() != 3 or q8.shape[1:] != (H, D):
        raise ValueError(f"q must be [m, {H}, {D}], got {tuple(q8.shape)}")
    if kv8.dim() != 2 or kv8.shape[1] != D:
        raise ValueError(f"kv must be [n, {D}], got {tuple(kv8.shape)}")
    m, n = q8.shape[0], kv8.shape[0]
    _need(kv_scale, "kv_scale", _F32)
    _numel(kv_scale, "kv_scale", n)
    _need(weights, "weights", _F32)
    _shape(weights, "weights", (m, H))
    _need(ks, "ks", _I32T)
    _numel(ks, "ks", m)
    _need(ke, "ke", _I32T)
    _numel(ke, "ke", m)
    return q8, kv8, m, n


def _paged_inputs(q, kv_pool, scale_pool, weights, row_len, block_table, width: int):
    """Checks of the paged logits inputs; returns (q8, pool8, B, next_n)."""
    q8 = _fp8(q, "q")
    pool8 = _fp8(kv_pool, "kv_pool")
    if q8.dim() != 4 or q8.shape[2:] != (H, D):
        raise ValueError(f"q must be [B, next_n, {H}, {D}], got {tuple(q8.shape)}")
    if pool8.dim() != 3 or pool8.shape[2] != D:
        raise ValueError(f"kv_pool must be [pages, page_size, {D}], got {tuple(pool8.shape)}")
    B, nn = q8.shape[0], q8.shape[1]
    pages, page = pool8.shape[0], pool8.shape[1]
    _need(scale_pool, "scale_pool", _F32)
    if scale_pool.numel() != pages * page:
        raise ValueError(f"scale_pool must hold pages * page_size = {pages * page} floats, "
                         f"got {scale_pool.numel()}")
    _need(weights, "weights", _F32)
    _shape(weights, "weights", (B * nn, H))
    _need(row_len, "row_len", _I32T)
    _numel(row_len, "row_len", B * nn)
    _need(block_table, "block_table", _I32T)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [B = {B}, max_pages], got {tuple(block_table.shape)}")
    if int(width) < 0 or int(width) > block_table.shape[1] * page:
        raise ValueError(f"width must lie in [0, max_pages * page_size = {block_table.shape[1] * page}]")
    return q8, pool8, B, nn


def _out_rows(out: Optional[torch.Tensor], rows: int, k: int, dev) -> torch.Tensor:
    if out is None:
        return torch.empty((rows, k), dtype=torch.int32, device=dev)
    _need(out, "out", _I32T)
    if out.dim() != 2 or out.shape[0] != rows or out.shape[1] < k:
        raise ValueError(f"out must be [{rows}, >= {k}] int32, got {tuple(out.shape)}")
    return out


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def indexer_logits_ragged(q, kv, kv_scale, weights, ks, ke, *, clean: bool = True,
                          logits: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                          stream=None) -> torch.Tensor:
    """Ragged-prefill logits [m, n] float32 (or into ``logits`` [m, ld >= n]).

    ``workspace`` (uint8) holds the launch's work-queue counters: fp8idx_workspace_bytes(OP_LOGITS_RAGGED,
    ...) = 256 bytes from its first 256-byte aligned address on.  One is allocated when it is not
    given.  Calls that may run at the same time need distinct workspaces.
    """
    q8, kv8, m, n = _ragged_inputs(q, kv, kv_scale, weights, ks, ke)
    if logits is not None:
        _need(logits, "logits", _F32)
        if logits.dim() != 2 or logits.shape[0] != m or logits.shape[1] < n:
            raise ValueError(f"logits must be [{m}, >= {n}] float32, got {tuple(logits.shape)}")
    dev = _dev(q8, "q")
    _same_device(dev, kv=kv8, kv_scale=kv_scale, weights=weights, ks=ks, ke=ke, logits=logits,
                 workspace=workspace)
    if logits is None:
        logits = torch.empty((m, n), dtype=torch.float32, device=dev)
    L = load_library()
    need = int(L.fp8idx_workspace_bytes(OP_LOGITS_RAGGED, m, n, 1, 0))
    wp, wb = _workspace(need, dev, workspace)
    with torch.cuda.device(dev):
        st = L.indexer_logits_ragged(
            _ptr(q8), _ptr(kv8), _ptr(kv_scale), _ptr(weights), _ptr(ks), _ptr(ke), m, n, H, D,
            _ptr(logits), logits.shape[1], int(bool(clean)), wp, wb, _stream(dev, stream))
    _check("indexer_logits_ragged", st)
    return logits


def indexer_logits_ragged_noalloc(q, kv, kv_scale, weights, ks, ke, *, logits: torch.Tensor, clean: bool = True,
                                  stream=None) -> torch.Tensor:
    """indexer_logits_ragged into the caller's ``logits`` [m, ld >= n] with no allocation at all: the
    work-queue counters are the library's static per-device array, so calls that may overlap in time
    on one GPU race (use indexer_logits_ragged with distinct workspaces for those)."""
    q8, kv8, m, n = _ragged_inputs(q, kv, kv_scale, weights, ks, ke)
    _need(logits, "logits", _F32)
    if logits.dim() != 2 or logits.shape[0] != m or logits.shape[1] < n:
        raise ValueError(f"logits must be [{m}, >= {n}] float32, got {tuple(logits.shape)}")
    dev = _dev(q8, "q")
    _same_device(dev, kv=kv8, kv_scale=kv_scale, weights=weights, ks=ks, ke=ke, logits=logits)
    with torch.cuda.device(dev):
        st = load_library().indexer_logits_ragged_noalloc(
            _ptr(q8), _ptr(kv8), _ptr(kv_scale), _ptr(weights), _ptr(ks), _ptr(ke), m, n, H, D,
            _ptr(logits), logits.shape[1], int(bool(clean)), _stream(dev, stream))
    _check("indexer_logits_ragged_noalloc", st)
    return logits


def indexer_logits_paged(q, kv_pool, scale_pool, weights, row_len, block_table, *, width: int,
                         clean: bool = True, logits: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Paged-decode logits [B * next_n, width] float32."""
    q8, pool8, B, nn = _paged_inputs(q, kv_pool, scale_pool, weights, row_len, block_table, width)
    if logits is not None:
        _need(logits, "logits", _F32)
        if logits.dim() != 2 or logits.shape[0] != B * nn or logits.shape[1] < width:
            raise ValueError(f"logits must be [{B * nn}, >= {width}] float32, got {tuple(logits.shape)}")
    dev = _dev(q8, "q")
    _same_device(dev, kv_pool=pool8, scale_pool=scale_pool, weights=weights, row_len=row_len,
                 block_table=block_table, logits=logits)
    if logits is None:
        logits = torch.empty((B * nn, width), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        st = load_library().indexer_logits_paged(
            _ptr(q8), _ptr(pool8), _ptr(scale_pool), _ptr(weights), _ptr(row_len), _ptr(block_table),
            B, nn, H, D, pool8.shape[1], block_table.shape[1], pool8.shape[0],
            _ptr(logits), logits.shape[1], int(width), int(bool(clean)), _stream(dev, stream))
    _check("indexer_logits_paged", st)
    return logits


def indexer_topk(logits, ke, k: int, *, ks=None, width: Optional[int] = None, row0: int = 0,
                 map: Optional[TopkMap] = None, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Top-k [rows, k] int32 over logits [rows, ld] within [ks, ke)."""
    if not isinstance(logits, torch.Tensor) or logits.dtype != torch.float32 or logits.dim() != 2 \
            or logits.stride(1) != 1:
        raise ValueError("logits must be a 2-D float32 tensor with unit column stride")
    rows = logits.shape[0]
    ld = logits.stride(0) if rows > 1 else logits.shape[1]
    width = logits.shape[1] if width is None else int(width)
    if width < 0 or width > logits.shape[1]:
        raise ValueError(f"width must lie in [0, {logits.shape[1]}] (the logits columns)")
    _need(ke, "ke", _I32T)
    _numel(ke, "ke", rows)
    if ks is not None:
        _need(ks, "ks", _I32T)
        _numel(ks, "ks", rows)
    if map is not None:
        map.check()
    out = _out_rows(out, rows, k, logits.device)
    dev = _dev(logits, "logits")
    _same_device(dev, ke=ke, ks=ks, out=out, workspace=workspace)
    _map_devices(map, dev)
    L = load_library()
    need = int(L.fp8idx_workspace_bytes(OP_TOPK, rows, width, k, 0))
    wp, wb = _workspace(need, dev, workspace)
    with torch.cuda.device(dev):
        st = L.indexer_topk(_ptr(logits), ld, rows, width, _ptr(ks), _ptr(ke), k, row0, _cmap(map),
                            _ptr(out), out.shape[1], wp, wb, _stream(dev, stream))
    _check("indexer_topk", st)
    return out


def indexer_logits_topk_ragged(q, kv, kv_scale, weights, ks, ke, k: int, *,
                               map: Optional[TopkMap] = None, logits_cap_bytes: int = 0,
                               out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                               stream=None) -> torch.Tensor:
    """Fused ragged logits + top-k, row-chunked under ``logits_cap_bytes`` (0 = one chunk)."""
    q8, kv8, m, n = _ragged_inputs(q, kv, kv_scale, weights, ks, ke)
    if map is not None:
        map.check()
    out = _out_rows(out, m, k, q8.device)
    dev = _dev(q8, "q")
    _same_device(dev, kv=kv8, kv_scale=kv_scale, weights=weights, ks=ks, ke=ke, out=out, workspace=workspace)
    _map_devices(map, dev)
    L = load_library()
    need = int(L.fp8idx_workspace_bytes(OP_LOGITS_TOPK_RAGGED, m, n, k, logits_cap_bytes))
    wp, wb = _workspace(need, dev, workspace)
    with torch.cuda.device(dev):
        st = L.indexer_logits_topk_ragged(
            _ptr(q8), _ptr(kv8), _ptr(kv_scale), _ptr(weights), _ptr(ks), _ptr(ke), m, n, H, D, k,
            _cmap(map), _ptr(out), out.shape[1], logits_cap_bytes, wp, wb, _stream(dev, stream))
    _check("indexer_logits_topk_ragged", st)
    return out


def indexer_logits_topk_ragged_overlap(q, kv, kv_scale, weights, ks, ke, k: int, *, side_stream,
                                       map: Optional[TopkMap] = None, logits_cap_bytes: int = 0,
                                       out: Optional[torch.Tensor] = None,
                                       workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """indexer_logits_topk_ragged with chunk N - 1's top-k on ``side_stream`` while chunk N's logits run."""
    q8, kv8, m, n = _ragged_inputs(q, kv, kv_scale, weights, ks, ke)
    if map is not None:
        map.check()
    out = _out_rows(out, m, k, q8.device)
    dev = _dev(q8, "q")
    _same_device(dev, kv=kv8, kv_scale=kv_scale, weights=weights, ks=ks, ke=ke, out=out, workspace=workspace)
    _map_devices(map, dev)
    L = load_library()
    need = int(L.fp8idx_workspace_bytes(OP_LOGITS_TOPK_RAGGED_OVERLAP, m, n, k, logits_cap_bytes))
    wp, wb = _workspace(need, dev, workspace)
    with torch.cuda.device(dev):
        st = L.indexer_logits_topk_ragged_overlap(
            _ptr(q8), _ptr(kv8), _ptr(kv_scale), _ptr(weights), _ptr(ks), _ptr(ke), m, n, H, D, k,
            _cmap(map), _ptr(out), out.shape[1], logits_cap_bytes, wp, wb, _stream(dev, stream),
            _stream(dev, side_stream))
    _check("indexer_logits_topk_ragged_overlap", st)
    return out


def indexer_logits_topk_paged(q, kv_pool, scale_pool, weights, row_len, block_table, k: int, *,
                              width: int, map_to_slots: bool = True, logits_cap_bytes: int = 0,
                              out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                              stream=None) -> torch.Tensor:
    """Fused paged logits + top-k -> [B * next_n, k] int32 physical slots (or raw positions)."""
    q8, pool8, B, nn = _paged_inputs(q, kv_pool, scale_pool, weights, row_len, block_table, width)
    out = _out_rows(out, B * nn, k, q8.device)
    dev = _dev(q8, "q")
    _same_device(dev, kv_pool=pool8, scale_pool=scale_pool, weights=weights, row_len=row_len,
                 block_table=block_table, out=out, workspace=workspace)
    L = load_library()
    need = int(L.fp8idx_workspace_bytes_paged(B, nn, width, k, logits_cap_bytes))
    wp, wb = _workspace(need, dev, workspace)
    with torch.cuda.device(dev):
        st = L.indexer_logits_topk_paged(
            _ptr(q8), _ptr(pool8), _ptr(scale_pool), _ptr(weights), _ptr(row_len), _ptr(block_table),
            B, nn, H, D, pool8.shape[1], block_table.shape[1], pool8.shape[0], int(width), k,
            int(bool(map_to_slots)), _ptr(out), out.shape[1], logits_cap_bytes, wp, wb, _stream(dev, stream))
    _check("indexer_logits_topk_paged", st)
    return out


def _probe(name: str, blocks: int, iters: int, out: Optional[torch.Tensor], stream):
    dev = torch.device("cuda", torch.cuda.current_device())
    if out is None:
        out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    else:
        _need(out, "out", _F32, dev)
        if out.numel() < blocks * 256:
            raise ValueError("out must hold blocks * 256 floats")
    flops = ctypes.c_double(0.0)
    L = load_library()
    with torch.cuda.device(dev):
        st = getattr(L, name)(int(blocks), int(iters), _ptr(out), ctypes.byref(flops), _stream(dev, stream))
    _check(name, st)
    return out, flops.value


def fp8idx_probe_mfma_fp8(blocks: int, iters: int, *, out: Optional[torch.Tensor] = None, stream=None):
    """Launch the fp8 MFMA throughput probe (a measurement helper, not an indexer step).

    Returns (out, flops): out is the float32 [blocks * 256] sink the kernel writes, flops the
    launch's MFMA flops.  The caller times the launch (events on `stream`).
    """
    return _probe("fp8idx_probe_mfma_fp8", blocks, iters, out, stream)


def fp8idx_probe_logits_core(blocks: int, iters: int, *, out: Optional[torch.Tensor] = None, stream=None):
    """Launch the logits-core probe: the logits kernels' per-fragment MFMA + exact-epilogue code on
    register operands, no memory traffic (a measurement helper, not an indexer step).

    Returns (out, flops) like fp8idx_probe_mfma_fp8; the caller times the launch.
    """
    return _probe("fp8idx_probe_logits_core", blocks, iters, out, stream)


def indexer_quant_fp8(x, *, codes: Optional[torch.Tensor] = None, scale: Optional[torch.Tensor] = None,
                      stream=None):
    """Per-row e4m3fn quantisation of float32 x [rows, D] (or [..., D], flattened to rows).

    Returns (codes uint8 [rows, D], scale float32 [rows]) with x ~ decode(codes) * scale.
    """
    dev = _dev(x, "x")
    _need(x, "x", _F32, dev)
    D = x.shape[-1]
    rows = x.numel() // D if D else 0
    if codes is None:
        codes = torch.empty((rows, D), dtype=torch.uint8, device=dev)
    else:
        codes = _fp8(codes, "codes", dev)
    if scale is None:
        scale = torch.empty((rows,), dtype=torch.float32, device=dev)
    else:
        _need(scale, "scale", _F32, dev)
    if codes.numel() != rows * D or scale.numel() != rows:
        raise ValueError("codes must hold rows * D bytes and scale rows floats")
    L = load_library()
    with torch.cuda.device(dev):
        st = L.indexer_quant_fp8(_ptr(x), D, rows, D, _ptr(codes), D, _ptr(scale), _stream(dev, stream))
    _check("indexer_quant_fp8", st)
    return codes.view(rows, D), scale


def indexer_prepare_ragged(seq_len, q_len, req_idx, table, *, max_q: int, max_keys: int = 0,
                           ragged_mem: bool = True, stream=None):
    """Ragged prefill index preparation -> dict(cu_seq, cu_q, ks, ke, ragged_mem) of int32 device tensors.

    ks/ke hold max_q entries and ragged_mem max_keys entries; entries past the totals are left as allocated.
    """
    for t, n in ((seq_len, "seq_len"), (q_len, "q_len"), (req_idx, "req_idx"), (table, "table")):
        _need(t, n, _I32T)
    B = seq_len.numel()
    _numel(seq_len, "seq_len", B)
    _numel(q_len, "q_len", B)
    _numel(req_idx, "req_idx", B)
    if table.dim() != 2:
        raise ValueError("table must be [rows, ld] int32")
    dev = _dev(seq_len, "seq_len")
    _same_device(dev, q_len=q_len, req_idx=req_idx, table=table)
    out = {"cu_seq": torch.empty(B + 1, dtype=torch.int32, device=dev),
           "cu_q": torch.empty(B + 1, dtype=torch.int32, device=dev),
           "ks": torch.empty(max(max_q, 0), dtype=torch.int32, device=dev),
           "ke": torch.empty(max(max_q, 0), dtype=torch.int32, device=dev),
           "ragged_mem": torch.empty(max(max_keys, 0), dtype=torch.int32, device=dev) if ragged_mem else None}
    L = load_library()
    with torch.cuda.device(dev):
        st = L.indexer_prepare_ragged(_ptr(seq_len), _ptr(q_len), _ptr(req_idx), _ptr(table), table.shape[1],
                                      table.shape[0], B, _ptr(out["cu_seq"]), _ptr(out["cu_q"]), _ptr(out["ks"]),
                                      _ptr(out["ke"]), max_q, _ptr(out["ragged_mem"]), max_keys,
                                      _stream(dev, stream))
    _check("indexer_prepare_ragged", st)
    return out


def indexer_prepare_decode(seq_len, req_idx, req_to_page, next_n: int, *, max_pages: Optional[int] = None,
                           stream=None):
    """Paged decode / MTP index preparation -> (row_len [B * next_n], block_table [B, max_pages]) int32."""
    for t, n in ((seq_len, "seq_len"), (req_idx, "req_idx"), (req_to_page, "req_to_page")):
        _need(t, n, _I32T)
    B = seq_len.numel()
    _numel(seq_len, "seq_len", B)
    _numel(req_idx, "req_idx", B)
    if req_to_page.dim() != 2:
        raise ValueError("req_to_page must be [rows, ld] int32")
    mp = req_to_page.shape[1] if max_pages is None else int(max_pages)
    if mp < 0 or mp > req_to_page.shape[1]:
        raise ValueError(f"max_pages must lie in [0, {req_to_page.shape[1]}] (the req_to_page columns)")
    dev = _dev(seq_len, "seq_len")
    _same_device(dev, req_idx=req_idx, req_to_page=req_to_page)
    row_len = torch.empty(B * next_n, dtype=torch.int32, device=dev)
    bt = torch.empty((B, mp), dtype=torch.int32, device=dev)
    L = load_library()
    with torch.cuda.device(dev):
        st = L.indexer_prepare_decode(_ptr(seq_len), _ptr(req_idx), _ptr(req_to_page), req_to_page.shape[1],
                                      req_to_page.shape[0], B, next_n, _ptr(row_len), _ptr(bt), mp,
                                      _stream(dev, stream))
    _check("indexer_prepare_decode", st)
    return row_len, bt


def fp8idx_sparse_mla_workspace_bytes(T: int, H: int, topk: int) -> int:
    return int(load_library().fp8idx_sparse_mla_workspace_bytes(int(T), int(H), int(topk)))


def indexer_sparse_mla(q, kv, kv_scale, indices, sm_scale: float, *, out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                       workspace: Optional[torch.Tensor] = None, stream=None):
    """Sparse MLA attention over top-k slots -> (out float32 [T, H, 512], lse float32 [T, H] or None).

    q: bf16 [T, H, 576] (or int16 / uint16 bit patterns); kv: e4m3fn [S, 576] (or uint8 codes);
    kv_scale: float32 [S]; indices: int32 [T, topk] slot ids (-1 or >= S skipped).
    """
    dev = _dev(q, "q")
    q16 = _need(q, "q", (torch.bfloat16, torch.int16, torch.uint16), dev)
    kv8 = _fp8(kv, "kv", dev)
    _need(kv_scale, "kv_scale", _F32, dev)
    _need(indices, "indices", _I32T, dev)
    if q16.dim() != 3 or q16.shape[2] != MLA_DQK:
        raise ValueError("q must be [T, H, 576]")
    if kv8.dim() != 2 or kv8.shape[1] != MLA_DQK or kv_scale.numel() != kv8.shape[0]:
        raise ValueError("kv must be [S, 576] with kv_scale [S]")
    T, Hh = q16.shape[0], q16.shape[1]
    if indices.dim() != 2 or indices.shape[0] != T:
        raise ValueError("indices must be [T, topk]")
    topk = indices.shape[1]
    if out is None:
        out = torch.empty((T, Hh, MLA_DV), dtype=torch.float32, device=dev)
    else:
        _need(out, "out", _F32, dev)
    if lse is None and want_lse:
        lse = torch.empty((T, Hh), dtype=torch.float32, device=dev)
    elif lse is not None:
        _need(lse, "lse", _F32, dev)
    L = load_library()
    need = int(L.fp8idx_sparse_mla_workspace_bytes(T, Hh, topk)) if T > 0 else 0
    ws = None
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need + 256, dtype=torch.uint8, device=dev)
        if workspace.numel() < need:
            raise ValueError(f"workspace too small: {workspace.numel()} < {need}")
        base = workspace.data_ptr()
        ws = (base + 255) // 256 * 256
        if ws + need > base + workspace.numel():
            raise ValueError("workspace too small after 256-byte alignment")
    with torch.cuda.device(dev):
        st = L.indexer_sparse_mla(_ptr(q16), _ptr(kv8), _ptr(kv_scale), kv8.shape[0], _ptr(indices), topk, T, Hh,
                                  MLA_DQK, MLA_DV, topk, float(sm_scale), _ptr(out), _ptr(lse), ws, need,
                                  _stream(dev, stream))
    _check("indexer_sparse_mla", st)
    return out, lse
