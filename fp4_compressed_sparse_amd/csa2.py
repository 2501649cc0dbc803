"""Thin Python binding of libcsa2.so (the C ABI declared in include/csa2.h).

Argument marshalling only: torch tensors provide device memory and the current HIP stream;
every step of the computation runs in the library's gfx950 kernels.  Importing this module
raises if the library has not been built -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

D_LAT, D_ROPE, D_Q, D_IDX, D_SWA, PAGE = 512, 64, 576, 64, 128, 64
FULL, REINDEX, REUSE, REINDEX_POOL = 0, 1, 2, 3
KV_MXFP4, KV_FP4_E4M3 = 0, 1
OP_INDEX_TOPK, OP_SPARSE_ATTN, OP_LAYER_GROUP, OP_INDEX_TOPK_POOL = 1, 2, 3, 4
STATUS = {0: "CSA2_OK", 1: "CSA2_ERR_NULL", 2: "CSA2_ERR_SHAPE", 3: "CSA2_ERR_ALIGN",
          4: "CSA2_ERR_MODE", 5: "CSA2_ERR_WORKSPACE", 6: "CSA2_ERR_UNSUPPORTED",
          7: "CSA2_ERR_HIP"}

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_f32 = ctypes.c_float


class IndexArgs(ctypes.Structure):
    _fields_ = [("T", _i32), ("B", _i32), ("H_I", _i32), ("K", _i32), ("max_pages", _i32),
                ("n_pages", _i32), ("q_idx", _vp), ("w_idx", _vp), ("k_idx", _vp),
                ("page_table", _vp), ("seq_id", _vp), ("n_vis", _vp), ("idx_out", _vp)]


class PoolArgs(ctypes.Structure):
    _fields_ = [("ix", IndexArgs), ("sel", _vp), ("K_sel", _i32)]


class AppendArgs(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("c", _vp), ("z", _vp), ("c_idx", _vp), ("z_idx", _vp),
                ("dst_row", _vp), ("kv_lat", _vp), ("kv_scl", _vp), ("kv_rope", _vp),
                ("k_idx", _vp), ("kv_row_bytes", _i32)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("T", _i32), ("B", _i32), ("H", _i32), ("K", _i32), ("max_pages", _i32),
                ("n_pages", _i32), ("q", _vp), ("kv_lat", _vp), ("kv_scl", _vp),
                ("kv_rope", _vp), ("page_table", _vp), ("seq_id", _vp), ("idx", _vp),
                ("sm_scale", _f32), ("o", _vp), ("lse", _vp), ("H_kv", _i32), ("L_swa", _i32),
                ("q_swa", _vp), ("swa_k", _vp), ("swa_v", _vp), ("swa_start", _vp),
                ("swa_len", _vp), ("sm_scale_swa", _f32), ("o_swa", _vp), ("lse_swa", _vp),
                ("kv_format", _i32), ("kv_row_bytes", _i32)]


class LayerDesc(ctypes.Structure):
    _fields_ = [("mode", _i32), ("q", _vp), ("q_swa", _vp), ("q_idx", _vp), ("w_idx", _vp),
                ("k_idx", _vp), ("kv_lat", _vp), ("kv_scl", _vp), ("kv_rope", _vp),
                ("swa_k", _vp), ("swa_v", _vp), ("idx_out", _vp), ("o", _vp), ("lse", _vp),
                ("o_swa", _vp), ("lse_swa", _vp)]


class GroupArgs(ctypes.Structure):
    _fields_ = [("T", _i32), ("B", _i32), ("H", _i32), ("H_I", _i32), ("K", _i32),
                ("H_kv", _i32), ("L_swa", _i32), ("max_pages", _i32), ("n_pages", _i32),
                ("page_table", _vp), ("seq_id", _vp), ("n_vis", _vp), ("swa_start", _vp),
                ("swa_len", _vp), ("sm_scale", _f32), ("sm_scale_swa", _f32),
                ("kv_format", _i32), ("kv_row_bytes", _i32)]


EXPORTS = ["csa2_index_topk", "csa2_index_topk_pool", "csa2_sparse_attn_fp4", "csa2_layer_group", "csa2_layer_group_noalloc", "csa2_mxfp4_quantize", "csa2_kv_append", "csa2_fp4e4m3_quantize",
           "csa2_workspace_bytes", "csa2_last_error", "csa2_status_string", "csa2_abi_version",
           "csa2_plan_cus", "csa2_timing_enable", "csa2_timing_read"]


def _load():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    L.csa2_index_topk.restype = _i32
    L.csa2_index_topk.argtypes = [ctypes.POINTER(IndexArgs), _vp, ctypes.c_size_t, _vp]
    L.csa2_index_topk_pool.restype = _i32
    L.csa2_index_topk_pool.argtypes = [ctypes.POINTER(PoolArgs), _vp, ctypes.c_size_t, _vp]
    L.csa2_sparse_attn_fp4.restype = _i32
    L.csa2_sparse_attn_fp4.argtypes = [ctypes.POINTER(AttnArgs), _vp, ctypes.c_size_t, _vp]
    L.csa2_layer_group.restype = _i32
    L.csa2_layer_group.argtypes = [ctypes.POINTER(LayerDesc), _i32, ctypes.POINTER(GroupArgs),
                                   _vp, ctypes.c_size_t, _vp]
    L.csa2_layer_group_noalloc.restype = _i32
    L.csa2_layer_group_noalloc.argtypes = [ctypes.POINTER(LayerDesc), _i32,
                                           ctypes.POINTER(GroupArgs), _vp]
    L.csa2_fp4e4m3_quantize.restype = _i32
    L.csa2_fp4e4m3_quantize.argtypes = [_vp, ctypes.c_int64, _vp, _vp, _vp, _i32, _vp]
    L.csa2_kv_append.restype = _i32
    L.csa2_kv_append.argtypes = [ctypes.POINTER(AppendArgs), _vp]
    L.csa2_mxfp4_quantize.restype = _i32
    L.csa2_mxfp4_quantize.argtypes = [_vp, ctypes.c_int64, _vp, _vp, _vp, _i32, _vp]
    L.csa2_workspace_bytes.restype = ctypes.c_size_t
    L.csa2_workspace_bytes.argtypes = [_i32, _vp]
    L.csa2_last_error.restype = ctypes.c_char_p
    L.csa2_last_error.argtypes = []
    L.csa2_status_string.restype = ctypes.c_char_p
    L.csa2_status_string.argtypes = [_i32]
    L.csa2_abi_version.restype = _i32
    L.csa2_plan_cus.restype = _i32
    L.csa2_plan_cus.argtypes = []
    L.csa2_timing_enable.restype = _i32
    L.csa2_timing_enable.argtypes = [_i32]
    L.csa2_timing_read.restype = _i32
    L.csa2_timing_read.argtypes = [_vp, _vp, _vp, _i32]
    return L


lib = _load()


class Csa2Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def _check(st: int):
    if st != 0:
        raise Csa2Error(st, lib.csa2_last_error().decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ws(nbytes: int, device):
    if nbytes == 0:
        return None
    # 256-byte alignment: the caching allocator hands out 512-byte aligned blocks
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _bits(t):
    """bf16 tensors are passed as raw 16-bit patterns."""
    return t


# ------------------------------------------------------------------ entry points
def index_args(q_idx, w_idx, k_idx, page_table, seq_id, n_vis, K, idx_out, n_pages=None):
    T, H_I = q_idx.shape[0], q_idx.shape[1]
    return IndexArgs(T, page_table.shape[0], H_I, K, page_table.shape[1],
                     n_pages if n_pages is not None else k_idx.shape[0] // PAGE if k_idx.dim() == 2
                     else k_idx.shape[0],
                     _p(q_idx), _p(w_idx), _p(k_idx), _p(page_table), _p(seq_id), _p(n_vis),
                     _p(idx_out))


def index_topk(q_idx, w_idx, k_idx, page_table, seq_id, n_vis, K, idx_out=None, stream=None,
               workspace=None):
    """Indexer scoring + Top-K.  q_idx bf16 [T, H_I, 64]; w_idx f32 [T, H_I];
    k_idx bf16 [n_pages, 64, 64]; page_table/seq_id/n_vis int32.  Returns idx int32 [T, K]."""
    T = q_idx.shape[0]
    if idx_out is None:
        idx_out = torch.empty((T, K), dtype=torch.int32, device=q_idx.device)
    a = index_args(q_idx, w_idx, k_idx, page_table, seq_id, n_vis, K, idx_out)
    need = lib.csa2_workspace_bytes(OP_INDEX_TOPK, ctypes.byref(a))
    ws = workspace if workspace is not None else _ws(need, q_idx.device)
    _check(lib.csa2_index_topk(ctypes.byref(a), _p(ws), need if workspace is None else
                               ws.numel() * ws.element_size(), _stream(stream)))
    return idx_out


def index_topk_pool(q_idx, w_idx, k_idx, page_table, seq_id, n_vis, K, sel, idx_out=None,
                    stream=None, workspace=None):
    """Hierarchical-indexer search: scoring + Top-K over the candidate pool of sel int32
    [T, K_sel] (ascending entries, -1 tail; e.g. a Full layer's selection).  Other
    arguments as index_topk.  Returns idx int32 [T, K]."""
    T = q_idx.shape[0]
    if idx_out is None:
        idx_out = torch.empty((T, K), dtype=torch.int32, device=q_idx.device)
    a = PoolArgs(index_args(q_idx, w_idx, k_idx, page_table, seq_id, n_vis, K, idx_out),
                 _p(sel), sel.shape[1])
    need = lib.csa2_workspace_bytes(OP_INDEX_TOPK_POOL, ctypes.byref(a))
    ws = workspace if workspace is not None else _ws(need, q_idx.device)
    _check(lib.csa2_index_topk_pool(ctypes.byref(a), _p(ws), need if workspace is None else
                                    ws.numel() * ws.element_size(), _stream(stream)))
    return idx_out


def attn_args(q, kv_lat, kv_scl, kv_rope, page_table, seq_id, idx, o, lse, sm_scale=None,
              q_swa=None, swa_k=None, swa_v=None, swa_start=None, swa_len=None,
              sm_scale_swa=None, o_swa=None, lse_swa=None, kv_format=KV_MXFP4, kv_row_bytes=0):
    T, H = q.shape[0], q.shape[1]
    K = idx.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D_Q)
    if sm_scale_swa is None:
        sm_scale_swa = 1.0 / math.sqrt(D_SWA)
    H_kv = swa_k.shape[2] if swa_k is not None else 1
    L_swa = swa_k.shape[1] if swa_k is not None else 1
    return AttnArgs(T, page_table.shape[0], H, K, page_table.shape[1], kv_lat.shape[0],
                    _p(q), _p(kv_lat), _p(kv_scl), _p(kv_rope), _p(page_table), _p(seq_id),
                    _p(idx), sm_scale, _p(o), _p(lse), H_kv, L_swa, _p(q_swa), _p(swa_k),
                    _p(swa_v), _p(swa_start), _p(swa_len), sm_scale_swa, _p(o_swa), _p(lse_swa),
                    kv_format, kv_row_bytes)


def sparse_attn_fp4(q, kv_lat, kv_scl, kv_rope, page_table, seq_id, idx, sm_scale=None,
                    q_swa=None, swa_k=None, swa_v=None, swa_start=None, swa_len=None,
                    sm_scale_swa=None, stream=None, out=None, kv_format=KV_MXFP4,
                    kv_row_bytes=0):
    """Sparse FP4 global attention (+ SWA when q_swa is given).
    kv_lat u8 [n_pages, 64, 256]; kv_scl u8 [n_pages, 64, 16]; kv_rope bf16 [n_pages, 64, 64]:
    dense planes (kv_row_bytes 0) or views of one packed buffer (see kv_packed).
    Returns (o, lse) or (o, lse, o_swa, lse_swa)."""
    T, H = q.shape[0], q.shape[1]
    dev = q.device
    if out is None:
        out = {"o": torch.empty((T, H, D_LAT), dtype=torch.float32, device=dev),
               "lse": torch.empty((T, H), dtype=torch.float32, device=dev)}
        if q_swa is not None:
            out["o_swa"] = torch.empty((T, H, D_SWA), dtype=torch.float32, device=dev)
            out["lse_swa"] = torch.empty((T, H), dtype=torch.float32, device=dev)
    a = attn_args(q, kv_lat, kv_scl, kv_rope, page_table, seq_id, idx, out["o"], out["lse"],
                  sm_scale, q_swa, swa_k, swa_v, swa_start, swa_len, sm_scale_swa,
                  out.get("o_swa"), out.get("lse_swa"), kv_format, kv_row_bytes)
    need = lib.csa2_workspace_bytes(OP_SPARSE_ATTN, ctypes.byref(a))
    ws = _ws(need, dev)
    _check(lib.csa2_sparse_attn_fp4(ctypes.byref(a), _p(ws), need, _stream(stream)))
    if q_swa is None:
        return out["o"], out["lse"]
    return out["o"], out["lse"], out["o_swa"], out["lse_swa"]


def group_args(T, B, H, H_I, K, H_kv, L_swa, max_pages, n_pages, page_table, seq_id, n_vis,
               swa_start, swa_len, sm_scale=None, sm_scale_swa=None, kv_format=KV_MXFP4,
               kv_row_bytes=0):
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D_Q)
    if sm_scale_swa is None:
        sm_scale_swa = 1.0 / math.sqrt(D_SWA)
    return GroupArgs(T, B, H, H_I, K, H_kv, L_swa, max_pages, n_pages, _p(page_table),
                     _p(seq_id), _p(n_vis), _p(swa_start), _p(swa_len), sm_scale, sm_scale_swa,
                     kv_format, kv_row_bytes)


def layer_desc(mode, q, o, lse, q_swa=None, q_idx=None, w_idx=None, k_idx=None, kv_lat=None,
               kv_scl=None, kv_rope=None, swa_k=None, swa_v=None, idx_out=None, o_swa=None,
               lse_swa=None):
    return LayerDesc(mode, _p(q), _p(q_swa), _p(q_idx), _p(w_idx), _p(k_idx), _p(kv_lat),
                     _p(kv_scl), _p(kv_rope), _p(swa_k), _p(swa_v), _p(idx_out), _p(o), _p(lse),
                     _p(o_swa), _p(lse_swa))


def layer_group(descs, g: GroupArgs, stream=None, workspace=None, device=None):
    """Run a Full/Reindex/Reuse group.  descs: list of LayerDesc (see layer_desc)."""
    n = len(descs)
    arr = (LayerDesc * n)(*descs)
    need = lib.csa2_workspace_bytes(OP_LAYER_GROUP, ctypes.byref(g))
    ws = workspace if workspace is not None else _ws(need, device or torch.device("cuda"))
    _check(lib.csa2_layer_group(arr, n, ctypes.byref(g), _p(ws),
                                need if workspace is None else ws.numel() * ws.element_size(), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 48 << 20


def layer_group_noalloc(descs, g: GroupArgs, stream=None):
    """The layer group with the library's static device scratch as its workspace (no
    allocation by the library or here)."""
    n = len(descs)
    arr = (LayerDesc * n)(*descs)
    _check(lib.csa2_layer_group_noalloc(arr, n, ctypes.byref(g), _stream(stream)))


def mxfp4_quantize(x, lat, scl, dst_row=None, stream=None, row_bytes=0):
    """x f32 [rows, 512] -> lat u8 [*, 256], scl u8 [*, 16] at rows dst_row (int64) or
    0..rows-1; row_bytes: the planes' row layout (0 = dense)."""
    rows = x.shape[0]
    _check(lib.csa2_mxfp4_quantize(_p(x), rows, _p(lat), _p(scl), _p(dst_row), row_bytes,
                                   _stream(stream)))


def fp4e4m3_quantize(x, lat, scl, dst_row=None, stream=None, row_bytes=0):
    """x f32 [rows, 512] -> lat u8 [*, 256], scl u8 [*, 32] (E4M3 per 16 channels) at rows
    dst_row (int64) or 0..rows-1; row_bytes: the planes' row layout (0 = dense)."""
    rows = x.shape[0]
    _check(lib.csa2_fp4e4m3_quantize(_p(x), rows, _p(lat), _p(scl), _p(dst_row), row_bytes,
                                     _stream(stream)))


def kv_append(c, z, kv_lat, kv_scl, kv_rope, dst_row=None, c_idx=None, z_idx=None,
              k_idx=None, stream=None, kv_row_bytes=0):
    """KV append: entries pooled from blocks of 4 raw tokens.  c, z f32 [n, 4, 576];
    c_idx, z_idx f32 [n, 4, 64] (optional, with k_idx); writes rows dst_row (int64) or
    0..n-1 of kv_lat u8 [*, 256], kv_scl u8 [*, 16], kv_rope bf16 [*, 64], k_idx bf16 [*, 64]."""
    a = AppendArgs(c.shape[0], _p(c), _p(z), _p(c_idx), _p(z_idx), _p(dst_row), _p(kv_lat),
                   _p(kv_scl), _p(kv_rope), _p(k_idx), kv_row_bytes)
    _check(lib.csa2_kv_append(ctypes.byref(a), _stream(stream)))


def kv_packed(n_pages, kv_format=KV_MXFP4, device=None, row_bytes=None):
    """One buffer of packed main-KV rows (codes | rope | scales, 400 bytes per entry, 416 with
    E4M3 scales, unless row_bytes says more) and its three plane views, for the
    kv_row_bytes layout.  Returns (buf, kv_lat, kv_scl, kv_rope, row_bytes)."""
    scl_b = 32 if kv_format == KV_FP4_E4M3 else 16
    rb = row_bytes or (256 + 128 + scl_b)
    buf = torch.zeros((n_pages, 64, rb), dtype=torch.uint8, device=device)
    lat = buf[..., 0:256]
    rope = buf[..., 256:384].view(torch.bfloat16)
    scl = buf[..., 384:384 + scl_b]
    return buf, lat, scl, rope, rb


def workspace_bytes(op: int, args) -> int:
    return lib.csa2_workspace_bytes(op, ctypes.byref(args))


def timing_enable(on: bool = True):
    _check(lib.csa2_timing_enable(1 if on else 0))


def timing_read(max_kernels: int = 32):
    """{kernel name: (launches, total_ms)} since the last read; synchronizes the events."""
    names = ctypes.create_string_buffer(64 * max_kernels)
    launches = (ctypes.c_int64 * max_kernels)()
    ms = (ctypes.c_double * max_kernels)()
    n = lib.csa2_timing_read(names, launches, ms, max_kernels)
    out = {}
    for i in range(n):
        nm = names.raw[64 * i: 64 * (i + 1)].split(b"\0", 1)[0].decode()
        out[nm] = (int(launches[i]), float(ms[i]))
    return out


def abi_version() -> int:
    return lib.csa2_abi_version()


def plan_cus() -> int:
    """Compute units the library's launch plans assume for the current device."""
    return lib.csa2_plan_cus()
