"""CSA2 oracle: Python marshalling around the plain-C, double-precision reference (oracle.c).

TEST INFRASTRUCTURE ONLY.  The GPU library never imports, links or calls this; only the
tests, the smoke check and the benchmark's CPU-baseline leg do.  It shares no code with the
GPU path.

Sources are cited by page and section: [summary] is the picx.dev whiteboard summary of
"DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression", [blog] the cyber-feed.org
repost of the blog article of that title.

Parity unpinned: the decomposition of the pages' 890 bytes/token into per-layer pieces;
the block-pooling formula of the KV append path (kv_pool: a reading, pinned only on its
own mathematics); the whole path against the pages (they print no worked example).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

FULL, REINDEX, REUSE, REINDEX_POOL = 0, 1, 2, 3
LAT, ROPE, DQ, DIDX, DSWA, PAGE = 512, 64, 576, 64, 128, 64


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11",
                               "-fno-fast-math", os.path.join(_HERE, "oracle.c"), "-o", tmp,
                               "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.csa2o_e2m1_decode.restype = f64
        L.csa2o_e2m1_decode.argtypes = [i32]
        L.csa2o_e8m0_decode.restype = f64
        L.csa2o_e8m0_decode.argtypes = [i32]
        L.csa2o_mxfp4_quantize.restype = i32
        L.csa2o_mxfp4_quantize.argtypes = [vp, i64, vp, vp]
        L.csa2o_mxfp4_dequantize.argtypes = [vp, vp, i64, vp]
        L.csa2o_topk_from_scores.argtypes = [vp, i64, i32, vp]
        L.csa2o_index_topk.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, i32,
                                       vp, vp]
        L.csa2o_kv_pool.argtypes = [vp, vp, i64, i32, i32, vp]
        L.csa2o_e4m3_decode.restype = f64
        L.csa2o_e4m3_decode.argtypes = [i32]
        L.csa2o_e4m3_round.restype = i32
        L.csa2o_e4m3_round.argtypes = [f64]
        L.csa2o_fp4e4m3_quantize.restype = i32
        L.csa2o_fp4e4m3_quantize.argtypes = [vp, i64, vp, vp]
        L.csa2o_fp4e4m3_dequantize.argtypes = [vp, vp, i64, vp]
        L.csa2o_sparse_attn_fmt.argtypes = [i32, i32, i32, vp, vp, vp, i32, vp, vp, vp, vp,
                                            f64, vp, i32, vp, vp]
        L.csa2o_round_bf16_array.argtypes = [vp, i64, vp]
        L.csa2o_pool_positions.restype = i64
        L.csa2o_pool_positions.argtypes = [vp, i32, i64, vp]
        L.csa2o_index_topk_pool.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                            i32, vp, i32, vp, vp]
        L.csa2o_sparse_attn.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, f64, vp,
                                        i32, vp, vp]
        L.csa2o_swa_attn.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp, f64, vp, i32, vp,
                                     vp]
        L.csa2o_num_threads.restype = i32
        L.csa2o_footprint_bytes_per_token.restype = f64
        L.csa2o_footprint_bytes_per_token.argtypes = [vp, i32, i32, i32, i32, i32, i32]
        _lib = L
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def e2m1_decode(code: int) -> float:
    return lib().csa2o_e2m1_decode(int(code))


def e8m0_decode(byte: int) -> float:
    return lib().csa2o_e8m0_decode(int(byte))


def mxfp4_quantize(x: np.ndarray):
    """fp32 [rows, 512] -> (lat uint8 [rows, 256], scl uint8 [rows, 16])."""
    x = _c(x, np.float32).reshape(-1, LAT)
    rows = x.shape[0]
    lat = np.zeros((rows, LAT // 2), dtype=np.uint8)
    scl = np.zeros((rows, LAT // 32), dtype=np.uint8)
    if lib().csa2o_mxfp4_quantize(_p(x), rows, _p(lat), _p(scl)) != 0:
        raise ValueError("MXFP4 quantization of a non-finite value")
    return lat, scl


def mxfp4_dequantize(lat: np.ndarray, scl: np.ndarray) -> np.ndarray:
    lat = _c(lat, np.uint8).reshape(-1, LAT // 2)
    scl = _c(scl, np.uint8).reshape(-1, LAT // 32)
    out = np.empty((lat.shape[0], LAT), dtype=np.float64)
    lib().csa2o_mxfp4_dequantize(_p(lat), _p(scl), lat.shape[0], _p(out))
    return out


def e4m3_decode(byte: int) -> float:
    return lib().csa2o_e4m3_decode(int(byte))


def e4m3_round(v: float) -> int:
    return lib().csa2o_e4m3_round(float(v))


def fp4e4m3_quantize(x: np.ndarray):
    """fp32 [rows, 512] -> (lat uint8 [rows, 256], scl uint8 [rows, 32]): E2M1 codes with
    one E4M3 scale per 16 channels.  [summary] Architecture Components, item 5 (its literal
    format)."""
    x = _c(x, np.float32).reshape(-1, LAT)
    rows = x.shape[0]
    lat = np.zeros((rows, LAT // 2), dtype=np.uint8)
    scl = np.zeros((rows, LAT // 16), dtype=np.uint8)
    if lib().csa2o_fp4e4m3_quantize(_p(x), rows, _p(lat), _p(scl)) != 0:
        raise ValueError("FP4/E4M3 quantization of a non-finite value")
    return lat, scl


def fp4e4m3_dequantize(lat: np.ndarray, scl: np.ndarray) -> np.ndarray:
    lat = _c(lat, np.uint8).reshape(-1, LAT // 2)
    scl = _c(scl, np.uint8).reshape(-1, LAT // 16)
    out = np.empty((lat.shape[0], LAT), dtype=np.float64)
    lib().csa2o_fp4e4m3_dequantize(_p(lat), _p(scl), lat.shape[0], _p(out))
    return out


def kv_pool(c, z) -> np.ndarray:
    """Block pooling of the KV append path: c, z fp32 [n, R, D] -> [n, D] float64, the
    softmax(z)-over-the-block weighted sum of c per channel.  [summary] Architecture
    Components, item 1 (Eq. 1: C and Z projections); the formula itself is a reading
    (parity unpinned against the pages)."""
    c, z = _c(c, np.float32), _c(z, np.float32)
    n, R, D = c.shape
    out = np.empty((n, D), dtype=np.float64)
    lib().csa2o_kv_pool(_p(c), _p(z), n, R, D, _p(out))
    return out


def round_bf16(x) -> np.ndarray:
    """float64 -> bf16 bit patterns (round to nearest, ties to even)."""
    x = _c(x, np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().csa2o_round_bf16_array(_p(x), x.size, _p(out))
    return out


def kv_append(c, z, c_idx=None, z_idx=None):
    """KV append of n entries, each pooled from 4 raw tokens: c, z fp32 [n, 4, 576]
    (latent 512 ; rope 64), c_idx, z_idx fp32 [n, 4, 64] or None.  Returns the pooled values
    (float64) and the cache contents: MXFP4 latent (of the pooled value rounded to fp32, the
    precision the cache write decides in), bf16 rope and bf16 indexer key."""
    y = kv_pool(c, z)
    lat, scl = mxfp4_quantize(y[:, :LAT].astype(np.float32))
    out = {"pooled": y, "lat": lat, "scl": scl, "rope": round_bf16(y[:, LAT:])}
    if c_idx is not None:
        yi = kv_pool(c_idx, z_idx)
        out["pooled_idx"] = yi
        out["k_idx"] = round_bf16(yi)
    return out


def topk_from_scores(s: np.ndarray, K: int) -> np.ndarray:
    s = _c(s, np.float64)
    out = np.empty(K, dtype=np.int32)
    lib().csa2o_topk_from_scores(_p(s), s.shape[0], K, _p(out))
    return out


def index_topk(K, max_pages, q_idx, w_idx, k_idx, page_table, seq_id, n_vis, rows=None,
               want_scores=False):
    """Indexer scoring + Top-K.  q_idx bf16 bits [T, H_I, 64]; w_idx f32 [T, H_I];
    k_idx bf16 bits [n_pages*64, 64] (physical rows); page_table i32 [B, max_pages].
    Returns idx [n_rows, K] (and scores [n_rows, max_pages*64] if want_scores)."""
    q_idx = _c(q_idx, np.uint16)
    T, H_I = q_idx.shape[0], q_idx.shape[1]
    w_idx, k_idx = _c(w_idx, np.float32), _c(k_idx, np.uint16)
    pt, sid, nv = _c(page_table, np.int32), _c(seq_id, np.int32), _c(n_vis, np.int32)
    rows = _c(np.arange(T) if rows is None else rows, np.int32)
    out = np.empty((rows.shape[0], K), dtype=np.int32)
    scores = (np.full((rows.shape[0], max_pages * PAGE), np.nan) if want_scores else None)
    lib().csa2o_index_topk(T, H_I, K, max_pages, _p(q_idx), _p(w_idx), _p(k_idx), _p(pt),
                           _p(sid), _p(nv), _p(rows), rows.shape[0], _p(out),
                           _p(scores) if want_scores else None)
    return (out, scores) if want_scores else out


def pool_positions(sel_row, n_vis) -> np.ndarray:
    """Candidate pool of the hierarchical indexer for one row: the union of the aligned
    8-position blocks that hold the Full layer's selected entries (sel_row, -1 = unused),
    cut to the n_vis visible entries, ascending.  [summary] Architecture Components,
    item 3."""
    sel = _c(sel_row, np.int32)
    pool = np.empty(max(8 * sel.shape[0], 1), dtype=np.int32)
    m = lib().csa2o_pool_positions(_p(sel), sel.shape[0], int(n_vis), _p(pool))
    return pool[:m].copy()


def index_topk_pool(K, max_pages, q_idx, w_idx, k_idx, page_table, seq_id, n_vis, sel,
                    rows=None, want_scores=False):
    """Reindex scoring + Top-K restricted to the candidate pool built from sel [T, K_sel]
    (the Full layer's selection).  Returns idx [n_rows, K] (and scores [n_rows,
    max_pages*64], NaN outside the pool, if want_scores).  [summary] Architecture
    Components, items 2 and 3."""
    q_idx = _c(q_idx, np.uint16)
    T, H_I = q_idx.shape[0], q_idx.shape[1]
    w_idx, k_idx = _c(w_idx, np.float32), _c(k_idx, np.uint16)
    pt, sid, nv = _c(page_table, np.int32), _c(seq_id, np.int32), _c(n_vis, np.int32)
    sel = _c(sel, np.int32)
    rows = _c(np.arange(T) if rows is None else rows, np.int32)
    out = np.empty((rows.shape[0], K), dtype=np.int32)
    scores = (np.full((rows.shape[0], max_pages * PAGE), np.nan) if want_scores else None)
    lib().csa2o_index_topk_pool(T, H_I, K, max_pages, _p(q_idx), _p(w_idx), _p(k_idx),
                                _p(pt), _p(sid), _p(nv), _p(sel), sel.shape[1], _p(rows),
                                rows.shape[0], _p(out), _p(scores) if want_scores else None)
    return (out, scores) if want_scores else out


def sparse_attn(max_pages, q, kv_lat, kv_scl, kv_rope, page_table, seq_id, idx,
                sm_scale=None, rows=None, fmt=0):
    """Global sparse branch.  q bf16 bits [T, H, 576]; planes in physical rows (kv_scl
    [*, 16] E8M0 for fmt 0, [*, 32] E4M3 for fmt 1); idx i32 [T, K].  Returns
    (o [n_rows, H, 512], lse [n_rows, H]) in float64."""
    q = _c(q, np.uint16)
    T, H = q.shape[0], q.shape[1]
    idx = _c(idx, np.int32)
    K = idx.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(DQ)
    rows = _c(np.arange(T) if rows is None else rows, np.int32)
    o = np.empty((rows.shape[0], H, LAT), dtype=np.float64)
    lse = np.empty((rows.shape[0], H), dtype=np.float64)
    lat, scl = _c(kv_lat, np.uint8), _c(kv_scl, np.uint8)
    rope, pt, sid = _c(kv_rope, np.uint16), _c(page_table, np.int32), _c(seq_id, np.int32)
    lib().csa2o_sparse_attn_fmt(H, K, max_pages, _p(q), _p(lat), _p(scl), int(fmt), _p(rope),
                                _p(pt), _p(sid), _p(idx), float(sm_scale), _p(rows),
                                rows.shape[0], _p(o), _p(lse))
    return o, lse


def swa_attn(q_swa, swa_k, swa_v, seq_id, swa_start, swa_len, sm_scale=None, rows=None):
    """Sliding-window branch.  q_swa bf16 bits [T, H, 128]; swa_k/v [B, L_swa, H_kv, 128].
    Returns (o [n_rows, H, 128], lse [n_rows, H]) in float64."""
    q_swa = _c(q_swa, np.uint16)
    T, H = q_swa.shape[0], q_swa.shape[1]
    swa_k, swa_v = _c(swa_k, np.uint16), _c(swa_v, np.uint16)
    L_swa, H_kv = swa_k.shape[1], swa_k.shape[2]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(DSWA)
    rows = _c(np.arange(T) if rows is None else rows, np.int32)
    o = np.empty((rows.shape[0], H, DSWA), dtype=np.float64)
    lse = np.empty((rows.shape[0], H), dtype=np.float64)
    sid, st, ln = _c(seq_id, np.int32), _c(swa_start, np.int32), _c(swa_len, np.int32)
    lib().csa2o_swa_attn(H, H_kv, L_swa, _p(q_swa), _p(swa_k), _p(swa_v), _p(sid), _p(st),
                         _p(ln), float(sm_scale), _p(rows), rows.shape[0], _p(o), _p(lse))
    return o, lse


def resolve_sources(modes):
    """For each layer, the layer whose main KV it reads and the layer whose Top-K indices
    it reads: KV from the nearest Full layer at or before it, indices from the nearest
    Full or Reindex layer at or before it.  [summary] Architecture Components, item 2
    (Full computes its own main KV, indexer key and Top-K; Reindex reuses the preceding
    layer's main KV with fresh Top-K; Reuse borrows both from the preceding layer).  A
    pooled Reindex layer (REINDEX_POOL) is a Reindex layer whose search is the candidate
    pool of the group's first Full layer (item 3)."""
    if not modes or modes[0] != FULL:
        raise ValueError("the first layer of a group must be Full")
    kv_src, idx_src = [], []
    last_kv = last_idx = 0
    for i, m in enumerate(modes):
        if m == FULL:
            last_kv = last_idx = i
        elif m in (REINDEX, REINDEX_POOL):
            last_idx = i
        elif m != REUSE:
            raise ValueError(f"unknown mode {m}")
        kv_src.append(last_kv)
        idx_src.append(last_idx)
    return kv_src, idx_src


def layer_group(layers, K, max_pages, page_table, seq_id, n_vis, swa_start, swa_len,
                sm_scale=None, sm_scale_swa=None, rows=None):
    """Full / Reindex / Reuse layer group.  `layers` is a list of dicts with 'mode', 'q',
    'q_swa', 'swa_k', 'swa_v', and for Full/Reindex/pooled Reindex 'q_idx', 'w_idx',
    'k_idx', for Full the planes 'kv_lat', 'kv_scl', 'kv_rope'.  Pooled Reindex layers
    search the pool of layer 0's selection.  Returns per layer a dict with 'idx'
    (the indices it used), 'o', 'lse', 'o_swa', 'lse_swa' for the listed rows."""
    modes = [L["mode"] for L in layers]
    kv_src, idx_src = resolve_sources(modes)
    T = layers[0]["q"].shape[0]
    rows_ = np.arange(T, dtype=np.int32) if rows is None else np.asarray(rows, np.int32)
    results = []
    for i, L in enumerate(layers):
        if L["mode"] in (FULL, REINDEX):
            # Own scores over all rows the later layers may borrow: compute for all T
            idx_all = index_topk(K, max_pages, L["q_idx"], L["w_idx"], L["k_idx"], page_table,
                                 seq_id, n_vis, rows=np.arange(T))
        elif L["mode"] == REINDEX_POOL:
            idx_all = index_topk_pool(K, max_pages, L["q_idx"], L["w_idx"], L["k_idx"],
                                      page_table, seq_id, n_vis, results[0]["idx_all"],
                                      rows=np.arange(T))
        else:
            idx_all = results[idx_src[i]]["idx_all"]
        kv = layers[kv_src[i]]
        o, lse = sparse_attn(max_pages, L["q"], kv["kv_lat"], kv["kv_scl"], kv["kv_rope"],
                             page_table, seq_id, idx_all, sm_scale, rows=rows_)
        o_w, lse_w = swa_attn(L["q_swa"], L["swa_k"], L["swa_v"], seq_id, swa_start, swa_len,
                              sm_scale_swa, rows=rows_)
        results.append({"idx_all": idx_all, "idx": idx_all[rows_], "o": o, "lse": lse,
                        "o_swa": o_w, "lse_swa": lse_w})
    return results


def num_threads() -> int:
    return lib().csa2o_num_threads()


def footprint_bytes_per_token(modes, lat_bytes=256, scale_bytes=16, rope_bytes=128,
                              idx_bytes=128, ratio=4) -> float:
    m = _c(modes, np.int32)
    return lib().csa2o_footprint_bytes_per_token(_p(m), m.shape[0], lat_bytes, scale_bytes,
                                                  rope_bytes, idx_bytes, ratio)
