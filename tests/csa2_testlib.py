"""Shared helpers of the CSA2 tests: build one seeded workload on both sides and compare.

The host side (HostWorkload) quantizes and computes with the CPU oracle only; the device
side (DeviceWorkload) quantizes and computes with the GPU library only.  The two share the
seeded generator (synth) and nothing else.

Comparison rules (from the problem statement's tolerances):
  Top-K  : index sets equal to the oracle's, except members whose oracle score lies within
           1e-5 relative of the oracle's K-th score (1e-5 * max|s| when that score is 0);
           equal size, strictly ascending, in range, -1 padding identical.
  outputs: compared against the oracle run on the GPU's own index set; per tensor max-abs
           error <= 2e-3 and relative L2 error <= 1e-3; lse max-abs error <= 1e-3 with
           identical -inf positions.
"""
from __future__ import annotations

import numpy as np

import synth
from oracle import oracle as orc

FULL, REINDEX, REUSE, REINDEX_POOL = 0, 1, 2, 3
OWN_INDEX = (FULL, REINDEX, REINDEX_POOL)
O_MAX_ABS, O_REL_L2, LSE_MAX_ABS, TOPK_REL = 2e-3, 1e-3, 1e-3, 1e-5


class HostWorkload:
    """Oracle-side inputs and results for a synth.Workload."""

    def __init__(self, w: synth.Workload, modes=None, fmt=0):
        self.w = w
        self.fmt = fmt
        self.modes = list(modes if modes is not None else w.modes)
        self.pt = w.page_table()
        self.kv = {}
        quant = orc.fp4e4m3_quantize if fmt == 1 else orc.mxfp4_quantize
        for li, m in enumerate(self.modes):
            if m == FULL:
                lat_l, scl_l = [], []
                for b in range(w.B):
                    l, s = quant(w.latent_seq(b, li))
                    lat_l.append(l)
                    scl_l.append(s)
                lat = w.to_physical(lambda b: lat_l[b], self.pt)
                scl = w.to_physical(lambda b: scl_l[b], self.pt)
                rope = w.to_physical(lambda b: w.rope_seq(b, li), self.pt)
                self.kv[li] = (lat, scl, rope)
        self.lat, self.scl, self.rope = self.kv[0]

    def layer_inputs(self, li):
        w, m = self.w, self.modes[li]
        L = {"mode": m, "q": w.q(li), "q_swa": w.q_swa(li), "swa_k": w.swa_k(li),
             "swa_v": w.swa_v(li)}
        if m in OWN_INDEX:
            L.update(q_idx=w.q_idx(li), w_idx=w.w_idx(li),
                     k_idx=w.to_physical(lambda b: w.k_idx_seq(b, li), self.pt))
        if m == FULL:
            lat, scl, rope = self.kv[li]
            L.update(kv_lat=lat, kv_scl=scl, kv_rope=rope)
        return L

    def scores(self, li, rows):
        w = self.w
        L = self.layer_inputs(li)
        _, s = orc.index_topk(w.K, w.P, L["q_idx"], L["w_idx"], L["k_idx"], self.pt,
                              w.seq_id(), w.n_vis(), rows=rows, want_scores=True)
        return s

    def pool_search(self, li, rows, sel):
        """Oracle pooled search of layer li for `rows` over the pool of sel [T, K_sel]:
        (idx [n_rows, K], scores [n_rows, E] with NaN outside the pool)."""
        w = self.w
        L = self.layer_inputs(li)
        return orc.index_topk_pool(w.K, w.P, L["q_idx"], L["w_idx"], L["k_idx"], self.pt,
                                   w.seq_id(), w.n_vis(), sel, rows=rows, want_scores=True)

    def run_layer_group(self, rows):
        """Oracle Top-K scores of the listed rows for every layer (the scores of the layer
        whose indices it uses).  A pooled Reindex layer searches the pool of the oracle's
        own layer-0 selection: its entry has the pooled 'scores' (NaN outside the pool),
        'pooled' True, and layer 0's selection of the rows as 'sel0'."""
        kv_src, idx_src = orc.resolve_sources(self.modes)
        out, cache = [], {}
        sel0 = None
        for li in range(len(self.modes)):
            src = idx_src[li]
            if src not in cache:
                if self.modes[src] == REINDEX_POOL:
                    if sel0 is None:
                        s0 = cache[0]
                        sel0 = -np.ones((self.w.T, self.w.K), np.int32)
                        for r, t in enumerate(rows):
                            n = int(self.w.n_vis()[t])
                            sel0[t] = orc.topk_from_scores(s0[r, :n], self.w.K)
                    cache[src] = self.pool_search(src, rows, sel0)[1]
                else:
                    cache[src] = self.scores(src, rows)
            ent = {"scores": cache[src], "pooled": self.modes[src] == REINDEX_POOL}
            if ent["pooled"]:
                ent["sel0"] = sel0[rows]
            out.append(ent)
        return out

    def attn_on(self, idx_rows, li, rows):
        """Oracle global + SWA outputs of layer li for `rows`, using the given index rows
        (one per listed row)."""
        w = self.w
        kv_src, _ = orc.resolve_sources(self.modes)
        lat, scl, rope = self.kv[kv_src[li]]
        T = w.T
        idx_full = -np.ones((T, idx_rows.shape[1]), np.int32)
        idx_full[rows] = idx_rows
        q, q_swa = w.q(li), w.q_swa(li)
        o, lse = orc.sparse_attn(w.P, q, lat, scl, rope, self.pt, w.seq_id(), idx_full,
                                 rows=rows, fmt=self.fmt)
        ow, lw = orc.swa_attn(q_swa, w.swa_k(li), w.swa_v(li), w.seq_id(), w.swa_start(),
                              w.swa_len(), rows=rows)
        return {"o": o, "lse": lse, "o_swa": ow, "lse_swa": lw}


class DeviceWorkload:
    """GPU-side inputs (device tensors) for a synth.Workload, quantized by the library."""

    def __init__(self, w: synth.Workload, device, modes=None, fmt=0):
        import torch
        from fp4_compressed_sparse_amd import csa2
        self.torch, self.csa2 = torch, csa2
        self.w, self.dev = w, device
        self.fmt = fmt
        self.modes = list(modes if modes is not None else w.modes)
        pt = w.page_table()
        self.pt_host = pt
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
        b16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(
            torch.bfloat16)
        self.t, self.b16 = t, b16
        self.page_table = t(pt.astype(np.int32))
        self.seq_id = t(w.seq_id())
        self.n_vis = t(w.n_vis())
        self.swa_start = t(w.swa_start())
        self.swa_len = t(w.swa_len())
        self.layers = []
        for li, m in enumerate(self.modes):
            L = {"mode": m, "q": b16(w.q(li)), "q_swa": b16(w.q_swa(li)),
                 "swa_k": b16(w.swa_k(li)), "swa_v": b16(w.swa_v(li))}
            if m in OWN_INDEX:
                L["q_idx"] = b16(w.q_idx(li))
                L["w_idx"] = t(w.w_idx(li))
                L["k_idx"] = b16(w.to_physical(lambda b: w.k_idx_seq(b, li), pt)).view(
                    w.n_pages, 64, 64)
                L["idx_out"] = torch.empty((w.T, w.K), dtype=torch.int32, device=device)
            if m == FULL:
                lat = torch.empty((w.n_pages, 64, 256), dtype=torch.uint8, device=device)
                scl = torch.empty((w.n_pages, 64, 32 if fmt == 1 else 16), dtype=torch.uint8,
                                  device=device)
                quant = csa2.fp4e4m3_quantize if fmt == 1 else csa2.mxfp4_quantize
                for b in range(w.B):
                    x = t(w.latent_seq(b, li))
                    dst = t(w.physical_rows(b, pt).astype(np.int64))
                    quant(x, lat, scl, dst)
                L["kv_lat"], L["kv_scl"] = lat, scl
                L["kv_rope"] = b16(w.to_physical(lambda b: w.rope_seq(b, li), pt)).view(
                    w.n_pages, 64, 64)
            L["o"] = torch.empty((w.T, w.H, 512), dtype=torch.float32, device=device)
            L["lse"] = torch.empty((w.T, w.H), dtype=torch.float32, device=device)
            L["o_swa"] = torch.empty((w.T, w.H, 128), dtype=torch.float32, device=device)
            L["lse_swa"] = torch.empty((w.T, w.H), dtype=torch.float32, device=device)
            self.layers.append(L)

    def planes_host(self, li=0):
        L = self.layers[li]
        return (L["kv_lat"].cpu().numpy().reshape(-1, 256),
                L["kv_scl"].cpu().numpy().reshape(-1, L["kv_scl"].shape[-1]))

    def group_args(self):
        w = self.w
        return self.csa2.group_args(w.T, w.B, w.H, w.H_I, w.K, w.H_kv, w.L_swa, w.P, w.n_pages,
                                    self.page_table, self.seq_id, self.n_vis, self.swa_start,
                                    self.swa_len, kv_format=self.fmt)

    def descs(self):
        c = self.csa2
        out = []
        for L in self.layers:
            m = L["mode"]
            out.append(c.layer_desc(
                m, L["q"], L["o"], L["lse"], q_swa=L["q_swa"], q_idx=L.get("q_idx"),
                w_idx=L.get("w_idx"), k_idx=L.get("k_idx"), kv_lat=L.get("kv_lat"),
                kv_scl=L.get("kv_scl"), kv_rope=L.get("kv_rope"), swa_k=L["swa_k"],
                swa_v=L["swa_v"], idx_out=L.get("idx_out"), o_swa=L["o_swa"],
                lse_swa=L["lse_swa"]))
        return out

    def run_layer_group(self, to_host=True):
        self.csa2.layer_group(self.descs(), self.group_args(), device=self.dev)
        if not to_host:
            return None
        _, idx_src = orc.resolve_sources(self.modes)
        res = []
        for li, L in enumerate(self.layers):
            res.append({"idx": self.layers[idx_src[li]]["idx_out"].cpu().numpy(),
                        "o": L["o"].cpu().numpy(), "lse": L["lse"].cpu().numpy(),
                        "o_swa": L["o_swa"].cpu().numpy(), "lse_swa": L["lse_swa"].cpu().numpy()})
        return res


# ------------------------------------------------------------------ comparisons
def check_topk(idx_gpu, scores, K, n_vis, rows=None):
    """idx_gpu: [T or n_rows, K]; scores: oracle scores [n_rows, E] of the same rows."""
    rows = np.arange(scores.shape[0]) if rows is None else np.asarray(rows)
    n_boundary = 0
    for r, t in enumerate(rows):
        n = int(n_vis[t])
        g = np.asarray(idx_gpu[t] if idx_gpu.shape[0] != len(rows) else idx_gpu[r])
        m = min(K, n)
        assert np.all(g[m:] == -1), f"row {t}: padding"
        sel = g[:m]
        assert np.all(sel >= 0) and np.all(sel < n), f"row {t}: index out of range"
        assert np.all(np.diff(sel) > 0), f"row {t}: not strictly ascending"
        s = scores[r, :n]
        ref = orc.topk_from_scores(s, K)[:m]
        diff = np.setxor1d(sel, ref)
        if diff.size:
            order = np.lexsort((np.arange(n), -s))
            tau = s[order[m - 1]]
            tol = TOPK_REL * (abs(tau) if tau != 0 else np.abs(s).max())
            bad = diff[np.abs(s[diff] - tau) > tol]
            assert bad.size == 0, (f"row {t}: {bad.size} index differences beyond the score "
                                   f"tolerance (tau={tau}, worst gap "
                                   f"{np.abs(s[bad] - tau).max()})")
            n_boundary += diff.size
    return n_boundary


def check_topk_pool(idx_gpu, scores, K, rows=None):
    """Pooled search: scores [n_rows, E] hold the oracle's scores on the pool and NaN
    elsewhere.  Same rules as check_topk, over the pool: min(K, pool size) picks, all in
    the pool, ascending, -1 padded; equal to the oracle's pooled selection except within
    the score tolerance of its K-th pool score."""
    rows = np.arange(scores.shape[0]) if rows is None else np.asarray(rows)
    n_boundary = 0
    for r, t in enumerate(rows):
        s = scores[r]
        pool = np.flatnonzero(~np.isnan(s))
        g = np.asarray(idx_gpu[t] if idx_gpu.shape[0] != len(rows) else idx_gpu[r])
        m = min(K, pool.size)
        assert np.all(g[m:] == -1), f"row {t}: padding"
        sel = g[:m]
        assert np.all(np.isin(sel, pool)), f"row {t}: pick outside the pool"
        assert np.all(np.diff(sel) > 0), f"row {t}: not strictly ascending"
        sp = s[pool]
        order = np.lexsort((pool, -sp))
        ref = pool[order[:m]]
        diff = np.setxor1d(sel, ref)
        if diff.size:
            tau = sp[order[m - 1]]
            tol = TOPK_REL * (abs(tau) if tau != 0 else np.abs(sp).max())
            bad = diff[np.abs(s[diff] - tau) > tol]
            assert bad.size == 0, (f"row {t}: {bad.size} pooled index differences beyond the "
                                   f"score tolerance (tau={tau})")
            n_boundary += diff.size
    return n_boundary


def _cmp(name, got, ref, max_abs, rel_l2):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    err = np.abs(got - ref)
    ma = err.max() if err.size else 0.0
    nrm = np.linalg.norm(ref)
    rl = np.linalg.norm(got - ref) / nrm if nrm > 0 else np.linalg.norm(got - ref)
    assert ma <= max_abs, f"{name}: max-abs error {ma:.3e} > {max_abs}"
    assert rl <= rel_l2, f"{name}: rel-L2 error {rl:.3e} > {rel_l2}"
    return ma, rl


def _cmp_lse(name, got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    ninf_g, ninf_r = np.isneginf(got), np.isneginf(ref)
    assert np.array_equal(ninf_g, ninf_r), f"{name}: -inf positions differ"
    fin = ~ninf_r
    ma = np.abs(got[fin] - ref[fin]).max() if fin.any() else 0.0
    assert ma <= LSE_MAX_ABS, f"{name}: max-abs error {ma:.3e} > {LSE_MAX_ABS}"
    return ma


def check_attn(res, ref, rows=None, swa=True):
    """res: GPU results (full T); ref: oracle results for `rows` (default all)."""
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    stats = {"o": _cmp("o", sel(res["o"]), ref["o"], O_MAX_ABS, O_REL_L2),
             "lse": _cmp_lse("lse", sel(res["lse"]), ref["lse"])}
    if swa:
        stats["o_swa"] = _cmp("o_swa", sel(res["o_swa"]), ref["o_swa"], O_MAX_ABS, O_REL_L2)
        stats["lse_swa"] = _cmp_lse("lse_swa", sel(res["lse_swa"]), ref["lse_swa"])
    return stats
