#!/usr/bin/env python3
"""Benchmark of the CSA2 decode hot path on one MI355X.

Workload (the headline decode case): 64 query rows, each with its own 128K-token context
compressed 4:1 into 32,768 MXFP4 entries (512-d E2M1 latent + per-32 E8M0 scales + 64-d
bf16 rope, paged in 64-entry pages through a shuffled page table), 64 query heads of dim
576, an 8-head x 64 bf16 indexer, Top-K = 2048, and a bf16 sliding window of 128 tokens
with 64 KV heads of dim 128.  Seeded synthetic N(0,1) data, 1% hot indexer keys.

One step = one Full-mode CSA2 layer through csa2_layer_group: indexer scoring, Top-K,
FP4 gather attention (+ split merge) and the SWA branch (on the library's side stream,
concurrent with the others), inputs resident in HBM.  The step clock runs without
per-kernel events and cycles through independent copies of the inputs, so that no step
finds its inputs in the last-level cache; a separate pass of the same steps, run before
the clock, brackets every launch with HIP events on the stream it runs on, after a read
sweep that evicts the last-level cache before each step.  A steady-state step (the same
loop after 150 more steps) is reported beside the value, not in it.  Prints one JSON line (metric: decode query-tokens/s), with the roofline of the
dominant kernel of the critical path (the global branch; algorithmic bytes / its average
duration) and the CPU oracle timed on a sample of the same workload.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2,
                    help="1..5: which named workload (2 = the headline decode)")
    ap.add_argument("--cpu-rows", type=int, default=64,
                    help="query rows of the CPU-oracle baseline sample (0 = skip)")
    ap.add_argument("--flush-mb", type=int, default=512,
                    help="MiB read before each step of the per-kernel timing pass, so that no "
                         "kernel reads its inputs from the 256 MB last-level cache")
    ap.add_argument("--kernel-pass-only", action="store_true",
                    help="skip the whole-step clock; run only the per-kernel pass (warm-up "
                         "steps included), so that a profiler's kernel averages match it")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the extra lines for the 1M-context decode and the chunked "
                         "prefill workloads")
    ap.add_argument("--kv-layout", default="planes", choices=("packed", "planes"),
                    help="main-KV cache rows: three dense planes (the default) or packed "
                         "(one 400-byte row per entry, 416 with E4M3 scales)")
    ap.add_argument("--kv-format", type=int, default=0, choices=(0, 1),
                    help="main-KV cache format of the timed workload: 0 = MXFP4 (E8M0 per 32), "
                         "1 = E2M1 with an E4M3 scale per 16 channels")
    ap.add_argument("--reindex-pool", action="store_true",
                    help="the workload's Reindex layers search the candidate pool of its Full "
                         "layer (workload 3)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="fold rocprofv3 --pmc output directories of this workload into "
                         "profiles/counters_<workload>.json and exit")
    ap.add_argument("--calibration-dirs", nargs="*", default=[],
                    help="with --summarize-counters: FETCH_SIZE and WRITE_SIZE runs of "
                         "--calibrate-copy")
    ap.add_argument("--peaks-only", action="store_true",
                    help="only measure this GPU's MFMA and LDS peaks")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of known size (counter calibration)")
    ap.add_argument("--graph-probe", action="store_true",
                    help="only time the workload's step replayed from HIP graphs (one per "
                         "input copy) beside the eager step, in this process (one-layer "
                         "workloads)")
    return ap.parse_args()


# ---------------------------------------------------------------------------- inputs
class Inputs:
    """Device-resident inputs of one workload, built from the seeded generator; the MXFP4
    planes are written by the library's own quantizer."""

    def __init__(self, w, dev, fmt=0):
        import numpy as np
        import torch
        from fp4_compressed_sparse_amd import csa2
        row_bytes = 0
        self.w, self.dev, self.csa2 = w, dev, csa2
        pt = w.page_table()
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        b16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(
            torch.bfloat16)
        self.page_table = t(pt.astype(np.int32))
        self.seq_id, self.n_vis = t(w.seq_id()), t(w.n_vis())
        self.swa_start, self.swa_len = t(w.swa_start()), t(w.swa_len())
        rows_per_page = 64
        self.layers = []
        for li, m in enumerate(w.modes):
            L = {"mode": m, "q": b16(w.q(li)), "q_swa": b16(w.q_swa(li)),
                 "swa_k": b16(w.swa_k(li)), "swa_v": b16(w.swa_v(li))}
            if m in (0, 1, 3):
                L["q_idx"], L["w_idx"] = b16(w.q_idx(li)), t(w.w_idx(li))
                kidx = torch.empty((w.n_pages, rows_per_page, 64), dtype=torch.bfloat16,
                                   device=dev)
                for b in range(w.B):
                    kidx.view(-1, 64)[t(w.physical_rows(b, pt))] = b16(w.k_idx_seq(b, li))
                L["k_idx"] = kidx
                L["idx_out"] = torch.empty((w.T, w.K), dtype=torch.int32, device=dev)
            if m == 0:
                lat = torch.empty((w.n_pages, 64, 256), dtype=torch.uint8, device=dev)
                scl = torch.empty((w.n_pages, 64, 32 if fmt else 16), dtype=torch.uint8,
                                  device=dev)
                rope = torch.empty((w.n_pages, 64, 64), dtype=torch.bfloat16, device=dev)
                quant = csa2.fp4e4m3_quantize if fmt else csa2.mxfp4_quantize
                for b in range(w.B):
                    dst = t(w.physical_rows(b, pt))
                    quant(t(w.latent_seq(b, li)), lat, scl, dst)
                    rope.view(-1, 64)[dst] = b16(w.rope_seq(b, li))
                L["kv_lat"], L["kv_scl"], L["kv_rope"] = lat, scl, rope
                if KV_LAYOUT == "packed":         # one row per entry: codes | rope | scales
                    buf, plat, pscl, prope, row_bytes = csa2.kv_packed(w.n_pages, fmt, dev)
                    plat.copy_(lat)
                    pscl.copy_(scl)
                    prope.copy_(rope)
                    del lat, scl, rope
                    L["kv_buf"] = buf
                    L["kv_lat"], L["kv_scl"], L["kv_rope"] = plat, pscl, prope
            L["o"] = torch.empty((w.T, w.H, 512), dtype=torch.float32, device=dev)
            L["lse"] = torch.empty((w.T, w.H), dtype=torch.float32, device=dev)
            L["o_swa"] = torch.empty((w.T, w.H, 128), dtype=torch.float32, device=dev)
            L["lse_swa"] = torch.empty((w.T, w.H), dtype=torch.float32, device=dev)
            self.layers.append(L)
        self.g = csa2.group_args(w.T, w.B, w.H, w.H_I, w.K, w.H_kv, w.L_swa, w.P, w.n_pages,
                                 self.page_table, self.seq_id, self.n_vis, self.swa_start,
                                 self.swa_len, kv_format=fmt, kv_row_bytes=row_bytes)
        self.descs = [csa2.layer_desc(
            L["mode"], L["q"], L["o"], L["lse"], q_swa=L["q_swa"], q_idx=L.get("q_idx"),
            w_idx=L.get("w_idx"), k_idx=L.get("k_idx"), kv_lat=L.get("kv_lat"),
            kv_scl=L.get("kv_scl"), kv_rope=L.get("kv_rope"), swa_k=L["swa_k"],
            swa_v=L["swa_v"], idx_out=L.get("idx_out"), o_swa=L["o_swa"],
            lse_swa=L["lse_swa"]) for L in self.layers]
        need = csa2.workspace_bytes(csa2.OP_LAYER_GROUP, self.g)
        self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

    def step(self):
        self.csa2.layer_group(self.descs, self.g, workspace=self.ws)



LLC_BYTES = 256 << 20                        # MI355X last-level cache (Infinity Cache)
KV_LAYOUT = "planes"                         # main-KV rows of the timed inputs (--kv-layout)


def input_copies(w, fmt=0):
    """How many independent copies of the inputs the whole-step clock cycles through: enough
    that at least twice the last-level cache is streamed between two steps on the same
    copy (bytes per step: the algorithmic bytes, a pooled layer counted as a dense one);
    2 to 8."""
    wd = dataclasses.replace(w, modes=[1 if m == 3 else m for m in w.modes])
    per_step = sum(algorithmic_bytes(wd, None, fmt).values())
    return max(2, min(8, 1 + -(-2 * LLC_BYTES // max(per_step, 1))))


def input_sets(w, dev, fmt=0):
    """Independent copies of the workload's device inputs (same values, own memory): a step
    then finds nothing of its inputs left in the last-level cache by the previous step on
    them, as in a model where the other layers' data passes through that cache between two
    steps of one layer."""
    return [Inputs(w, dev, fmt) for _ in range(input_copies(w, fmt))]


def graph_probe(w, dev, steps, rounds=5):
    """The step replayed from HIP graphs against the eager step, in one process: each input
    copy's layer-group call (SWA side stream, fork and join included) is captured once
    through torch's capture, and replays alternate over the copies like the eager clock.
    Also checks that a replay reproduces the eager call's outputs bit for bit."""
    import torch
    ss = input_sets(w, dev, 0)
    for s in ss:
        s.step()
    torch.cuda.synchronize()
    keys = ("o", "lse", "o_swa", "lse_swa", "idx_out")
    ref = {k: ss[0].layers[0][k].clone() for k in keys}

    def clock(fn):
        res = []
        for _ in range(rounds):
            for i in range(3):
                fn(i)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                fn(i)
            torch.cuda.synchronize()
            res.append((time.perf_counter() - t0) * 1e3 / steps)
        return min(res)

    eager = clock(lambda i: ss[i % len(ss)].step())
    graphs = []
    for s in ss:
        side = torch.cuda.Stream()                 # warm-up on a non-default stream first
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            s.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            s.step()
        graphs.append(g)
    same = True
    for _ in range(2):
        for k in keys:
            ss[0].layers[0][k].zero_()
        torch.cuda.synchronize()
        graphs[0].replay()
        torch.cuda.synchronize()
        same = same and all(torch.equal(ss[0].layers[0][k], ref[k]) for k in keys)
    graph = clock(lambda i: graphs[i % len(graphs)].replay())
    return {"graph_ms_per_step": round(graph, 4), "eager_ms_per_step": round(eager, 4),
            "replay_bit_identical": bool(same), "input_copies": len(ss)}


def graph_probe_child(workload, steps):
    """graph_probe in a child process (a fault there cannot take this process's line with
    it); None for a workload of several layers, whose capture is not timed here."""
    import subprocess
    import synth
    if len(synth.workload(workload).modes) != 1:
        return None
    try:
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--graph-probe",
                            "--workload", str(workload), "--steps", str(steps),
                            "--kv-layout", KV_LAYOUT],
                           capture_output=True, text=True, timeout=300)
        lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
        if r.returncode != 0 or not lines:
            return {"error": f"exit {r.returncode}: {r.stderr.strip()[-300:]}"}
        return json.loads(lines[-1])
    except Exception as e:                         # noqa: BLE001 - reported, not raised
        return {"error": repr(e)[:300]}


# ------------------------------------------------------------------ algorithmic bytes
def pool_sizes(w, sel):
    """Entries in each row's candidate pool: the aligned 8-entry blocks holding the row's
    selected entries (sel [T, K], -1 unused), cut to the visible entries."""
    import numpy as np
    nv = w.n_vis().astype(np.int64)
    out = np.zeros(w.T, np.int64)
    for t in range(w.T):
        blk = np.unique(sel[t][sel[t] >= 0] // 8)
        out[t] = int(np.minimum(8, nv[t] - 8 * blk).sum())
    return out


def algorithmic_bytes(w, pools=None, fmt=0):
    """Bytes each kernel class must move per step (what the method itself reads/writes once,
    not what an implementation re-reads), returned per kernel name of the library:
    per sequence, its indexer keys up to the largest visibility of its rows (128 B each),
    its distinct selected entries (at most min(E, the rows' selections), 400 B each) and the
    union of its rows' SWA windows (H_kv x 128 x 2 x 2 B per token); per row, queries, the
    Top-K output and fp32 outputs.  With one row per sequence (decode) this is the per-row
    scan n_vis x 128 B, gather K x 400 B and window n_win x H_kv x 512 B.  A pooled Reindex
    layer reads each row's pool (pools[t] entries, 128 B each) and its K selections."""
    import numpy as np
    nv = w.n_vis().astype(np.int64)
    sel = np.minimum(nv, w.K)
    sid = w.seq_id().astype(np.int64)
    start = w.swa_start().astype(np.int64)
    win = w.swa_len().astype(np.int64)
    keys = gathered = window = 0
    for b in np.unique(sid):
        r = sid == b
        keys += int(nv[r].max())
        gathered += min(int(w.E), int(sel[r].sum()))
        tok = np.zeros(int((start[r] + win[r]).max()) if r.any() else 0, bool)
        for s0, l in zip(start[r], win[r]):
            tok[s0:s0 + l] = True
        window += int(tok.sum())
    n_idx_layers = sum(1 for m in w.modes if m in (0, 1))
    n_pool_layers = sum(1 for m in w.modes if m == 3)
    n_layers = len(w.modes)
    idx_score = n_idx_layers * (keys * 128 + w.T * w.H_I * (64 * 2 + 4))
    topk = n_idx_layers * w.T * w.K * 4
    entry = 416 if fmt else 400                      # E4M3 per 16: 32 scale bytes, not 16
    attn = n_layers * (gathered * entry + w.T * w.H * (576 * 2 + 512 * 4 + 4))
    swa = n_layers * (window * w.H_kv * 128 * 2 * 2 + w.T * w.H * (128 * 2 + 128 * 4 + 4))
    out = {"idx_score": idx_score, "topk": topk, "sparse_attn": attn, "swa": swa}
    if n_pool_layers:
        out["idx_pool_score"] = n_pool_layers * (int(pools.sum()) * 128 + w.T * w.K * 4 +
                                                 w.T * w.H_I * (64 * 2 + 4))
        out["topk_pool"] = n_pool_layers * w.T * w.K * 4
    return out


def algorithmic_flops(w, pools=None):
    """Matrix-math work per step: indexer 2 H_I 64 n_vis (pool entries for a pooled
    layer), attention 2 H sel (576 + 512), SWA 2 H len 128 x 2 per row (the fp8 hi/lo query
    split is not counted)."""
    import numpy as np
    nv = w.n_vis().astype(np.int64)
    sel = np.minimum(nv, w.K)
    win = w.swa_len().astype(np.int64)
    n_idx_layers = sum(1 for m in w.modes if m in (0, 1))
    n_pool_layers = sum(1 for m in w.modes if m == 3)
    n_layers = len(w.modes)
    return (n_idx_layers * 2 * w.H_I * 64 * int(nv.sum()) +
            n_pool_layers * 2 * w.H_I * 64 * int(pools.sum() if pools is not None else 0) +
            n_layers * 2 * w.H * 1088 * int(sel.sum()) +
            n_layers * 2 * w.H * 256 * int(win.sum()))


def measure_extra(w, dev, steps, warmup, flush_mb, fmt=0):
    """Whole-step time and per-kernel times of another workload (smaller bench)."""
    import torch
    from fp4_compressed_sparse_amd import csa2
    sets = input_sets(w, dev, fmt)
    inp = sets[0]
    for i in range(warmup):
        sets[i % len(sets)].step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        sets[i % len(sets)].step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    scratch = (torch.ones(flush_mb << 18, dtype=torch.float32, device=dev)
               if flush_mb > 0 else None)
    csa2.timing_read()
    csa2.timing_enable(True)
    for _ in range(steps):
        if scratch is not None:
            scratch.sum()
        inp.step()
    torch.cuda.synchronize()
    csa2.timing_enable(False)
    kt = csa2.timing_read()
    pools = (pool_sizes(w, inp.layers[0]["idx_out"].cpu().numpy()) if 3 in w.modes else None)
    algo = algorithmic_bytes(w, pools, fmt)
    flops = algorithmic_flops(w, pools)
    step_bytes = sum(algo.values())
    out = {"workload": w.name, "query_rows": w.T, "entries_per_seq": w.E, "top_k": w.K,
           "input_copies": len(sets),
           "kv_format": "E2M1 + E4M3 per 16" if fmt else "MXFP4 (E2M1 + E8M0 per 32)",
           "kv_layout": KV_LAYOUT,
           "layers": [["full", "reindex", "reuse", "reindex_pool"][m] for m in w.modes],
           "steps": steps, "ms_per_step": round(ms, 4),
           "query_tokens_per_s": round(w.T / (ms * 1e-3), 1),
           "step_algo_bytes": step_bytes,
           "step_hbm_gbs": round(step_bytes / (ms * 1e-3) / 1e9, 1),
           "step_hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "step_algo_flops": flops,
           "step_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
           "step_mfma_frac_bf16": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
           "kernels": {k: {"launches": n, "avg_us": round(t * 1e3 / n, 3)}
                       for k, (n, t) in kt.items()}}
    for k, v in out["kernels"].items():
        if k in algo and k not in ("topk", "topk_pool"):
            v["algo_bytes"] = algo[k] / (v["launches"] / steps)
            v["gbs"] = round(v["algo_bytes"] / (v["avg_us"] * 1e-6) / 1e9, 1)
    if pools is not None:
        out["pool_entries_per_row"] = round(float(pools.mean()), 1)
    del inp
    torch.cuda.empty_cache()
    return out


def measure_append(dev, n, steps, flush_mb):
    """The KV append kernel alone: n entries, each pooled from 4 raw tokens (C and Z of
    576 channels, indexer key and logits of 64), written to scattered cache rows."""
    import numpy as np
    import torch
    import synth
    from fp4_compressed_sparse_amd import csa2
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    c = t(synth.normal_f32(7, 1, 0, n * 4 * 576).reshape(n, 4, 576))
    z = t(synth.normal_f32(7, 2, 0, n * 4 * 576).reshape(n, 4, 576))
    ci = t(synth.normal_f32(7, 3, 0, n * 4 * 64).reshape(n, 4, 64))
    zi = t(synth.normal_f32(7, 4, 0, n * 4 * 64).reshape(n, 4, 64))
    rows = t(synth.permutation(7, 5, n).astype(np.int64))
    lat = torch.empty((n, 256), dtype=torch.uint8, device=dev)
    scl = torch.empty((n, 16), dtype=torch.uint8, device=dev)
    rope = torch.empty((n, 64), dtype=torch.int16, device=dev)
    kidx = torch.empty((n, 64), dtype=torch.int16, device=dev)
    run = lambda: csa2.kv_append(c, z, lat, scl, rope, dst_row=rows, c_idx=ci, z_idx=zi,
                                 k_idx=kidx)
    run()
    scratch = (torch.ones(flush_mb << 18, dtype=torch.float32, device=dev)
               if flush_mb > 0 else None)
    torch.cuda.synchronize()
    csa2.timing_read()
    csa2.timing_enable(True)
    for _ in range(steps):
        if scratch is not None:
            scratch.sum()
        run()
    torch.cuda.synchronize()
    csa2.timing_enable(False)
    launches, ms = csa2.timing_read()["kv_append"]
    us = ms * 1e3 / launches
    algo = n * (2 * 4 * 576 * 4 + 2 * 4 * 64 * 4 + 8 + 256 + 16 + 128 + 128)
    return {"workload": f"kv_append_{n}", "entries": n, "raw_tokens": 4 * n,
            "kernels": {"kv_append": {"launches": launches, "avg_us": round(us, 3),
                                      "algo_bytes": algo,
                                      "gbs": round(algo / (us * 1e-6) / 1e9, 1)}},
            "entries_per_s": round(n / (us * 1e-6), 1)}


KERNEL_SOURCES = {"idx_score": "k_index.hip", "topk": "k_index.hip", "idx_sample": "k_index.hip",
                  "topk_thr": "k_index.hip", "idx_exact": "k_index.hip", "topk_exact": "k_index.hip",
                  "idx_pool_score": "k_index.hip", "topk_pool": "k_index.hip",
                  "topk_ck_hist": "k_index.hip", "topk_ck_compact": "k_index.hip",
                  "topk_ck_select": "k_index.hip", "sparse_attn": "k_attn.hip",
                  "attn_merge": "k_attn.hip", "swa": "k_swa.hip", "kv_append": "k_quant.hip",
                  "mxfp4_quantize": "k_quant.hip"}


def kernel_source_sha(name):
    src = KERNEL_SOURCES.get(name)
    if src is None:
        return None
    path = os.path.join(ROOT, "fp4_compressed_sparse_amd", "csrc", src)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def library_kernel(device_name):
    """The library's timing name of a device kernel symbol (as rocprofv3 prints it)."""
    n = device_name
    # the row-tiled scoring by mode (template argument 2): the sample, the candidate
    # scoring, and the full-key scoring, which the benchmark workloads only run as the exact
    # re-run of rows the candidates could not settle (as does the streamed Top-K)
    if "idx_gemm_kernel" in n:
        return {"1>": "idx_sample", "2>": "idx_score"}.get(n.split("(")[0][-2:], "idx_exact")
    for pat, key in (("idx_score_kernel", "idx_score"), ("topk_thr_kernel", "topk_thr"),
                     ("topk_cand_kernel", "topk"),
                     ("idx_pool_score_kernel", "idx_pool_score"), ("topk_stream_kernel", "topk_exact"),
                     ("topk_ck_hist", "topk_ck_hist"), ("topk_ck_compact", "topk_ck_compact"),
                     ("topk_ck_select", "topk_ck_select"), ("sparse_attn_kernel", "sparse_attn"),
                     ("attn_merge_kernel", "attn_merge"), ("swa_", "swa"),
                     ("kv_append", "kv_append"), ("mxfp4_quantize", "mxfp4_quantize")):
        if pat in n:
            return key
    if "topk_pool_kernel" in n:
        return "topk_pool"
    if "topk_row_kernel" in n:
        return "topk"
    return None


def counter_record(workload_name, kernel):
    """The committed rocprofv3 counter summary of a kernel on a workload
    (profiles/counters_<workload>.json), or None if there is none or the kernel's source
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"counters_{workload_name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel)
    if not rec or rec.get("source_sha") != kernel_source_sha(kernel):
        return None
    return rec


def counter_traffic(workload_name, kernel):
    """HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE) from the committed counter
    summary, or None."""
    rec = counter_record(workload_name, kernel)
    return rec.get("hbm_bytes_per_launch") if rec else None


MFMA_PEAK_TFLOPS = {"f8": 5000.0, "f16": 2500.0, "bf16": 2500.0, "f6f4": 10100.0}


def counter_mfma(workload_name, kernel, avg_us):
    """Matrix-core use of a kernel from its committed counters: FLOPs per launch by operand
    type (SQ_INSTS_VALU_MFMA_MOPS_*, 512 FLOPs per unit) and the fraction of the kernel's
    duration that the whole device's matrix cores need for them at the published dense peak
    of each type (1.0 = every matrix core busy for the whole kernel)."""
    rec = counter_record(workload_name, kernel)
    if not rec or "mfma_flops_per_launch" not in rec:
        return None
    fl = rec["mfma_flops_per_launch"]
    busy_s = sum(v / (MFMA_PEAK_TFLOPS[k] * 1e12) for k, v in fl.items() if k in MFMA_PEAK_TFLOPS)
    return {"flops_per_launch": fl, "tflops": round(sum(fl.values()) / (avg_us * 1e-6) / 1e12, 1),
            "frac_of_device_peak": round(busy_s / (avg_us * 1e-6), 4)}


def summarize_counters(name, dirs, calib_dirs=None):
    """Fold rocprofv3 --pmc runs of bench.py (dirs holding run_counter_collection.csv; one
    counter group per run) into profiles/counters_<name>.json: per library kernel, the mean
    per dispatch of every counter, calibrated HBM bytes and matrix-core FLOPs by type, with
    the hash of the kernel's source.  calib_dirs: FETCH_SIZE and WRITE_SIZE runs of
    --calibrate-copy (1 GiB read and 1 GiB written per dispatch)."""
    import csv
    import glob
    sums, counts, dev_names = {}, {}, {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                k = library_kernel(r["Kernel_Name"])
                if k is None:
                    continue
                c = r["Counter_Name"]
                sums.setdefault(k, {}).setdefault(c, 0.0)
                sums[k][c] += float(r["Counter_Value"])
                counts.setdefault(k, {}).setdefault(c, 0)
                counts[k][c] += 1
                dev_names[k] = r["Kernel_Name"].split("(")[0]
    fetch_factor, write_factor = 2.0, 1.0
    calib = {}
    for d in calib_dirs or []:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                # the in-place add reads and writes the 1 GiB buffer; the fill before it
                # only writes it
                if "_add<" in r["Kernel_Name"]:
                    calib.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if calib.get("FETCH_SIZE"):
        fetch_factor = (1 << 30) / 1024 / (sum(calib["FETCH_SIZE"]) / len(calib["FETCH_SIZE"]))
    if calib.get("WRITE_SIZE"):
        write_factor = (1 << 30) / 1024 / (sum(calib["WRITE_SIZE"]) / len(calib["WRITE_SIZE"]))
    out = {"_calibration": {"fetch_factor": round(fetch_factor, 4),
                            "write_factor": round(write_factor, 4),
                            "how": "a 1 GiB fp32 copy (bench.py --calibrate-copy) read back: "
                                   "bytes = FETCH_SIZE x 1024 x fetch_factor, "
                                   "WRITE_SIZE x 1024 x write_factor"}}
    for k, cs in sums.items():
        mean = {c: v / counts[k][c] for c, v in cs.items()}
        rec = {"kernel": dev_names[k], "dispatches": max(counts[k].values()),
               "source_sha": kernel_source_sha(k),
               "counters_per_dispatch": {c: round(v, 1) for c, v in sorted(mean.items())}}
        if "FETCH_SIZE" in mean and "WRITE_SIZE" in mean:
            rd = mean["FETCH_SIZE"] * 1024 * fetch_factor
            wr = mean["WRITE_SIZE"] * 1024 * write_factor
            rec.update(hbm_read_bytes_per_launch=int(rd), hbm_write_bytes_per_launch=int(wr),
                       hbm_bytes_per_launch=int(rd + wr))
        mops = {t: mean.get(f"SQ_INSTS_VALU_MFMA_MOPS_{t.upper()}") for t in ("f8", "f16",
                                                                             "bf16", "f6f4")}
        if any(v is not None for v in mops.values()):
            rec["mfma_flops_per_launch"] = {t: int(v * 512) for t, v in mops.items() if v}
        out[k] = rec
    path = os.path.join(ROOT, "profiles", f"counters_{name}.json")
    json.dump(out, open(path, "w"), indent=1)
    return path


# ------------------------------------------------------------------ CPU baseline
def cpu_baseline(w, rows, min_seconds=10.0):
    """The CPU oracle as it stands, on `rows` query rows of the same workload: indexer
    scoring, Top-K, sparse FP4 attention and SWA (inputs prepared beforehand)."""
    import numpy as np
    from oracle import oracle as orc
    pt = w.page_table()
    lat_l, scl_l = [], []
    for b in range(w.B):
        l, s = orc.mxfp4_quantize(w.latent_seq(b))
        lat_l.append(l)
        scl_l.append(s)
    lat = w.to_physical(lambda b: lat_l[b], pt)
    scl = w.to_physical(lambda b: scl_l[b], pt)
    rope = w.to_physical(w.rope_seq, pt)
    kidx = w.to_physical(w.k_idx_seq, pt)
    q, q_swa, q_idx, w_idx = w.q(), w.q_swa(), w.q_idx(), w.w_idx()
    swa_k, swa_v = w.swa_k(), w.swa_v()
    sel_rows = np.linspace(0, w.T - 1, rows).round().astype(np.int32)
    sel_rows = np.unique(sel_rows)
    # the sample is repeated until about min_seconds of CPU time have been measured
    reps, dt = 0, 0.0
    while reps == 0 or (dt < min_seconds and reps < 200):
        t0 = time.perf_counter()
        idx = orc.index_topk(w.K, w.P, q_idx, w_idx, kidx, pt, w.seq_id(), w.n_vis(),
                             rows=sel_rows)
        idx_full = -np.ones((w.T, w.K), np.int32)
        idx_full[sel_rows] = idx
        orc.sparse_attn(w.P, q, lat, scl, rope, pt, w.seq_id(), idx_full, rows=sel_rows)
        orc.swa_attn(q_swa, swa_k, swa_v, w.seq_id(), w.swa_start(), w.swa_len(),
                     rows=sel_rows)
        dt += time.perf_counter() - t0
        reps += 1
    return {"value": round(reps * len(sel_rows) / dt, 3), "unit": "query-tokens/s",
            "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"{len(sel_rows)} of {w.T} query rows of one step (indexer scores over "
                      f"all {w.E} entries, Top-K, FP4 sparse attention, SWA), fp64, "
                      f"repeated {reps} times: {dt:.2f} s wall"}


def measure_hbm(dev, reps=5):
    """A reference rate of this GPU's HBM, to read the achieved rates against besides the
    8 TB/s peak: a 1 GiB fp32 copy (1 GiB read + 1 GiB written; bytes moved / time), the
    median of `reps` event-timed runs on torch's stream."""
    import torch
    n = 1 << 28
    x = torch.ones(n, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        y.copy_(x)
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    del x, y
    tc = sorted(ts)[reps // 2]
    return {"copy_gbs": round(8 * n / tc / 1e9, 1),
            "how": "median of 5 event-timed 1 GiB fp32 copies, (read + written bytes) / time"}


def measure_peaks():
    """Peaks measured on this GPU (libcsa2_peaks.so): dense MFMA TFLOP/s per operand type,
    from a loop of independent MFMAs on every SIMD, and the LDS read bandwidth in TB/s.
    Context beside the published peaks that the roofline fractions use."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "fp4_compressed_sparse_amd", "libcsa2_peaks.so"))
    lib.csa2peak_mfma_tflops.restype = ctypes.c_double
    lib.csa2peak_mfma_tflops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.csa2peak_lds_tbs.restype = ctypes.c_double
    lib.csa2peak_lds_tbs.argtypes = []
    kinds = {"bf16_16x16x32": 0, "f16_16x16x32": 1, "fp8xfp4_scaled_16x16x128": 2,
             "fp8_scaled_16x16x128": 3, "fp4_scaled_16x16x128": 4}
    out = {f"mfma_{k}_tflops": round(lib.csa2peak_mfma_tflops(v, 2), 1) for k, v in kinds.items()}
    out["lds_read_tbs"] = round(lib.csa2peak_lds_tbs(), 2)
    out["how"] = ("two 4-wave workgroups per CU, 8 independent MFMA chains per wave, 2048 "
                  "iterations; LDS: one 1024-thread workgroup per CU reading 16 B per lane per "
                  "step, conflict-free; event-timed, median-free mean of 5 launches")
    return out


# ------------------------------------------------------------------ main
def main():
    args = parse_args()
    global KV_LAYOUT
    KV_LAYOUT = args.kv_layout
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the hot path shards by sequence with no "
              f"exchange); --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    if args.summarize_counters:
        import synth
        w = synth.workload(args.workload)
        if args.kv_format:
            w = dataclasses.replace(w, name=w.name + "_e4m3")
        print(summarize_counters(w.name, args.summarize_counters, args.calibration_dirs))
        return

    import torch
    import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")

    if args.peaks_only:
        print(json.dumps(measure_peaks()))
        return

    if args.calibrate_copy:
        n = 1 << 28                          # 1 GiB of fp32 read + 1 GiB written per copy
        x = torch.ones(n, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(max(args.steps, 1)):
            torch.add(x, 0.0, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4,
                          "launches": max(args.steps, 1)}))
        return

    from fp4_compressed_sparse_amd import csa2
    w = synth.workload(args.workload)
    if args.graph_probe:
        if len(w.modes) != 1:
            print("--graph-probe times one-layer workloads only", file=sys.stderr)
            sys.exit(2)
        print(json.dumps(graph_probe(w, dev, args.steps)))
        return
    if args.reindex_pool:
        w = dataclasses.replace(w, name=w.name.replace("reindex", "reindexpool"),
                                modes=[3 if m == 1 else m for m in w.modes])
    if args.kv_format:
        w = dataclasses.replace(w, name=w.name + "_e4m3")
    t_build = time.perf_counter()
    sets = (input_sets(w, dev, args.kv_format) if not args.kernel_pass_only
            else [Inputs(w, dev, args.kv_format)])
    inp = sets[0]
    torch.cuda.synchronize()
    t_build = time.perf_counter() - t_build
    print(f"[bench] {w.name}: {len(sets)} input set(s) built in {t_build:.1f} s",
          file=sys.stderr, flush=True)

    scratch = (torch.ones(args.flush_mb << 18, dtype=torch.float32, device=dev)
               if args.flush_mb > 0 else None)

    def kernel_pass():
        # per-kernel durations: K steps with HIP events around each launch, recorded on the
        # stream that launch runs on; a read sweep before each step evicts the last-level
        # cache (no dirty lines left behind)
        csa2.timing_read()                   # drop anything recorded so far
        csa2.timing_enable(True)
        for _ in range(args.steps):
            if scratch is not None:
                scratch.sum()
            inp.step()
        torch.cuda.synchronize()
        csa2.timing_enable(False)
        return csa2.timing_read()

    elapsed = float("nan")
    hbm = None
    if args.kernel_pass_only:
        csa2.timing_enable(True)
        for i in range(args.warmup):
            if scratch is not None:
                scratch.sum()
            sets[i % len(sets)].step()
        torch.cuda.synchronize()
        kt = kernel_pass()
    else:
        # The per-kernel pass and the copy reference run first, so that the clock below
        # times a GPU at the clocks it sustains under load rather than one coming up from
        # the idle of the input set-up (the first ~50 steps after it run about 4% slower).
        kt = kernel_pass()
        hbm = measure_hbm(dev)
        for i in range(args.warmup):
            sets[i % len(sets)].step()
        torch.cuda.synchronize()
        # whole-step clock: no per-kernel events inside the timed region; consecutive steps
        # run on different input copies, so none finds its inputs in the last-level cache
        t0 = time.perf_counter()
        for i in range(args.steps):
            sets[i % len(sets)].step()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        print(f"[bench] timed {args.steps} steps in {elapsed * 1e3:.2f} ms", file=sys.stderr,
              flush=True)
        # Beside the value (never in it): the same step once the GPU has run it for a while.
        # After an idle the first 100-150 steps run up to 8% slower than the steady state a
        # serving loop sees; 150 more steps, then 100 timed the same way.
        for i in range(150):
            sets[i % len(sets)].step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(100):
            sets[i % len(sets)].step()
        torch.cuda.synchronize()
        ss_ms = (time.perf_counter() - t1) * 1e3 / 100
        steady = {"ms_per_step": round(ss_ms, 4),
                  "query_tokens_per_s": round(w.T / (ss_ms * 1e-3), 1),
                  "steps": 100, "after_steps": args.warmup + args.steps + 150,
                  "how": "the timed loop again, 100 steps after 150 more untimed ones; "
                         "not part of value"}
    ms_step = elapsed * 1e3 / args.steps
    qtok_s = w.T / (ms_step * 1e-3)
    if args.kernel_pass_only:
        ms_step = qtok_s = None
    pools = (pool_sizes(w, inp.layers[0]["idx_out"].cpu().numpy()) if 3 in w.modes else None)
    algo = algorithmic_bytes(w, pools, args.kv_format)
    step_bytes = sum(algo.values())
    kernels = {k: {"launches": n, "avg_us": round(ms * 1e3 / n, 3)} for k, (n, ms) in kt.items()}
    for k, v in kernels.items():
        if k in algo:
            per_launch = algo[k] / (v["launches"] / args.steps)
            v["algo_bytes"] = per_launch
            v["gbs"] = round(per_launch / (v["avg_us"] * 1e-6) / 1e9, 1)
    flops_attn = 2 * w.H * 1088 * int(min(w.E, w.K)) * w.T        # per launch (one layer)

    def roof(kernel):
        dk = kernels[kernel]
        achieved = dk.get("gbs")
        r = {"bound": "hbm", "kernel": kernel, "achieved": achieved, "peak": HBM_PEAK_GBS,
             "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4) if achieved else None,
             "traffic": counter_traffic(w.name, kernel),
             "algo_bytes_per_launch": dk.get("algo_bytes"), "avg_us": dk["avg_us"]}
        cm = counter_mfma(w.name, kernel, dk["avg_us"])
        if cm:
            r["mfma_counters"] = cm
        return r

    # the roofline kernel: the FP4 gather-attention (the kernel the hot path is built
    # around; it sits at the ridge, so its matrix-core use is reported too); the longest
    # kernel of the global branch, the step's critical path, is reported beside it
    roofline = roof("sparse_attn")
    roofline["mfma_algorithmic"] = {
        "flops_per_launch": flops_attn,
        "tflops": round(flops_attn / (kernels["sparse_attn"]["avg_us"] * 1e-6) / 1e12, 1),
        "frac_bf16_peak": round(flops_attn / (kernels["sparse_attn"]["avg_us"] * 1e-6) / 1e12
                                / MFMA_BF16_PEAK_TFLOPS, 4)}
    critical = max((k for k in kt if k != "swa"), key=lambda k: kt[k][1])
    roofline_cp = roof(critical)

    result = {
        "metric": "decode query-tokens/s and achieved HBM GB/s (% peak) at 128K ctx, Top-K 2048",
        "value": round(qtok_s, 1) if qtok_s else None,
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4) if ms_step else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4+bf16 (bf16/fp16 MFMA, fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.T, "context_tokens": 4 * w.E,
                   "entries_per_seq": w.E, "top_k": w.K, "heads": w.H, "head_dim": 576,
                   "indexer_heads": w.H_I, "swa_window": w.n_win, "swa_kv_heads": w.H_kv,
                   "kv_format": ("E2M1 + E4M3 per 16" if args.kv_format else
                                 "MXFP4 (E2M1, E8M0 per 32)") + " latent 512 + bf16 rope 64",
                   "kv_layout": KV_LAYOUT,
                   "layers": [["full", "reindex", "reuse", "reindex_pool"][m] for m in w.modes],
                   "parallelism": "single GPU"},
        "step_algo_bytes": step_bytes,
        "step_hbm_gbs": round(step_bytes / (ms_step * 1e-3) / 1e9, 1) if ms_step else None,
        "step_hbm_frac": (round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                          if ms_step else None),
        "input_copies": len(sets),
        "kernels": kernels,
        "roofline": roofline,
        "roofline_critical_path": roofline_cp,
    }
    if not args.kernel_pass_only:
        hbm["step_frac_of_copy"] = (round(result["step_hbm_gbs"] / hbm["copy_gbs"], 4)
                                    if ms_step else None)
        achieved = roofline["achieved"]
        hbm["roofline_frac_of_copy"] = (round(achieved / hbm["copy_gbs"], 4)
                                        if achieved else None)
        result["steady_state"] = steady
        result["hbm_measured"] = hbm
        result["peaks_measured"] = measure_peaks()
    if not args.no_extra and not args.kernel_pass_only:
        result["extra"] = []
        w3 = synth.workload(3)
        w3p = dataclasses.replace(w3, name=w3.name.replace("reindex", "reindexpool"),
                                  modes=[0, 3, 2])
        w2e = dataclasses.replace(synth.workload(2), name=synth.workload(2).name + "_e4m3")
        # (the prefill's first ten or so steps run up to 8% slower: 10 timed after 10 more)
        for wx, steps, warm, fmt in ((synth.workload(4), 20, 3, 0), (synth.workload(5), 10, 10, 0),
                                     (w3, 10, 3, 0), (w3p, 10, 3, 0), (w2e, 20, 3, 1)):
            print(f"[bench] extra workload {wx.name}", file=sys.stderr, flush=True)
            result["extra"].append(measure_extra(wx, dev, steps, warm, args.flush_mb, fmt))
        print("[bench] extra: KV append", file=sys.stderr, flush=True)
        result["extra"].append(measure_append(dev, 32768, 20, args.flush_mb))
        # the one-layer decode steps replayed from HIP graphs, beside the eager clock
        if not args.kv_format and not args.reindex_pool:
            print("[bench] graph replay", file=sys.stderr, flush=True)
            result["graph_replay"] = graph_probe_child(args.workload, args.steps)
            for e in result["extra"]:
                if e.get("workload") == synth.workload(4).name:
                    e["graph_replay"] = graph_probe_child(4, 20)
    if args.cpu_rows > 0:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, min(args.cpu_rows, w.T))
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


if __name__ == "__main__":
    main()
