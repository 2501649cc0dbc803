"""Seeded synthetic inputs for the CSA2 hot path (shared by the oracle's tests and the GPU path).

Only draws and lays out numbers; none of the attention method's arithmetic lives here.
The recipe (shapes, value distributions, hot entries, page shuffles) follows the workloads
named in the pages' problem statement: decode batches at 4K-1M context with 4:1 compressed
entries, a Full->Reindex->Reuse layer group, and a chunked causal prefill.

Stream ids (per layer `l`, added as +16*l):
  1 q, 2 q_swa, 3 q_idx, 4 w_idx, 5 latent, 6 rope, 7 k_idx, 8 swa_k, 9 swa_v,
  10 hot placement, 11 page shuffle.
Counters index the logical (unpaged) arrays in row-major order.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

ENTRIES_PER_PAGE = 64
D_LAT = 512
D_ROPE = 64
D_Q = D_LAT + D_ROPE
D_IDX = 64
D_SWA = 128

FULL, REINDEX, REUSE = 0, 1, 2


def build(force: bool = False) -> str:
    """Compile libsynth.so with gcc (OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        src = os.path.join(_HERE, "synth.c")
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11",
                               src, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64 = ctypes.c_uint64, ctypes.c_int64
        vp = ctypes.c_void_p
        L.synth_u64.restype = u64
        L.synth_u64.argtypes = [u64, u64, u64]
        L.synth_normal_f32.argtypes = [u64, u64, u64, i64, vp]
        L.synth_normal_bf16.argtypes = [u64, u64, u64, i64, ctypes.c_float, vp]
        L.synth_permutation.argtypes = [u64, u64, i64, vp]
        L.synth_sample.argtypes = [u64, u64, i64, i64, vp, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def normal_f32(seed: int, stream: int, offset: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    lib().synth_normal_f32(seed, stream, offset, n, _ptr(out))
    return out


def normal_bf16(seed: int, stream: int, offset: int, n: int, mult: float = 1.0) -> np.ndarray:
    """bf16 bit patterns (uint16) of the same draws as normal_f32, times `mult`."""
    out = np.empty(n, dtype=np.uint16)
    lib().synth_normal_bf16(seed, stream, offset, n, mult, _ptr(out))
    return out


def u64(seed: int, stream: int, counter: int) -> int:
    return int(lib().synth_u64(seed, stream, counter))


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    lib().synth_permutation(seed, stream, n, _ptr(out))
    return out


def sample(seed: int, stream: int, n: int, k: int) -> np.ndarray:
    scratch = np.empty(n, dtype=np.int32)
    out = np.empty(k, dtype=np.int32)
    lib().synth_sample(seed, stream, n, k, _ptr(scratch), _ptr(out))
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    """Shapes of one synthetic CSA2 workload.

    B sequences, T query rows, E compressed entries per sequence (a multiple of 64),
    H query heads (dim 576), H_I indexer heads (dim 64), K selected entries per row,
    H_kv SWA KV heads (dim 128), L_swa SWA buffer tokens per sequence, n_win window.
    """
    name: str
    B: int
    T: int
    E: int
    H: int
    H_I: int
    K: int
    H_kv: int
    L_swa: int
    n_win: int = 128
    seed: int = 1001
    hot: str = "uniform"          # 'uniform' | 'runs' | 'none'
    n_hot: int = 0
    hot_runs: int = 16
    shuffle: bool = True
    prefill: bool = False
    modes: list = field(default_factory=lambda: [FULL])
    # explicit per-row metadata (ragged test cases); None = the workload's own rule
    seq_id_rows: np.ndarray | None = None
    n_vis_rows: np.ndarray | None = None
    swa_start_rows: np.ndarray | None = None
    swa_len_rows: np.ndarray | None = None

    @property
    def P(self) -> int:
        return self.E // ENTRIES_PER_PAGE

    @property
    def n_pages(self) -> int:
        return self.B * self.P

    # ---- per-row metadata -------------------------------------------------
    def seq_id(self) -> np.ndarray:
        if self.seq_id_rows is not None:
            return np.asarray(self.seq_id_rows, np.int32)
        if self.prefill:
            return np.zeros(self.T, dtype=np.int32)
        return (np.arange(self.T, dtype=np.int64) % self.B).astype(np.int32)

    def n_vis(self) -> np.ndarray:
        if self.n_vis_rows is not None:
            return np.asarray(self.n_vis_rows, np.int32)
        if self.prefill:
            # Entry j (raw tokens 4j..4j+3) is visible once its block is complete.
            prefix = self.E - self.T // 4
            i = np.arange(self.T, dtype=np.int64)
            return (prefix + (i + 1) // 4).astype(np.int32)
        return np.full(self.T, self.E, dtype=np.int32)

    def swa_start(self) -> np.ndarray:
        if self.swa_start_rows is not None:
            return np.asarray(self.swa_start_rows, np.int32)
        if self.prefill:
            return np.arange(self.T, dtype=np.int32)
        return np.full(self.T, self.L_swa - self.n_win, dtype=np.int32)

    def swa_len(self) -> np.ndarray:
        if self.swa_len_rows is not None:
            return np.asarray(self.swa_len_rows, np.int32)
        return np.full(self.T, self.n_win, dtype=np.int32)

    def page_table(self) -> np.ndarray:
        if not self.shuffle:
            return np.arange(self.n_pages, dtype=np.int32).reshape(self.B, self.P)
        return permutation(self.seed, 11, self.n_pages).reshape(self.B, self.P)

    # ---- draws ---------------------------------------------------------------
    def q(self, layer: int = 0) -> np.ndarray:
        n = self.T * self.H * D_Q
        return normal_bf16(self.seed, 1 + 16 * layer, 0, n).reshape(self.T, self.H, D_Q)

    def q_swa(self, layer: int = 0) -> np.ndarray:
        n = self.T * self.H * D_SWA
        return normal_bf16(self.seed, 2 + 16 * layer, 0, n).reshape(self.T, self.H, D_SWA)

    def q_idx(self, layer: int = 0) -> np.ndarray:
        n = self.T * self.H_I * D_IDX
        return normal_bf16(self.seed, 3 + 16 * layer, 0, n).reshape(self.T, self.H_I, D_IDX)

    def w_idx(self, layer: int = 0) -> np.ndarray:
        n = self.T * self.H_I
        return np.abs(normal_f32(self.seed, 4 + 16 * layer, 0, n)).reshape(self.T, self.H_I)

    def latent_seq(self, b: int, layer: int = 0) -> np.ndarray:
        """fp32 [E, 512] latent rows of sequence b (logical entry order)."""
        n = self.E * D_LAT
        return normal_f32(self.seed, 5 + 16 * layer, b * n, n).reshape(self.E, D_LAT)

    def rope_seq(self, b: int, layer: int = 0) -> np.ndarray:
        n = self.E * D_ROPE
        return normal_bf16(self.seed, 6 + 16 * layer, b * n, n).reshape(self.E, D_ROPE)

    def hot_entries(self, b: int, layer: int = 0) -> np.ndarray:
        stream = 10 + 16 * layer + 4096 * (b + 1)
        if self.hot == "none" or self.n_hot == 0:
            return np.zeros(0, dtype=np.int32)
        if self.hot == "uniform":
            return np.sort(sample(self.seed, stream, self.E, self.n_hot))
        # 'runs': hot_runs contiguous runs at seeded offsets, one run per equal segment
        seg = self.E // self.hot_runs
        run = self.n_hot // self.hot_runs
        starts = [s * seg + u64(self.seed, stream, s) % (seg - run + 1)
                  for s in range(self.hot_runs)]
        return np.concatenate([np.arange(s, s + run) for s in starts]).astype(np.int32)

    def k_idx_seq(self, b: int, layer: int = 0) -> np.ndarray:
        """bf16 [E, 64] indexer keys of sequence b; hot entries scaled by 4 (exact)."""
        n = self.E * D_IDX
        x = normal_f32(self.seed, 7 + 16 * layer, b * n, n).reshape(self.E, D_IDX)
        hot = self.hot_entries(b, layer)
        x[hot] *= 4.0
        return f32_to_bf16_bits(x)

    def swa_k(self, layer: int = 0) -> np.ndarray:
        n = self.B * self.L_swa * self.H_kv * D_SWA
        return normal_bf16(self.seed, 8 + 16 * layer, 0, n).reshape(
            self.B, self.L_swa, self.H_kv, D_SWA)

    def swa_v(self, layer: int = 0) -> np.ndarray:
        n = self.B * self.L_swa * self.H_kv * D_SWA
        return normal_bf16(self.seed, 9 + 16 * layer, 0, n).reshape(
            self.B, self.L_swa, self.H_kv, D_SWA)

    def selection(self, K_sel: int, stream: int = 48) -> np.ndarray:
        """int32 [T, K_sel]: a seeded selection per row shaped like a Top-K output (distinct
        visible entries, ascending, -1 tail): min(K_sel, n_vis) entries, half of them in
        runs of 8 consecutive entries at seeded offsets (so that several fall in one
        aligned 8-entry block, as selections around hot regions do), the rest uniform."""
        nv = self.n_vis()
        out = np.full((self.T, K_sel), -1, dtype=np.int32)
        for t in range(self.T):
            n = int(nv[t])
            m = min(K_sel, n)
            if m == n:
                out[t, :m] = np.arange(n, dtype=np.int32)
                continue
            picks = set()
            r = 0
            while n >= 16 and len(picks) < m // 2:
                start = u64(self.seed, stream, (t << 20) + r) % (n - 7)
                picks.update(range(start, start + 8))
                r += 1
            rest = sample(self.seed, stream + 1 + 4096 * t, n, min(n, 2 * m))
            for j in rest.tolist():
                if len(picks) >= m:
                    break
                picks.add(j)
            out[t, :m] = np.sort(np.fromiter(picks, dtype=np.int64))[:m]
        return out

    # ---- paging ------------------------------------------------------------
    def physical_rows(self, b: int, pt: np.ndarray | None = None) -> np.ndarray:
        """Physical cache row of each logical entry of sequence b."""
        if pt is None:
            pt = self.page_table()
        j = np.arange(self.E, dtype=np.int64)
        return (pt[b][j // ENTRIES_PER_PAGE].astype(np.int64) * ENTRIES_PER_PAGE
                + j % ENTRIES_PER_PAGE)

    def to_physical(self, per_seq, pt: np.ndarray | None = None) -> np.ndarray:
        """Scatter per-sequence logical arrays [E, ...] (callable b -> array) into the
        paged physical layout [n_pages * 64, ...]."""
        if pt is None:
            pt = self.page_table()
        first = per_seq(0)
        out = np.empty((self.n_pages * ENTRIES_PER_PAGE,) + first.shape[1:], dtype=first.dtype)
        for b in range(self.B):
            arr = first if b == 0 else per_seq(b)
            out[self.physical_rows(b, pt)] = arr
        return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


# The workloads of the pages' problem statement, 1-based as in the text:
#  1 CPU-sized Full-mode decode, 2 decode 64 x 128K (the headline), 3 Full->Reindex->Reuse
#  group 32 x 256K, 4 decode 4 x 1M, 5 chunked causal prefill 4096 on a 512K prefix.
def workload(idx: int) -> Workload:
    if idx == 1:
        return Workload("decode_1x4k_h16_k256", B=1, T=1, E=1024, H=16, H_I=4, K=256,
                        H_kv=16, L_swa=128, seed=1001, hot="uniform", n_hot=32, shuffle=False)
    if idx == 2:
        return Workload("decode_64x128k_h64_k2048", B=64, T=64, E=32768, H=64, H_I=8, K=2048,
                        H_kv=64, L_swa=128, seed=1002, hot="uniform", n_hot=328, shuffle=True)
    if idx == 3:
        return Workload("group_full_reindex_reuse_32x256k", B=32, T=32, E=65536, H=64, H_I=8,
                        K=2048, H_kv=64, L_swa=128, seed=1003, hot="uniform", n_hot=655,
                        shuffle=True, modes=[FULL, REINDEX, REUSE])
    if idx == 4:
        return Workload("decode_4x1m_h64_k2048", B=4, T=4, E=262144, H=64, H_I=8, K=2048,
                        H_kv=64, L_swa=128, seed=1004, hot="runs", n_hot=2624, hot_runs=16,
                        shuffle=True)
    if idx == 5:
        return Workload("prefill_4096_on_512k", B=1, T=4096, E=132096, H=64, H_I=8, K=2048,
                        H_kv=64, L_swa=127 + 4096, seed=1005, hot="none", n_hot=0,
                        shuffle=False, prefill=True)
    raise ValueError(idx)
