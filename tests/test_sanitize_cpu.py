"""The CPU oracle (oracle/oracle.c) and the seeded generator (synth/synth.c) built with
AddressSanitizer and UndefinedBehaviorSanitizer, driven through their Python wrappers over
every entry point on small inputs (ragged visibility, empty rows, both cache formats, pooled
search, SWA, KV pooling, footprint).  Any out-of-bounds access, use of freed memory or
undefined behaviour aborts the child process."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SAN = ["-O1", "-g", "-fPIC", "-shared", "-std=c11", "-fno-fast-math", "-fopenmp",
       "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]

DRIVER = r'''
import sys
import numpy as np
sys.path.insert(0, ROOT)
import synth
import synth.synth as ss
from oracle import oracle as orc
ss._LIB_PATH = SYNTH_SO
orc._LIB_PATH = ORACLE_SO

w = synth.Workload(name="san", B=3, T=5, E=1536, H=16, H_I=3, K=100, H_kv=8, L_swa=200,
                   seed=5, hot="uniform", n_hot=12, shuffle=True,
                   seq_id_rows=[0, 1, 2, 1, 0], n_vis_rows=[1536, 700, 33, 0, 1],
                   swa_start_rows=[0, 72, 10, 5, 199], swa_len_rows=[128, 128, 0, 77, 1])
pt = w.page_table()
rows = np.arange(w.T)
for fmt in (0, 1):
    quant = orc.fp4e4m3_quantize if fmt else orc.mxfp4_quantize
    deq = orc.fp4e4m3_dequantize if fmt else orc.mxfp4_dequantize
    parts = [quant(w.latent_seq(b)) for b in range(w.B)]
    lat = w.to_physical(lambda b: parts[b][0], pt)
    scl = w.to_physical(lambda b: parts[b][1], pt)
    assert np.isfinite(deq(lat[:64], scl[:64])).all()
    rope = w.to_physical(w.rope_seq, pt)
    kidx = w.to_physical(w.k_idx_seq, pt)
    idx, s = orc.index_topk(w.K, w.P, w.q_idx(), w.w_idx(), kidx, pt, w.seq_id(), w.n_vis(),
                            rows=rows, want_scores=True)
    o, lse = orc.sparse_attn(w.P, w.q(), lat, scl, rope, pt, w.seq_id(), idx, rows=rows,
                             fmt=fmt)
    assert np.isneginf(lse[3]).all()
sel = w.selection(40)
pidx, ps = orc.index_topk_pool(w.K, w.P, w.q_idx(), w.w_idx(), kidx, pt, w.seq_id(), w.n_vis(),
                               sel, rows=rows, want_scores=True)
assert (pidx[3] == -1).all()
ow, lw = orc.swa_attn(w.q_swa(), w.swa_k(), w.swa_v(), w.seq_id(), w.swa_start(), w.swa_len(),
                      rows=rows)
c = synth.normal_f32(7, 1, 0, 3 * 4 * 576).reshape(3, 4, 576)
z = synth.normal_f32(7, 2, 0, 3 * 4 * 576).reshape(3, 4, 576)
ci = synth.normal_f32(7, 3, 0, 3 * 4 * 64).reshape(3, 4, 64)
zi = synth.normal_f32(7, 4, 0, 3 * 4 * 64).reshape(3, 4, 64)
orc.kv_append(c, z, ci, zi)
orc.topk_from_scores(np.zeros(50), 64)
orc.footprint_bytes_per_token([0, 1, 2])
synth.permutation(3, 4, 1000)
print("sanitized ok")
'''


def test_oracle_and_generator_under_asan_and_ubsan(tmp_path):
    asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"]).decode().strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's libasan is not installed")
    oracle_so = str(tmp_path / "liboracle_san.so")
    synth_so = str(tmp_path / "libsynth_san.so")
    subprocess.check_call(["gcc", *SAN, os.path.join(ROOT, "oracle", "oracle.c"), "-o",
                           oracle_so, "-lm"])
    subprocess.check_call(["gcc", *SAN, os.path.join(ROOT, "synth", "synth.c"), "-o",
                           synth_so, "-lm"])
    code = (f"ROOT = {ROOT!r}\nORACLE_SO = {oracle_so!r}\nSYNTH_SO = {synth_so!r}\n" + DRIVER)
    env = dict(os.environ, LD_PRELOAD=asan, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "sanitized ok" in out, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
