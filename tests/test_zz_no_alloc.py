"""The allocation-free layer group (csa2_layer_group_noalloc) against csa2_layer_group through
the C ABI: two calls in a row, the second on a smaller workload, each bit-identical to the
workspace entry point's outputs on the same inputs."""
import sys

import numpy as np
import pytest

import synth
import csa2_testlib as tl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _w(**kw):
    base = dict(name="t", B=2, T=2, E=1024, H=64, H_I=8, K=256, H_kv=64, L_swa=128, seed=91,
                hot="uniform", n_hot=10, shuffle=True)
    base.update(kw)
    return synth.Workload(**base)


def _outputs(d):
    _, idx_src = tl.orc.resolve_sources(d.modes)
    out = []
    for li, L in enumerate(d.layers):
        out.append({"idx": d.layers[idx_src[li]]["idx_out"].cpu().numpy(),
                    **{k: L[k].cpu().numpy() for k in ("o", "lse", "o_swa", "lse_swa")}})
    return out


def _clear(d):
    for L in d.layers:
        for k in ("o", "lse", "o_swa", "lse_swa"):
            L[k].fill_(float("nan"))
        if "idx_out" in L:
            L["idx_out"].fill_(-7)


def test_noalloc_matches_workspace_entry_point():
    from fp4_compressed_sparse_amd import csa2
    dev = torch.device("cuda:0")
    cases = [
        # a decode group at a size that uses most of the scratch: 3 layers, 16 rows of
        # 65,536 entries (the chunked Top-K is not used: rows of at most 65,536 keys)
        _w(name="noalloc_big", B=4, T=16, E=65536, K=2048, H=64, H_I=8, H_kv=64, n_hot=600,
           seq_id_rows=(np.arange(16) % 4).astype(np.int32), modes=[0, 1, 2]),
        # then a smaller one, so that the second call finds the first call's data in the
        # scratch
        _w(name="noalloc_small", B=2, T=3, E=2048, K=256, H=32, H_I=4, H_kv=16, n_hot=20,
           seq_id_rows=[0, 1, 1], modes=[0, 2]),
    ]
    for w in cases:
        print("[case]", w.name, flush=True)
        d = tl.DeviceWorkload(w, dev)
        need = csa2.workspace_bytes(csa2.OP_LAYER_GROUP, d.group_args())
        assert 0 < need <= csa2.NOALLOC_SCRATCH_BYTES
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=dev)
        csa2.layer_group(d.descs(), d.group_args(), workspace=ws)
        torch.cuda.synchronize()
        ref = _outputs(d)
        _clear(d)
        torch.cuda.synchronize()
        csa2.layer_group_noalloc(d.descs(), d.group_args())
        torch.cuda.synchronize()
        got = _outputs(d)
        for li, (a, b) in enumerate(zip(ref, got)):
            for k in a:
                np.testing.assert_array_equal(a[k], b[k], err_msg=f"{w.name} layer {li} {k}")
