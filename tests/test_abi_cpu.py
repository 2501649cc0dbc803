"""CPU checks of the C ABI: the library loads, exports every function include/csa2.h
declares, the Python structs match the C layout, and host-side validation rejects bad
arguments before any HIP call (no GPU is touched: every call here fails validation or is
an empty T = 0 request)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")


@pytest.fixture(scope="module")
def c():
    from fp4_compressed_sparse_amd import csa2
    return csa2


def header_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", txt)))


def test_exports_every_declared_function(c):
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(c.lib, n), f"{n} not exported"
    assert set(names) == set(c.EXPORTS)


def test_struct_layout_matches_header(c, tmp_path):
    structs = {"csa2_index_args": c.IndexArgs, "csa2_attn_args": c.AttnArgs,
               "csa2_layer_desc": c.LayerDesc, "csa2_group_args": c.GroupArgs,
               "csa2_pool_args": c.PoolArgs, "csa2_append_args": c.AppendArgs}
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', 'int main(){']
    for cname, py in structs.items():
        lines.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'printf("{cname}.{fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c11", str(src), "-o", str(exe)])
    out = subprocess.check_output([str(exe)]).decode().split("\n")
    got = dict(l.split() for l in out if l)
    for cname, py in structs.items():
        assert int(got[cname]) == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert int(got[f"{cname}.{fname}"]) == getattr(py, fname).offset, (cname, fname)


def test_plan_cus_without_a_device(c):
    """With no device to query, the launch plans (and so the workspace sizes) assume one
    MI355X: 256 compute units."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is visible; the GPU test checks the queried count")
    assert c.plan_cus() == 256
    assert c.plan_cus() == 256          # cached


def test_version_and_strings(c):
    assert c.abi_version() == 3
    for st, name in c.STATUS.items():
        assert c.lib.csa2_status_string(st).decode() == name


FAKE = 0x7f0000000000          # aligned, never dereferenced (validation fails first)


def fake(k=0):
    return ctypes.c_void_p(FAKE + 4096 * k)


def good_index(c, **kw):
    a = c.IndexArgs(4, 2, 8, 256, 16, 32, fake(1), fake(2), fake(3), fake(4), fake(5), fake(6),
                    fake(7))
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def call_index(c, a, ws=None, ws_bytes=0):
    st = c.lib.csa2_index_topk(ctypes.byref(a), ws, ws_bytes, None)
    return st, c.lib.csa2_last_error().decode()


@pytest.mark.parametrize("field,value,status", [
    ("H_I", 0, 2), ("H_I", 17, 2), ("K", 0, 2), ("K", 65537, 2), ("T", -1, 2), ("B", 0, 2),
    ("max_pages", 0, 2), ("n_pages", 0, 2), ("n_pages", 1 << 25, 2),
    ("q_idx", None, 1), ("w_idx", None, 1), ("k_idx", None, 1), ("page_table", None, 1),
    ("seq_id", None, 1), ("n_vis", None, 1), ("idx_out", None, 1),
])
def test_index_validation(c, field, value, status):
    a = good_index(c, **{field: value})
    st, msg = call_index(c, a)
    assert st == status, msg
    assert msg


def test_index_alignment_and_workspace(c):
    a = good_index(c, k_idx=ctypes.c_void_p(FAKE + 8))
    st, msg = call_index(c, a)
    assert st == 3 and "k_idx" in msg
    a = good_index(c)
    need = c.lib.csa2_workspace_bytes(c.OP_INDEX_TOPK, ctypes.byref(a))
    assert need == 4 * 16 * 64 * 4
    st, msg = call_index(c, a, None, 0)
    assert st == 5
    st, msg = call_index(c, a, fake(9), need - 1)
    assert st == 5 and "needed" in msg
    st, msg = call_index(c, a, ctypes.c_void_p(FAKE + 16), need)
    assert st == 5 and "aligned" in msg
    assert c.lib.csa2_index_topk(None, None, 0, None) == 1


def test_index_chunked_row_length_limit(c):
    # few rows longer than 65536 entries run chunked, at most 4096 chunks of 4096 per row
    st, msg = call_index(c, good_index(c, max_pages=262145))
    assert st == 6 and "entries" in msg
    assert call_index(c, good_index(c, max_pages=262144))[0] == 5     # valid: workspace next
    assert call_index(c, good_index(c, T=65, max_pages=262145))[0] == 5   # streamed rows


def test_t_zero_is_noop(c):
    a = good_index(c, T=0, q_idx=None, idx_out=None)
    assert call_index(c, a)[0] == 0


def call_pool(c, a, ws=None, ws_bytes=0):
    st = c.lib.csa2_index_topk_pool(ctypes.byref(a), ws, ws_bytes, None)
    return st, c.lib.csa2_last_error().decode()


def test_pool_validation_and_workspace(c):
    good = lambda **kw: c.PoolArgs(good_index(c, **kw), fake(8), 2048)
    # pool size limits: 1..2048 selections, Top-K up to 8192
    for K_sel in (0, 2049):
        a = good()
        a.K_sel = K_sel
        st, msg = call_pool(c, a)
        assert st == 2 and "K_sel" in msg
    st, msg = call_pool(c, good(K=8193))
    assert st == 2 and "K=8193" in msg
    # the searching layer's indexer arguments go through the index validation
    st, msg = call_pool(c, good(q_idx=None))
    assert st == 1 and "q_idx" in msg
    a = good()
    a.sel = None
    st, msg = call_pool(c, a)
    assert st == 1 and "sel" in msg
    a = good()
    a.sel = ctypes.c_void_p(FAKE + 4)
    assert call_pool(c, a)[0] == 3
    # keys: 8 slots per selection and row, whatever the context
    a = good()
    need = c.lib.csa2_workspace_bytes(c.OP_INDEX_TOPK_POOL, ctypes.byref(a))
    assert need == 4 * 8 * 2048 * 4
    st, msg = call_pool(c, a, fake(9), need - 1)
    assert st == 5 and "needed" in msg
    # T = 0: nothing to do, no buffers needed
    a = c.PoolArgs(good_index(c, T=0, q_idx=None, idx_out=None), None, 16)
    assert call_pool(c, a)[0] == 0
    assert c.lib.csa2_index_topk_pool(None, None, 0, None) == 1


def good_attn(c, **kw):
    a = c.AttnArgs(4, 2, 64, 256, 16, 32, fake(1), fake(2), fake(3), fake(4), fake(5), fake(6),
                   fake(7), 1 / 24.0, fake(8), fake(9), 16, 128, fake(10), fake(11), fake(12),
                   fake(13), fake(14), 1 / 11.3, fake(15), fake(16))
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def call_attn(c, a, ws=None, ws_bytes=0):
    st = c.lib.csa2_sparse_attn_fp4(ctypes.byref(a), ws, ws_bytes, None)
    return st, c.lib.csa2_last_error().decode()


@pytest.mark.parametrize("field,value,status", [
    ("H", 48, 2), ("H", 0, 2), ("K", 0, 2), ("H_kv", 3, 2), ("H_kv", 4, 2), ("L_swa", 0, 2),
    ("sm_scale", float("nan"), 2), ("q", None, 1), ("kv_lat", None, 1), ("kv_scl", None, 1),
    ("kv_rope", None, 1), ("idx", None, 1), ("o", None, 1), ("lse", None, 1),
    ("swa_k", None, 1), ("swa_len", None, 1), ("o_swa", None, 1),
])
def test_attn_validation(c, field, value, status):
    a = good_attn(c, **{field: value})
    st, msg = call_attn(c, a)
    assert st == status, msg


def test_attn_kv_format(c):
    st, msg = call_attn(c, good_attn(c, kv_format=2))
    assert st == 6 and "kv_format" in msg
    assert call_attn(c, good_attn(c, kv_format=1))[0] == 5       # valid: reaches workspace
    q = c.lib.csa2_fp4e4m3_quantize
    assert q(None, 4, fake(1), fake(2), None, 0, None) == 1
    assert q(fake(0), -1, fake(1), fake(2), None, 0, None) == 2
    assert q(fake(0), 4, fake(1), ctypes.c_void_p(FAKE + 4), None, 0, None) == 3
    assert q(None, 0, None, None, None, 0, None) == 0
    # E4M3 rows hold 32 scale bytes: packed rows need at least 416 bytes
    assert q(fake(0), 4, fake(1), fake(2), None, 400, None) == 2
    assert q(None, 0, None, None, None, 416, None) == 0


def test_attn_swa_disabled_must_be_consistent(c):
    a = good_attn(c, q_swa=None)
    st, msg = call_attn(c, a)
    assert st == 4 and "swa_k" in msg
    a = good_attn(c, q_swa=None, swa_k=None, swa_v=None, swa_start=None, swa_len=None,
                  o_swa=None, lse_swa=None)
    need = c.lib.csa2_workspace_bytes(c.OP_SPARSE_ATTN, ctypes.byref(a))
    assert need > 0            # 4 rows of K=256 are split across workgroups
    st, msg = call_attn(c, a, None, 0)
    assert st == 5


def test_attn_misaligned(c):
    a = good_attn(c, kv_rope=ctypes.c_void_p(FAKE + 2))
    assert call_attn(c, a)[0] == 3


@pytest.mark.parametrize("fmt,row_bytes,status", [
    (0, 0, 5), (0, 400, 5), (0, 512, 5), (0, 4096, 5), (1, 416, 5), (1, 1024, 5),
    (0, 384, 2), (0, 408, 2), (1, 400, 2), (0, 4112, 2), (0, -400, 2),
])
def test_attn_row_layout(c, fmt, row_bytes, status):
    """kv_row_bytes: 0 (dense planes) or a multiple of 16 holding the whole entry (400 bytes,
    416 with E4M3 scales), up to 4096; valid layouts reach the workspace check."""
    st, msg = call_attn(c, good_attn(c, kv_format=fmt, kv_row_bytes=row_bytes))
    assert st == status, msg
    if status == 2:
        assert "row bytes" in msg


def layer(c, mode, full=True, **kw):
    d = c.LayerDesc(mode, fake(20), fake(21), fake(22), fake(23), fake(24), fake(25), fake(26),
                    fake(27), fake(28), fake(29), fake(30), fake(31), fake(32), fake(33),
                    fake(34))
    if mode != c.FULL:
        d.kv_lat = d.kv_scl = d.kv_rope = None
    if mode == c.REUSE:
        d.q_idx = d.w_idx = d.k_idx = d.idx_out = None
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def group(c, **kw):
    g = c.GroupArgs(4, 2, 64, 8, 256, 64, 128, 16, 32, fake(40), fake(41), fake(42), fake(43),
                    fake(44), 1 / 24.0, 1 / 11.3)
    for k, v in kw.items():
        setattr(g, k, v)
    return g


def call_group(c, layers, g, ws=None, ws_bytes=0):
    arr = (c.LayerDesc * len(layers))(*layers)
    st = c.lib.csa2_layer_group(arr, len(layers), ctypes.byref(g), ws, ws_bytes, None)
    return st, c.lib.csa2_last_error().decode()


def test_group_mode_rules(c):
    F, R, U = c.FULL, c.REINDEX, c.REUSE
    g = group(c)
    # first layer must be Full
    assert call_group(c, [layer(c, R)], g)[0] == 4
    assert call_group(c, [layer(c, U)], g)[0] == 4
    # Reuse must not carry indexer inputs or idx_out; Reindex must not carry KV planes
    assert call_group(c, [layer(c, F), layer(c, U, k_idx=fake(50))], g)[0] == 4
    assert call_group(c, [layer(c, F), layer(c, U, idx_out=fake(50))], g)[0] == 4
    assert call_group(c, [layer(c, F), layer(c, R, kv_lat=fake(50))], g)[0] == 4
    # required buffers
    st, msg = call_group(c, [layer(c, F, kv_scl=None)], g)
    assert st == 1 and "kv_scl" in msg
    st, msg = call_group(c, [layer(c, F), layer(c, R, q_idx=None)], g)
    assert st == 1 and "layer 1" in msg
    bad = layer(c, U)
    bad.mode = 7
    assert call_group(c, [layer(c, F), bad], g)[0] == 4
    # a valid schedule gets as far as the workspace check
    ok = [layer(c, F), layer(c, R), layer(c, U)]
    st, msg = call_group(c, ok, g)
    assert st == 5, msg
    need = c.lib.csa2_workspace_bytes(c.OP_LAYER_GROUP, ctypes.byref(g))
    assert need >= 4 * 16 * 64 * 4
    # a pooled Reindex layer: valid with K <= 2048, rejected above
    pooled = [layer(c, F), layer(c, c.REINDEX_POOL), layer(c, U)]
    assert call_group(c, pooled, g)[0] == 5
    st, msg = call_group(c, pooled, group(c, K=4096))
    assert st == 2 and "pool" in msg
    assert call_group(c, [layer(c, F), layer(c, c.REINDEX_POOL, kv_lat=fake(50))], g)[0] == 4
    # shapes are validated per op
    assert call_group(c, ok, group(c, H=40))[0] == 2
    assert call_group(c, ok, group(c, kv_row_bytes=400))[0] == 5
    st, msg = call_group(c, ok, group(c, kv_row_bytes=200))
    assert st == 2 and "row bytes" in msg
    assert call_group(c, ok, group(c, H_I=99))[0] == 2
    assert c.lib.csa2_layer_group(None, 1, ctypes.byref(g), None, 0, None) == 1


def test_noalloc_group_validation_and_limit(c):
    """The allocation-free layer group validates like csa2_layer_group, is a no-op for T = 0,
    and rejects a group whose workspace exceeds its static scratch (a 4096-row prefill over
    132,096 entries: 2 GiB) before any HIP call."""
    F, R, U = c.FULL, c.REINDEX, c.REUSE
    noalloc = c.lib.csa2_layer_group_noalloc

    def call(layers, g):
        arr = (c.LayerDesc * len(layers))(*layers)
        return noalloc(arr, len(layers), ctypes.byref(g), None), c.lib.csa2_last_error().decode()

    assert call([layer(c, R)], group(c))[0] == 4
    assert call([layer(c, F, q=None)], group(c))[0] == 1
    assert call([layer(c, F), layer(c, U)], group(c, T=0))[0] == 0
    big = group(c, T=4096, B=1, max_pages=2064, n_pages=2064)
    need = c.lib.csa2_workspace_bytes(c.OP_LAYER_GROUP, ctypes.byref(big))
    assert need > c.NOALLOC_SCRATCH_BYTES
    st, msg = call([layer(c, F), layer(c, R), layer(c, U)], big)
    assert st == 5 and "static scratch" in msg, msg


def test_quantize_validation(c):
    q = c.lib.csa2_mxfp4_quantize
    assert q(None, 4, fake(1), fake(2), None, 0, None) == 1
    assert q(fake(0), -1, fake(1), fake(2), None, 0, None) == 2
    assert q(ctypes.c_void_p(FAKE + 4), 4, fake(1), fake(2), None, 0, None) == 3
    assert q(fake(0), 4, fake(1), fake(2), ctypes.c_void_p(FAKE + 8), 0, None) == 3
    assert q(None, 0, None, None, None, 0, None) == 0
    for rb in (16, 392, 408, 4112, -16):                 # short, unaligned or too long rows
        st = q(fake(0), 4, fake(1), fake(2), None, rb, None)
        assert st == 2, rb
        assert "row bytes" in c.lib.csa2_last_error().decode()


def test_kv_append_validation(c):
    def call(**kw):
        a = c.AppendArgs(8, fake(1), fake(2), fake(3), fake(4), fake(5), fake(6), fake(7),
                         fake(8), fake(9))
        for k, v in kw.items():
            setattr(a, k, v)
        return c.lib.csa2_kv_append(ctypes.byref(a), None), c.lib.csa2_last_error().decode()
    assert call(n=-1)[0] == 2
    st, msg = call(z_idx=None)
    assert st == 4 and "c_idx" in msg
    assert call(k_idx=None)[0] == 4
    st, msg = call(c=None)
    assert st == 1 and "c" in msg
    assert call(kv_rope=None)[0] == 1
    assert call(kv_scl=ctypes.c_void_p(FAKE + 4))[0] == 3
    assert call(dst_row=ctypes.c_void_p(FAKE + 8))[0] == 3
    assert call(kv_row_bytes=392)[0] == 2
    assert call(kv_row_bytes=400, kv_lat=None)[0] == 1      # row layout valid, then buffers
    assert call(n=0, c=None, z=None)[0] == 0                 # nothing to write
    assert c.lib.csa2_kv_append(None, None) == 1


def test_workspace_sizes_of_named_workloads(c):
    import synth
    w = synth.workload(2)
    a = c.IndexArgs(w.T, w.B, w.H_I, w.K, w.P, w.n_pages, *([None] * 7))
    assert c.lib.csa2_workspace_bytes(c.OP_INDEX_TOPK, ctypes.byref(a)) == 64 * 32768 * 4
    assert c.lib.csa2_workspace_bytes(c.OP_INDEX_TOPK, None) == 0
    assert c.lib.csa2_workspace_bytes(99, ctypes.byref(a)) == 0
