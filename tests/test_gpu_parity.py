"""GPU parity: the gfx950 library (through its C ABI) against the CPU oracle.

Each case prints its name before running so a failure on the GPU names the case.
"""
import sys

import numpy as np
import pytest

import synth
import csa2_testlib as tl
from oracle import oracle as orc

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def csa2():
    from fp4_compressed_sparse_amd import csa2 as c
    return c


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available()
    return torch.device("cuda:0")


def W(**kw):
    base = dict(name="t", B=2, T=2, E=1024, H=64, H_I=8, K=256, H_kv=64, L_swa=128, seed=77,
                hot="uniform", n_hot=10, shuffle=True)
    base.update(kw)
    return synth.Workload(**base)


SMALL = {
    "cfg1_decode_1x4k_h16": synth.workload(1),
    "ragged_b3_t5_h64_gqa4": W(B=3, T=5, E=1536, K=512, H_kv=16, L_swa=200,
                               seq_id_rows=[0, 1, 2, 1, 0], n_vis_rows=[1536, 700, 33, 1100, 1],
                               swa_start_rows=[0, 72, 199, 10, 5],
                               swa_len_rows=[128, 128, 1, 0, 77]),
    "k_not_tile_multiple_h32_gqa8": W(B=2, T=3, E=640, H=32, H_I=3, K=100, H_kv=4, L_swa=64,
                                      seq_id_rows=[1, 0, 1], n_vis_rows=[640, 99, 350],
                                      swa_start_rows=[0, 0, 3], swa_len_rows=[64, 17, 61]),
    "h128_hi16_k64": W(B=1, T=2, E=512, H=128, H_I=16, K=64, H_kv=128, L_swa=128, n_hot=4),
    "h16_shuffled_b4_k2048": W(B=4, T=4, E=4096, H=16, H_I=4, K=2048, H_kv=16),
    "many_splits_b1_k2048_h64": W(B=1, T=1, E=8192, H=64, H_I=8, K=2048, H_kv=64),
}


def test_plan_cus_is_the_device_cu_count(csa2, dev):
    """The launch plans use the device's own compute-unit count, queried once."""
    n = torch.cuda.get_device_properties(dev).multi_processor_count
    assert csa2.plan_cus() == n


def test_quantize_bit_exact(csa2, dev):
    _say("quantize_bit_exact")
    rng = np.random.default_rng(1)
    rows = 512
    x = synth.normal_f32(5, 1, 0, rows * 512).reshape(rows, 512)
    mult = (2.0 ** rng.integers(-30, 30, size=(rows, 16))).astype(np.float32)
    x = (x.reshape(rows, 16, 32) * mult[:, :, None]).reshape(rows, 512).astype(np.float32)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 7.5], np.float32)
    for r in range(rows):
        blk = rng.integers(0, 16)
        sc = np.float32(2.0 ** rng.integers(-8, 8))
        x[r, blk * 32: blk * 32 + 10] = ties * sc * rng.choice([-1, 1], 10)
    x[0, :32] = 0.0
    x[0, 3] = -0.0
    x[1, :32] = np.float32(1e-40) * np.arange(32)            # subnormal block
    x[2, 32:64] = np.float32(3e38) * rng.choice([-1, 1], 32)  # near the float maximum
    lat_ref, scl_ref = orc.mxfp4_quantize(x)
    xd = torch.from_numpy(x).to(dev)
    lat = torch.zeros((rows, 256), dtype=torch.uint8, device=dev)
    scl = torch.zeros((rows, 16), dtype=torch.uint8, device=dev)
    csa2.mxfp4_quantize(xd, lat, scl)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(lat.cpu().numpy(), lat_ref)
    np.testing.assert_array_equal(scl.cpu().numpy(), scl_ref)
    # scattered destination rows
    perm = rng.permutation(rows + 7)[:rows]
    lat2 = torch.zeros((rows + 7, 256), dtype=torch.uint8, device=dev)
    scl2 = torch.zeros((rows + 7, 16), dtype=torch.uint8, device=dev)
    csa2.mxfp4_quantize(xd, lat2, scl2, torch.from_numpy(perm.astype(np.int64)).to(dev))
    np.testing.assert_array_equal(lat2.cpu().numpy()[perm], lat_ref)
    np.testing.assert_array_equal(scl2.cpu().numpy()[perm], scl_ref)


# ---------------------------------------------------------------- KV append
def _e2m1_midpoints():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "e2m1_codes.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    grid = sorted({abs(float(r[1])) for r in rows})
    return (np.array(grid[1:]) + np.array(grid[:-1])) / 2


def _check_append(got, y, tol):
    """got: GPU planes (lat, scl, rope, k_idx) of the written rows; y: the oracle's pooled
    values (float64 [n, 576] and [n, 64]); tol: absolute pooling tolerance per element.
    Codes, scales and bf16 values must equal the oracle's cache write of y except where y
    lies within tol of a decision boundary (a grid midpoint, a power of two for the shared
    exponent, a bf16 midpoint); there the GPU may take the neighbouring value."""
    n = y.shape[0]
    y_lat, t_lat = y[:, :512], tol[:, :512]
    ref_lat, ref_scl = orc.mxfp4_quantize(y_lat.astype(np.float32))
    Xg = got["scl"].astype(np.int64) - 127
    Xr = ref_scl.astype(np.int64) - 127
    amax = np.abs(y_lat).reshape(n, 16, 32).max(-1)
    tmax = t_lat.reshape(n, 16, 32).max(-1)
    same_x = Xg == Xr
    edge = np.abs(amax - 2.0 ** (np.maximum(Xg, Xr) + 2)) <= tmax
    assert np.all(same_x | edge), "shared exponent differs away from a power of two"
    unpack = lambda lat: np.stack([lat & 15, lat >> 4], -1).reshape(n, 512)
    cg, cr = unpack(got["lat"]), unpack(ref_lat)
    mids = _e2m1_midpoints()
    sc = 2.0 ** -np.repeat(Xr, 32, axis=1)
    tt = np.abs(y_lat) * sc
    near = (np.abs(tt[..., None] - mids).min(-1) <= t_lat * sc) | (np.abs(y_lat) <= t_lat)
    blk_ok = np.repeat(same_x, 32, axis=1)
    bad = blk_ok & (cg != cr) & ~near
    assert not bad.any(), f"{bad.sum()} MXFP4 codes differ away from a rounding boundary"
    adj = np.abs((cg & 7).astype(int) - (cr & 7).astype(int)) <= 1
    assert np.all(adj | ~blk_ok), "a code differs by more than one grid step"
    n_edge = int((blk_ok & (cg != cr)).sum()) + int((~same_x).sum())
    for key, yy, tt_ in (("rope", y[:, 512:], tol[:, 512:]), ("k_idx", got.get("y_idx"),
                                                                 got.get("t_idx"))):
        if yy is None:
            continue
        g = got[key]
        r = orc.round_bf16(yy)
        gv = synth.bf16_bits_to_f32(g).astype(np.float64)
        # a differing value must be the rounding of something within tol of y: at most
        # tol plus half a bf16 step (<= |y| 2^-8 + |gv| 2^-8) away
        near = np.abs(gv - yy) <= tt_ + (np.abs(yy) + np.abs(gv)) * 2.0 ** -8
        assert np.all((g == r) | near), f"{key}: bf16 value outside the tolerance"
        n_edge += int((g != r).sum())
    return n_edge


def _append_case(n, seed, with_idx=True, dst=True):
    c = synth.normal_f32(seed, 1, 0, n * 4 * 576).reshape(n, 4, 576)
    z = (2.0 * synth.normal_f32(seed, 2, 0, n * 4 * 576)).reshape(n, 4, 576).astype(np.float32)
    if n >= 40:
        z[0:10] = 0.5                                # equal logits: the mean
        z[10:20] = 0.0
        z[10:20, 2] = 30.0                           # one token dominates
        c[20:25, :, 64:96] = 0.0                     # an all-zero scale block
        c[25:30] *= np.float32(2.0 ** 20)
        c[30:35] *= np.float32(2.0 ** -20)
        z[35:40] *= np.float32(40.0)                 # near-hard selections
    ci = zi = None
    if with_idx:
        ci = synth.normal_f32(seed, 3, 0, n * 4 * 64).reshape(n, 4, 64)
        zi = (2.0 * synth.normal_f32(seed, 4, 0, n * 4 * 64)).reshape(n, 4, 64).astype(np.float32)
    rows = (np.random.default_rng(seed).permutation(n + 50)[:n].astype(np.int64) if dst
            else np.arange(n, dtype=np.int64))
    return c, z, ci, zi, rows


@pytest.mark.parametrize("n,with_idx,dst", [(1000, True, True), (5, False, False),
                                            (1, True, True)])
def test_kv_append_parity(csa2, dev, n, with_idx, dst):
    _say("kv_append", n, with_idx, dst)
    c, z, ci, zi, rows = _append_case(n, 17 + n, with_idx, dst)
    R = int(rows.max()) + 1
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    lat = torch.zeros((R, 256), dtype=torch.uint8, device=dev)
    scl = torch.zeros((R, 16), dtype=torch.uint8, device=dev)
    rope = torch.zeros((R, 64), dtype=torch.int16, device=dev)
    kidx = torch.zeros((R, 64), dtype=torch.int16, device=dev) if with_idx else None
    csa2.kv_append(t(c), t(z), lat, scl, rope, dst_row=t(rows) if dst else None, c_idx=t(ci),
                   z_idx=t(zi), k_idx=kidx)
    torch.cuda.synchronize()
    ref = orc.kv_append(c, z, ci, zi)
    tol = 4e-6 * np.abs(c).max(axis=1).astype(np.float64) + 1e-37
    got = {"lat": lat.cpu().numpy()[rows], "scl": scl.cpu().numpy()[rows],
           "rope": rope.cpu().numpy().view(np.uint16)[rows]}
    if with_idx:
        got["k_idx"] = kidx.cpu().numpy().view(np.uint16)[rows]
        got["y_idx"] = ref["pooled_idx"]
        got["t_idx"] = 4e-6 * np.abs(ci).max(axis=1).astype(np.float64) + 1e-37
    n_edge = _check_append(got, ref["pooled"], tol)
    assert n_edge <= max(2, n * 576 // 1000), f"{n_edge} boundary cases"
    if n >= 40:   # equal logits give the mean, exactly representable cases stay exact
        np.testing.assert_array_equal(got["scl"][20:25, 2:3], 0)   # zero block: scale 2^-127
    # rows not written stay untouched
    if dst:
        untouched = np.setdiff1d(np.arange(R), rows)
        assert not lat.cpu().numpy()[untouched].any()


def test_fp4e4m3_quantize_bit_exact(csa2, dev):
    """The E4M3-per-16 cache write against the oracle, bit for bit: random blocks over a
    wide range of magnitudes, elements exactly at s x a grid midpoint, maxima whose /6
    falls exactly between two E4M3 values, scales that round to 0, saturate at 448 or are
    subnormal, zero blocks and signed zeros."""
    _say("fp4e4m3_quantize_bit_exact")
    rng = np.random.default_rng(2)
    rows = 512
    x = synth.normal_f32(6, 1, 0, rows * 512).reshape(rows, 512)
    mult = (2.0 ** rng.integers(-24, 12, size=(rows, 32))).astype(np.float32)
    x = (x.reshape(rows, 32, 16) * mult[:, :, None]).reshape(rows, 512).astype(np.float32)
    e4 = np.array([orc.e4m3_decode(b) for b in range(0x7f)])
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for r in range(rows):
        g = rng.integers(0, 32)
        sb = int(rng.integers(1, 0x7e))
        sv = np.float32(e4[sb])
        blk = np.zeros(16, np.float32)
        blk[0] = np.float32(6.0) * sv                      # max -> scale exactly sv
        blk[1:8] = mids * sv * rng.choice([-1, 1], 7)      # ties at s x midpoints
        blk[8:] = rng.standard_normal(8).astype(np.float32) * sv
        x[r, 16 * g: 16 * g + 16] = blk
        g2 = (g + 1) % 32                                  # max / 6 on an E4M3 midpoint
        k = int(rng.integers(1, 0x7d))
        x[r, 16 * g2] = np.float32(6.0 * (e4[k] + e4[k + 1]) / 2)
    x[0, :16] = 0.0
    x[0, 3] = -0.0
    x[1, :16] = np.float32(1e-5) * np.arange(16)          # max / 6 below half of 2^-9: zeros
    x[2, 16:32] = np.float32(3e4) * rng.choice([-1, 1], 16)  # scale saturates at 448
    x[3, 32:48] = np.float32(0.01) * rng.standard_normal(16).astype(np.float32)  # subnormal
    lat_ref, scl_ref = orc.fp4e4m3_quantize(x)
    xd = torch.from_numpy(x).to(dev)
    lat = torch.zeros((rows, 256), dtype=torch.uint8, device=dev)
    scl = torch.zeros((rows, 32), dtype=torch.uint8, device=dev)
    csa2.fp4e4m3_quantize(xd, lat, scl)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(scl.cpu().numpy(), scl_ref)
    np.testing.assert_array_equal(lat.cpu().numpy(), lat_ref)
    perm = rng.permutation(rows + 5)[:rows]
    lat2 = torch.zeros((rows + 5, 256), dtype=torch.uint8, device=dev)
    scl2 = torch.zeros((rows + 5, 32), dtype=torch.uint8, device=dev)
    csa2.fp4e4m3_quantize(xd, lat2, scl2, torch.from_numpy(perm.astype(np.int64)).to(dev))
    np.testing.assert_array_equal(lat2.cpu().numpy()[perm], lat_ref)
    np.testing.assert_array_equal(scl2.cpu().numpy()[perm], scl_ref)


def _index_parity(csa2, dev, w, name, fmt=0):
    _say("index_topk", name)
    d = tl.DeviceWorkload(w, dev, fmt=fmt)
    L = d.layers[0]
    idx = csa2.index_topk(L["q_idx"], L["w_idx"], L["k_idx"], d.page_table, d.seq_id, d.n_vis,
                          w.K)
    torch.cuda.synchronize()
    h = tl.HostWorkload(w, fmt=fmt)
    rows = np.arange(w.T)
    tl.check_topk(idx.cpu().numpy(), h.scores(0, rows), w.K, w.n_vis())
    return d, h, idx


@pytest.mark.parametrize("name", list(SMALL))
def test_index_topk_parity(csa2, dev, name):
    _index_parity(csa2, dev, SMALL[name], name)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("name", list(SMALL))
def test_sparse_attn_parity(csa2, dev, name, fmt):
    w = SMALL[name]
    d, h, idx = _index_parity(csa2, dev, w, name, fmt=fmt)
    _say("sparse_attn", name, "kv_format", fmt)
    L = d.layers[0]
    o, lse, ow, lw = csa2.sparse_attn_fp4(L["q"], L["kv_lat"], L["kv_scl"], L["kv_rope"],
                                          d.page_table, d.seq_id, idx, q_swa=L["q_swa"],
                                          swa_k=L["swa_k"], swa_v=L["swa_v"],
                                          swa_start=d.swa_start, swa_len=d.swa_len,
                                          kv_format=fmt)
    torch.cuda.synchronize()
    rows = np.arange(w.T)
    ref = h.attn_on(idx.cpu().numpy(), 0, rows)
    res = {"o": o.cpu().numpy(), "lse": lse.cpu().numpy(), "o_swa": ow.cpu().numpy(),
           "lse_swa": lw.cpu().numpy()}
    tl.check_attn(res, ref)


def test_attn_arbitrary_index_lists(csa2, dev):
    """Holes, empty rows, unsorted lists and repeated entries (the attention is defined for
    any index list; the oracle runs on the same list)."""
    _say("attn_arbitrary_index_lists")
    w = W(B=2, T=4, E=1024, K=96, H=64, seq_id_rows=[0, 1, 1, 0])
    d = tl.DeviceWorkload(w, dev)
    h = tl.HostWorkload(w)
    rng = np.random.default_rng(3)
    idx = rng.integers(0, 1024, size=(4, 96)).astype(np.int32)
    idx[0, ::3] = -1                 # holes
    idx[1, :] = -1                   # empty row
    idx[2, 40:] = -1                 # ragged tail
    idx[3, 10:20] = idx[3, 0]        # repeated entry
    L = d.layers[0]
    o, lse = csa2.sparse_attn_fp4(L["q"], L["kv_lat"], L["kv_scl"], L["kv_rope"], d.page_table,
                                  d.seq_id, torch.from_numpy(idx).to(dev))
    torch.cuda.synchronize()
    ref = h.attn_on(idx, 0, np.arange(4))
    res = {"o": o.cpu().numpy(), "lse": lse.cpu().numpy()}
    tl.check_attn(res, ref, swa=False)
    assert np.all(res["o"][1] == 0) and np.all(np.isneginf(res["lse"][1]))


def _packed_copy(csa2, L, fmt, row_bytes=None):
    """The layer's dense main-KV planes copied into one buffer of packed rows."""
    buf, lat, scl, rope, rb = csa2.kv_packed(L["kv_lat"].shape[0], fmt, L["kv_lat"].device,
                                             row_bytes)
    lat.copy_(L["kv_lat"])
    scl.copy_(L["kv_scl"])
    rope.copy_(L["kv_rope"])
    return buf, lat, scl, rope, rb


PACKED = ["ragged_b3_t5_h64_gqa4", "k_not_tile_multiple_h32_gqa8", "h16_shuffled_b4_k2048",
          "many_splits_b1_k2048_h64"]


@pytest.mark.parametrize("name", PACKED)
@pytest.mark.parametrize("fmt,row_bytes", [(0, None), (0, 512), (1, None), (1, 448)])
def test_attn_packed_rows_match_planes(csa2, dev, name, fmt, row_bytes):
    """The attention over packed main-KV rows (kv_row_bytes: codes, rope and scales of an
    entry in one row) gives the dense-plane call's outputs bit for bit: the same bytes reach
    the same arithmetic.  Index lists with holes and an empty row."""
    _say("attn_packed_rows", name, fmt, row_bytes)
    w = SMALL[name]
    d = tl.DeviceWorkload(w, dev, modes=[0], fmt=fmt)
    L = d.layers[0]
    rng = np.random.default_rng(11)
    idx = np.sort(rng.integers(0, w.E, size=(w.T, w.K)), axis=1).astype(np.int32)
    idx[0, ::5] = -1
    if w.T > 1:
        idx[1, :] = -1
    idx = torch.from_numpy(idx).to(dev)
    args = (d.page_table, d.seq_id, idx)
    kw = dict(q_swa=L["q_swa"], swa_k=L["swa_k"], swa_v=L["swa_v"], swa_start=d.swa_start,
              swa_len=d.swa_len, kv_format=fmt)
    ref = csa2.sparse_attn_fp4(L["q"], L["kv_lat"], L["kv_scl"], L["kv_rope"], *args, **kw)
    buf, lat, scl, rope, rb = _packed_copy(csa2, L, fmt, row_bytes)
    got = csa2.sparse_attn_fp4(L["q"], lat, scl, rope, *args, kv_row_bytes=rb, **kw)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


@pytest.mark.parametrize("fmt,full", [(0, False), (1, False), (0, True)])
def test_layer_group_packed_rows_match_planes(csa2, dev, fmt, full):
    """A Full -> Reindex -> Reuse group over packed main-KV rows: selections and outputs
    equal the dense-plane group's bit for bit; also the headline decode layer (64 rows over
    32,768 entries, K = 2048) in the step's launch configuration."""
    _say("layer_group_packed_rows", fmt, "full" if full else "small")
    if full:
        w = synth.workload(2)
    else:
        w = W(name="group_packed", B=3, T=3, E=2048, K=256, H=64, H_I=8, H_kv=64, n_hot=20,
              seq_id_rows=[0, 1, 2], n_vis_rows=[2048, 1500, 700], modes=[0, 1, 2])
    d = tl.DeviceWorkload(w, dev, fmt=fmt)
    ref = d.run_layer_group()
    L = d.layers[0]
    buf, lat, scl, rope, rb = _packed_copy(csa2, L, fmt)
    L["kv_lat"], L["kv_scl"], L["kv_rope"] = lat, scl, rope
    for Li in d.layers:
        for k in ("o", "lse", "o_swa", "lse_swa"):
            Li[k].fill_(float("nan"))
        if "idx_out" in Li:
            Li["idx_out"].fill_(-7)
    g = d.group_args()
    g.kv_row_bytes = rb
    csa2.layer_group(d.descs(), g, device=dev)
    torch.cuda.synchronize()
    for li, Li in enumerate(d.layers):
        for k in ("o", "lse", "o_swa", "lse_swa"):
            np.testing.assert_array_equal(Li[k].cpu().numpy(), ref[li][k])
        if "idx_out" in Li:
            np.testing.assert_array_equal(Li["idx_out"].cpu().numpy(), ref[li]["idx"])


@pytest.mark.parametrize("row_bytes", [None, 512])
def test_cache_writes_into_packed_rows(csa2, dev, row_bytes):
    """The quantizers and the KV append write the same bytes into packed rows as into dense
    planes (rows dst_row, in any order), and nothing else: the other parts of a written row
    and the rows not written keep their contents."""
    _say("cache_writes_packed", row_bytes)
    n_pages, n = 20, 1000
    R = 64 * n_pages
    rows = np.random.default_rng(5).permutation(R)[:n].astype(np.int64)
    dst = torch.from_numpy(rows).to(dev)
    x = torch.from_numpy(synth.normal_f32(21, 1, 0, n * 512).reshape(n, 512)).to(dev)
    for fmt, quant in ((0, csa2.mxfp4_quantize), (1, csa2.fp4e4m3_quantize)):
        sb = 32 if fmt == 1 else 16
        lat = torch.zeros((R, 256), dtype=torch.uint8, device=dev)
        scl = torch.zeros((R, sb), dtype=torch.uint8, device=dev)
        quant(x, lat, scl, dst)
        buf, plat, pscl, _, rb = csa2.kv_packed(n_pages, fmt, dev, row_bytes)
        buf.fill_(0xA5)
        quant(x, plat, pscl, dst, row_bytes=rb)
        torch.cuda.synchronize()
        b = buf.cpu().numpy().reshape(R, rb)
        np.testing.assert_array_equal(b[rows, 0:256], lat.cpu().numpy()[rows])
        np.testing.assert_array_equal(b[rows, 384:384 + sb], scl.cpu().numpy()[rows])
        rest = np.ones(rb, bool)
        rest[0:256] = rest[384:384 + sb] = False
        assert np.all(b[rows][:, rest] == 0xA5)
        assert np.all(np.delete(b, rows, axis=0) == 0xA5)
    c, z, ci, zi, _ = _append_case(n, 31, with_idx=True, dst=False)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    lat = torch.zeros((R, 256), dtype=torch.uint8, device=dev)
    scl = torch.zeros((R, 16), dtype=torch.uint8, device=dev)
    rope = torch.zeros((R, 64), dtype=torch.int16, device=dev)
    kidx = torch.zeros((R, 64), dtype=torch.int16, device=dev)
    csa2.kv_append(t(c), t(z), lat, scl, rope, dst_row=dst, c_idx=t(ci), z_idx=t(zi), k_idx=kidx)
    buf, plat, pscl, prope, rb = csa2.kv_packed(n_pages, 0, dev, row_bytes)
    buf.fill_(0x5A)
    kidx2 = torch.zeros_like(kidx)
    csa2.kv_append(t(c), t(z), plat, pscl, prope, dst_row=dst, c_idx=t(ci), z_idx=t(zi),
                   k_idx=kidx2, kv_row_bytes=rb)
    torch.cuda.synchronize()
    b = buf.cpu().numpy().reshape(R, rb)
    np.testing.assert_array_equal(b[rows, 0:256], lat.cpu().numpy()[rows])
    np.testing.assert_array_equal(b[rows, 256:384], rope.cpu().numpy().view(np.uint8)[rows])
    np.testing.assert_array_equal(b[rows, 384:400], scl.cpu().numpy()[rows])
    np.testing.assert_array_equal(kidx2.cpu().numpy(), kidx.cpu().numpy())
    assert np.all(b[rows, 400:] == 0x5A)
    assert np.all(np.delete(b, rows, axis=0) == 0x5A)


def _planes_from(csa2, dev, w, x, h, d):
    """Quantize latent rows x [E, 512] of the single sequence of w on both sides (library
    quantizer on the GPU, oracle quantizer on the host) into each side's planes."""
    pt = w.page_table()
    lat, scl = orc.mxfp4_quantize(x)
    _, _, rope = h.kv[0]
    h.kv[0] = (w.to_physical(lambda b: lat, pt), w.to_physical(lambda b: scl, pt), rope)
    L = d.layers[0]
    dst = torch.from_numpy(w.physical_rows(0, pt).astype(np.int64)).to(dev)
    csa2.mxfp4_quantize(torch.from_numpy(x).to(dev), L["kv_lat"], L["kv_scl"], dst)
    torch.cuda.synchronize()
    got = L["kv_scl"].cpu().numpy().reshape(-1, 16)
    np.testing.assert_array_equal(got, h.kv[0][1])
    return scl


def test_attn_latent_scale_range(csa2, dev):
    """Latent blocks at the edges of the range in which the value product is exact in fp16
    (E8M0 scale bytes 104..140): values are exact from byte 104 up, so rows over blocks of
    bytes 104..140 meet the usual tolerances; below byte 104 a value rounds to fp16's
    subnormal grid (absolute error at most 2^-25 per value), so a row whose picks are all
    such blocks is held to that absolute bound; above byte 140 the product overflows and the
    affected output channels are non-finite (a loud failure, never a wrong finite value)."""
    _say("attn_latent_scale_range")
    w = W(B=1, T=4, E=512, K=128, H=64, seq_id_rows=[0, 0, 0, 0], shuffle=False)
    d = tl.DeviceWorkload(w, dev)
    h = tl.HostWorkload(w)
    rng = np.random.default_rng(17)
    x = w.latent_seq(0).astype(np.float32).reshape(512, 16, 32).copy()
    # entries 0..127: blocks scaled by 2^-27..2^-22 (bytes 98..104); 128..255: by 2^10..2^13
    # (bytes up to 140); 256..383: unscaled; 384: one block at 2^16 (byte 141 or more)
    x[:128] *= (2.0 ** rng.integers(-27, -21, size=(128, 16, 1))).astype(np.float32)
    x[128:256] *= (2.0 ** rng.integers(10, 14, size=(128, 16, 1))).astype(np.float32)
    x[384, 3] *= np.float32(2.0 ** 16)
    x[255, 0, 0] = np.float32(7.9 * 2.0 ** 13)                  # a block at byte 140
    x = x.reshape(512, 512)
    scl = _planes_from(csa2, dev, w, x, h, d)
    assert scl[:128].min() <= 100 and scl[:128].max() == 104
    assert scl[128:256].max() == 140
    assert scl[384, 3] >= 141
    idx = -np.ones((4, 128), np.int32)
    idx[0] = np.arange(128)                                     # all below byte 104
    idx[1] = np.r_[np.arange(0, 128, 2), np.arange(256, 320)]   # small + unscaled
    idx[2] = np.arange(128, 256)                                # bytes up to 140
    idx[3, :64] = np.r_[np.arange(320, 383), 384]               # one block above 140
    L = d.layers[0]
    _, _, rope = h.kv[0]
    lat_h, scl_h, _ = h.kv[0]
    pt = w.page_table()
    # blocks of 2^13 give logits near 10^4, where fp32 accumulation alone exceeds the lse
    # tolerance: row 2 runs with the logit scale reduced by 2^-13 on both sides
    for sm, rows in ((1.0 / 24.0, [0, 1, 3]), (2.0 ** -13 / 24.0, [2])):
        o, lse = csa2.sparse_attn_fp4(L["q"], L["kv_lat"], L["kv_scl"], L["kv_rope"],
                                      d.page_table, d.seq_id, torch.from_numpy(idx).to(dev),
                                      sm_scale=sm)
        torch.cuda.synchronize()
        o, lse = o.cpu().numpy(), lse.cpu().numpy()
        ro, rl = orc.sparse_attn(w.P, w.q(), lat_h, scl_h, rope, pt, w.seq_id(), idx,
                                 sm_scale=sm, rows=np.arange(4))
        for t in rows:
            if t == 0:
                assert np.all(np.isfinite(o[0]))
                err0 = np.abs(o[0] - ro[0]).max()             # 2^-25 per value, plus
                assert err0 <= 2.0 ** -24, err0               # fp32 accumulation
                tl._cmp_lse("lse row 0", lse[:1], rl[:1])
            elif t == 3:
                bad = ~np.isfinite(o[3])
                assert bad[:, 96:128].any() and not bad[:, :96].any() and not bad[:, 128:].any()
            else:
                # outputs in units of the picked blocks' scale (2^13 for row 2), the scale
                # the absolute tolerance is stated for
                u = 2.0 ** 13 if t == 2 else 1.0
                tl.check_attn({"o": o / u, "lse": lse}, {"o": ro[[t]] / u, "lse": rl[[t]]},
                              rows=np.array([t]), swa=False)


def test_attn_e4m3_scale_bytes(csa2, dev):
    """E4M3-per-16 latent planes written directly, with scale bytes over the whole format
    but its NaNs: subnormals m 2^-9 and 0, the largest values (448), and negative scales
    (the oracle decodes the sign bit; no quantizer writes one).  Every value code * scale is
    exact in fp16, so each row meets the usual tolerances in units of its largest value."""
    _say("attn_e4m3_scale_bytes")
    w = W(B=1, T=4, E=512, K=128, H=64, seq_id_rows=[0, 0, 0, 0], shuffle=False)
    d = tl.DeviceWorkload(w, dev, fmt=1)
    h = tl.HostWorkload(w, fmt=1)
    rng = np.random.default_rng(23)
    lat = rng.integers(0, 256, size=(512, 256), dtype=np.uint8)
    not_nan = np.r_[np.arange(0x00, 0x7f), np.arange(0x80, 0xff)]
    scl = np.empty((512, 32), np.uint8)
    scl[:128] = rng.integers(0x00, 0x18, size=(128, 32))        # subnormals, 0, smallest
    scl[128:256] = rng.integers(0x60, 0x7f, size=(128, 32))     # 2^5 .. 448
    scl[256:384] = rng.choice(not_nan, size=(128, 32))          # anything, sign included
    scl[384:] = rng.integers(0x30, 0x41, size=(128, 32))        # 2^-1 .. 2
    scl[5, :4] = np.arange(1, 5)                                # every subnormal step
    scl[130, 0] = 0x7e
    pt = w.page_table()
    _, _, rope = h.kv[0]
    lat_h = w.to_physical(lambda b: lat, pt)
    scl_h = w.to_physical(lambda b: scl, pt)
    L = d.layers[0]
    L["kv_lat"].copy_(torch.from_numpy(lat_h.reshape(L["kv_lat"].shape)).to(dev))
    L["kv_scl"].copy_(torch.from_numpy(scl_h.reshape(L["kv_scl"].shape)).to(dev))
    idx = -np.ones((4, 128), np.int32)
    idx[0] = np.arange(128)
    idx[1] = np.arange(128, 256)
    idx[2] = np.arange(256, 384)
    idx[3, :96] = np.r_[np.arange(384, 448), np.arange(0, 128, 4)]   # ragged, mixed
    e4 = np.array([orc.e4m3_decode(b) for b in range(256)])
    unit = [6 * np.abs(e4[scl[idx[t][idx[t] >= 0]]]).max() for t in range(4)]
    for sm, rows in ((1.0 / 24.0, [0, 3]), (1.0 / (24.0 * 512.0), [1, 2])):
        o, lse = csa2.sparse_attn_fp4(L["q"], L["kv_lat"], L["kv_scl"], L["kv_rope"],
                                      d.page_table, d.seq_id, torch.from_numpy(idx).to(dev),
                                      sm_scale=sm, kv_format=1)
        torch.cuda.synchronize()
        o, lse = o.cpu().numpy(), lse.cpu().numpy()
        ro, rl = orc.sparse_attn(w.P, w.q(), lat_h, scl_h, rope, pt, w.seq_id(), idx,
                                 sm_scale=sm, rows=np.arange(4), fmt=1)
        for t in rows:
            u = unit[t]
            tl.check_attn({"o": o / u, "lse": lse}, {"o": ro[[t]] / u, "lse": rl[[t]]},
                          rows=np.array([t]), swa=False)


def test_workspace_contents_do_not_matter(csa2, dev):
    """The layer group's outputs do not depend on what the workspace held before the call:
    a zeroed and an all-0xFF workspace give bit-identical outputs.  Rows longer than 65,536
    entries (the chunked Top-K and its histograms), a pooled Reindex layer, split
    attention."""
    _say("workspace_contents_do_not_matter")
    w = W(name="poison", B=2, T=4, E=70016, K=512, H=64, H_I=8, H_kv=64, n_hot=300,
          seq_id_rows=[0, 1, 1, 0], modes=[0, 3, 2])
    d = tl.DeviceWorkload(w, dev)
    need = csa2.workspace_bytes(csa2.OP_LAYER_GROUP, d.group_args())
    outs = []
    for fill in (0x00, 0xFF):
        ws = torch.full((need,), fill, dtype=torch.uint8, device=dev)
        for L in d.layers:
            for k in ("o", "lse", "o_swa", "lse_swa"):
                L[k].fill_(float("nan"))
            if "idx_out" in L:
                L["idx_out"].fill_(-7)
        csa2.layer_group(d.descs(), d.group_args(), workspace=ws)
        torch.cuda.synchronize()
        outs.append([{k: L[k].cpu().numpy() for k in ("o", "lse", "o_swa", "lse_swa")} |
                     ({"idx": L["idx_out"].cpu().numpy()} if "idx_out" in L else {})
                     for L in d.layers])
    for li, (a, b) in enumerate(zip(*outs)):
        for k in a:
            np.testing.assert_array_equal(a[k], b[k], err_msg=f"layer {li} {k}")


def test_topk_all_equal_scores(csa2, dev):
    """Every entry scores the same: the lowest K indices win, in order."""
    _say("topk_all_equal_scores")
    E, K = 4096, 300
    key = torch.from_numpy(synth.normal_bf16(9, 1, 0, 64).view(np.int16)).to(dev)
    k_idx = key.view(1, 1, 64).expand(E // 64, 64, 64).contiguous().view(torch.bfloat16)
    q = torch.from_numpy(synth.normal_bf16(9, 2, 0, 2 * 64).view(np.int16)).to(dev).view(
        torch.bfloat16).view(2, 1, 64)
    wv = torch.ones((2, 1), dtype=torch.float32, device=dev)
    pt = torch.arange(E // 64, dtype=torch.int32, device=dev).view(1, -1)
    sid = torch.zeros(2, dtype=torch.int32, device=dev)
    nv = torch.tensor([E, 1000], dtype=torch.int32, device=dev)
    idx = csa2.index_topk(q, wv, k_idx, pt, sid, nv, K).cpu().numpy()
    np.testing.assert_array_equal(idx[0], np.arange(K))
    np.testing.assert_array_equal(idx[1], np.arange(K))


def _bf16_bits(x):
    """float32 -> bf16 bit patterns by truncation (both sides then see the same values)."""
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("P,K", [(512, 2048), (1024, 2048), (512, 9000)],
                         ids=["32k_k2048", "64k_k2048", "32k_k9000"])
def test_topk_row_paths(csa2, dev, P, K):
    """The one-workgroup-per-row Top-K (rows of up to 64K keys) on exact scores (one head,
    a unit query, keys whose first channel carries the score) that steer each of its
    paths, compared with the oracle index for index: fewer than K keys within 32 octaves
    of the row maximum (digit passes from bit 31), one bin larger than the LDS list
    (digit passes over registers), ties at the K-th key inside the list, negative scores,
    a row ending inside the last wave's keys, a row that selects everything, and one whose
    ties at the K-th key are all kept.  Rows of 32K and 64K keys (32 and 64 keys per
    thread), and K above the 8192 outputs that the staged compaction holds."""
    _say("topk_row_paths", P, K)
    rng = np.random.default_rng(2024)
    E = 64 * P
    rows = []
    v = (1.0 + rng.integers(0, 128, E) / 128.0).astype(np.float32)
    v[rng.choice(E, 1000, replace=False)] = np.float32(2.0 ** 40)
    rows.append((v, 1.0, E))
    rows.append((np.full(E, 1.5, np.float32), 1.0, E))
    rows.append((np.float32(1.0) + rng.integers(0, 16, E).astype(np.float32) / np.float32(16), 1.0, E))
    rows.append((np.abs(rng.standard_normal(E)).astype(np.float32) + np.float32(0.01), -1.0, E))
    rows.append((rng.standard_normal(E).astype(np.float32), 1.0, min(20001, E - 7)))
    rows.append((rng.standard_normal(E).astype(np.float32), 1.0, K - 548))
    # every key at the K-th value kept (the bitmap compaction): the top keys come in groups
    # of dup equal bf16 values, K a multiple of dup, spanning under 32 octaves
    dup = 3 if K % 3 == 0 else 2
    pat = np.maximum(0x7F00 - rng.permutation(E) // dup, 0x0080).astype(np.uint32)
    rows.append(((pat << 16).view(np.float32), 1.0, E))
    T = len(rows)
    k_bits = np.zeros((T * E, 64), np.uint16)
    for b, (vals, _, _) in enumerate(rows):
        k_bits[b * E:(b + 1) * E, 0] = _bf16_bits(vals)
    q_bits = np.zeros((T, 1, 64), np.uint16)
    q_bits[:, 0, 0] = _bf16_bits(1.0)
    w = np.array([[r[1]] for r in rows], np.float32)
    pt = (np.arange(T, dtype=np.int32)[:, None] * P + np.arange(P, dtype=np.int32)).astype(np.int32)
    sid = np.arange(T, dtype=np.int32)
    nv = np.array([r[2] for r in rows], np.int32)
    ref = orc.index_topk(K, P, q_bits, w, k_bits, pt, sid, nv)
    bf = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    idx = csa2.index_topk(bf(q_bits), torch.from_numpy(w).to(dev),
                          bf(k_bits).view(T * P, 64, 64), torch.from_numpy(pt).to(dev),
                          torch.from_numpy(sid).to(dev), torch.from_numpy(nv).to(dev), K)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for t in range(T):
        np.testing.assert_array_equal(got[t], ref[t], err_msg=f"row {t}")


# Rows longer than 65536 keys, few of them: the chunked Top-K (4096-key chunks, one
# workgroup each), with a ragged last chunk, chunks past a short row's end and a row that
# selects everything.
CHUNKED = {
    "chunked_t3_70016_k2048": W(B=3, T=3, E=70016, H=16, H_I=4, K=2048, H_kv=16,
                                n_vis_rows=[70016, 66001, 1500], seq_id_rows=[0, 1, 2]),
    "chunked_t2_70016_k6000": W(B=2, T=2, E=70016, H=16, H_I=3, K=6000, H_kv=16,
                                n_vis_rows=[69999, 40000], seq_id_rows=[1, 0], hot="runs",
                                n_hot=600, hot_runs=6),
}


@pytest.mark.parametrize("name", list(CHUNKED))
def test_topk_chunked_parity(csa2, dev, name):
    _index_parity(csa2, dev, CHUNKED[name], name)


# From 256 rows on, scoring runs row-tiled (a tile of rows against each key page): tiles
# that mix sequences, rows past the end of the last tile, ragged and empty visibility, and
# indexer head counts padded to 4, 8 and 16.
def _gemm_rows(T, seqs, seed):
    rng = np.random.default_rng(seed)
    sid = np.repeat(np.arange(len(seqs)), seqs)[:T]
    sid = np.r_[sid, np.zeros(T - len(sid), np.int64)]
    sid[rng.choice(T, 7, replace=False)] = len(seqs) - 1       # strays inside other runs
    return sid.astype(np.int32)


def _gemm_nvis(T, E, seed):
    rng = np.random.default_rng(seed)
    nv = rng.integers(1, E + 1, T)
    nv[:5] = [0, 1, 63, 64, E]
    return nv.astype(np.int32)


GEMM = {
    "rowtiled_t300_b3_hi8": W(B=3, T=300, E=4160, H=16, H_I=8, K=256, H_kv=16,
                              seq_id_rows=_gemm_rows(300, [120, 60, 120], 5),
                              n_vis_rows=_gemm_nvis(300, 4160, 6)),
    "rowtiled_t260_b2_hi3": W(B=2, T=260, E=2112, H=16, H_I=3, K=100, H_kv=16,
                              seq_id_rows=_gemm_rows(260, [200, 60], 7),
                              n_vis_rows=_gemm_nvis(260, 2112, 8)),
    "rowtiled_t257_b1_hi16": W(B=1, T=257, E=2048, H=16, H_I=16, K=512, H_kv=16, hot="runs",
                               n_hot=64, hot_runs=4, seq_id_rows=np.zeros(257, np.int32),
                               n_vis_rows=_gemm_nvis(257, 2048, 9)),
}


@pytest.mark.parametrize("name", list(GEMM))
def test_index_topk_rowtiled_parity(csa2, dev, name):
    _index_parity(csa2, dev, GEMM[name], name)


# Row-tiled rows of at least 16384 keys select through sampled candidates: a threshold per
# row from the keys of every page_gap-th page, the scoring keeping only the keys at or above
# it (at most 128 per 2048-entry chunk, in entry order), the exact Top-K on those.  Rows
# where that fails (too few or too many candidates, a chunk over its cap, K close to the row
# length) go through the exact path again; clustered hot entries overflow chunks.
def _cand_nvis(T, E, K, seed):
    rng = np.random.default_rng(seed)
    nv = rng.integers(K // 2, E + 1, T)
    nv[:10] = [0, 1, K, K + 1, K + 64, 2 * K, E - 1, E, 2048, 2049]
    return nv.astype(np.int32)


CAND = {
    "cand_t300_b3_e20480_k512": W(B=3, T=300, E=20480, H=16, H_I=8, K=512, H_kv=16,
                                  seq_id_rows=_gemm_rows(300, [120, 60, 120], 21),
                                  n_vis_rows=_cand_nvis(300, 20480, 512, 22)),
    "cand_t260_b1_e16384_hi4_runs": W(B=1, T=260, E=16384, H=16, H_I=4, K=1024, H_kv=16,
                                      hot="runs", n_hot=2048, hot_runs=4,
                                      seq_id_rows=np.zeros(260, np.int32),
                                      n_vis_rows=_cand_nvis(260, 16384, 1024, 23)),
    "cand_t256_b2_e33024_hi16_k2048": W(B=2, T=256, E=33024, H=16, H_I=16, K=2048, H_kv=16,
                                        seq_id_rows=(np.arange(256) % 2).astype(np.int32),
                                        n_vis_rows=_cand_nvis(256, 33024, 2048, 24)),
}


@pytest.mark.parametrize("name", list(CAND))
def test_index_topk_candidates_parity(csa2, dev, name):
    _index_parity(csa2, dev, CAND[name], name)


def _cand_direct(csa2, dev, kf, qf, K, T):
    E = kf.shape[0]
    kb = synth.f32_to_bf16_bits(kf)
    qb = synth.f32_to_bf16_bits(qf.reshape(T, 1, 64))
    wv = np.ones((T, 1), np.float32)
    pt = np.arange(E // 64, dtype=np.int32)[None]
    sid = np.zeros(T, np.int32)
    nv = np.full(T, E, np.int32)
    t16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(
        torch.bfloat16)
    ti = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    idx = csa2.index_topk(t16(qb), ti(wv), t16(kb).view(E // 64, 64, 64), ti(pt), ti(sid),
                          ti(nv), K).cpu().numpy()
    return idx, (qb, wv, kb, pt, sid, nv)


def test_topk_candidates_all_equal_scores(csa2, dev):
    """Every key equal: every row's candidates overflow, the exact path keeps the lowest
    indices."""
    _say("topk_candidates_all_equal_scores")
    E, K, T = 16384, 300, 260
    kf = np.tile(synth.normal_f32(9, 1, 0, 64), (E, 1))
    qf = synth.normal_f32(9, 2, 0, T * 64)
    idx, _ = _cand_direct(csa2, dev, kf, qf, K, T)
    for r in range(T):
        np.testing.assert_array_equal(idx[r], np.arange(K))


@pytest.mark.parametrize("boost", ["sampled", "unsampled"])
def test_topk_candidates_sample_misses(csa2, dev, boost):
    """Rows whose sample misleads the threshold: the keys of the sampled pages (every
    ceil(pages / 64)-th page: every fourth at 16384 keys) scaled x8, so fewer than K keys
    reach it, or the other pages' keys scaled x8, so that chunks overflow.  Both go through
    the exact path and match the oracle."""
    _say("topk_candidates_sample_misses", boost)
    E, K, T = 16384, 512, 258
    page = np.arange(E) // 64
    gap = -(-(E // 64) // 64)
    in_sample = page % gap == 0
    kf = np.abs(synth.normal_f32(12, 1, 0, E * 64)).reshape(E, 64)
    kf[in_sample if boost == "sampled" else ~in_sample] *= 8.0
    qf = np.abs(synth.normal_f32(12, 2, 0, T * 64))
    idx, (qb, wv, kb, pt, sid, nv) = _cand_direct(csa2, dev, kf, qf, K, T)
    rows = np.array([0, 1, 129, 257])
    _, s_ref = orc.index_topk(K, E // 64, qb, wv, kb, pt, sid, nv, rows=rows, want_scores=True)
    tl.check_topk(idx[rows], s_ref, K, nv, rows=rows)
    assert np.all(np.diff(idx, axis=1) > 0)


def test_topk_candidates_window_miss(csa2, dev):
    """Rows whose sampled maximum sits more than 32 octaves above the rest: 200 keys scaled
    by 2^36, so the threshold's first digit window holds fewer than its rank; the rows are
    flagged, take the exact path and match the oracle (the 200 and the best of the rest)."""
    _say("topk_candidates_window_miss")
    E, K, T = 16384, 512, 258
    rng = np.random.default_rng(31)
    kf = np.abs(synth.normal_f32(13, 1, 0, E * 64)).reshape(E, 64)
    kf[rng.choice(E, 200, replace=False)] *= np.float32(2.0 ** 36)
    qf = np.abs(synth.normal_f32(13, 2, 0, T * 64))
    idx, (qb, wv, kb, pt, sid, nv) = _cand_direct(csa2, dev, kf, qf, K, T)
    rows = np.array([0, 1, 128, 257])
    _, s_ref = orc.index_topk(K, E // 64, qb, wv, kb, pt, sid, nv, rows=rows, want_scores=True)
    tl.check_topk(idx[rows], s_ref, K, nv, rows=rows)
    assert np.all(np.diff(idx, axis=1) > 0)


def _swa_windows(T, L, seed):
    rng = np.random.default_rng(seed)
    ln = rng.choice([0, 1, 17, 64, 128, 200], T)
    st = np.array([rng.integers(0, L - l + 1) for l in ln])
    st[:T // 2] = np.minimum(np.arange(T // 2), L - ln[:T // 2])   # a sliding run, as in prefill
    return st.astype(np.int32), ln.astype(np.int32)


_SW = _swa_windows(300, 400, 13)


def test_layer_group_rowtiled_swa_and_scoring(csa2, dev):
    """From 256 rows on, SWA also runs row-tiled on MFMA: tiles that mix sequences, GQA (4
    query heads per KV head), empty, one-token and long windows, a partial last tile."""
    w = W(name="rowtiled_t300_b3_gqa4", B=3, T=300, E=1024, H=16, H_I=4, K=64, H_kv=4,
          L_swa=400, seq_id_rows=_gemm_rows(300, [120, 60, 120], 11),
          n_vis_rows=_gemm_nvis(300, 1024, 12), swa_start_rows=_SW[0], swa_len_rows=_SW[1])
    d, res, _ = _group_case(csa2, dev, w, np.arange(300), w.name)
    empty = w.swa_len() == 0
    assert np.all(res[0]["o_swa"][empty] == 0) and np.all(np.isneginf(res[0]["lse_swa"][empty]))


_SW2 = _swa_windows(200, 400, 17)


def test_layer_group_persistent_swa_ragged(csa2, dev):
    """Decode-shaped rows with H = H_kv: the SWA branch runs on 128 persistent workgroups
    (3200 (row, KV head) units over 2048 waves, so some waves take two units), with empty,
    one-token and long windows over three sequences; attention runs beside it on the CUs
    left."""
    w = W(name="persist_swa_t200_b3_h16", B=3, T=200, E=1024, H=16, H_I=4, K=64, H_kv=16,
          L_swa=400, seq_id_rows=(np.arange(200) % 3).astype(np.int32),
          n_vis_rows=_gemm_nvis(200, 1024, 18), swa_start_rows=_SW2[0],
          swa_len_rows=_SW2[1])
    d, res, _ = _group_case(csa2, dev, w, np.arange(200), w.name)
    empty = w.swa_len() == 0
    assert empty.any()
    assert np.all(res[0]["o_swa"][empty] == 0) and np.all(np.isneginf(res[0]["lse_swa"][empty]))


# Many rows longer than 65536 keys: the streamed Top-K.  Distinct scores take the path that
# gathers the keys at or above the top digit into LDS; all-equal scores overflow that list
# and take the streamed digit passes.
STREAMED = {
    "streamed_t66_65600_k512": W(B=2, T=66, E=65600, H=16, H_I=4, K=512, H_kv=16,
                                 n_vis_rows=np.r_[[65600, 65537, 300, 40000],
                                                  np.full(62, 65600)].astype(np.int32),
                                 seq_id_rows=(np.arange(66) % 2).astype(np.int32)),
}


@pytest.mark.parametrize("name", list(STREAMED))
def test_topk_streamed_parity(csa2, dev, name):
    _index_parity(csa2, dev, STREAMED[name], name)


def test_topk_streamed_all_equal_scores(csa2, dev):
    _say("topk_streamed_all_equal_scores")
    E, K, T = 65600, 300, 66
    key = torch.from_numpy(synth.normal_bf16(9, 1, 0, 64).view(np.int16)).to(dev)
    k_idx = key.view(1, 1, 64).expand(E // 64, 64, 64).contiguous().view(torch.bfloat16)
    q = torch.from_numpy(synth.normal_bf16(9, 2, 0, T * 64).view(np.int16)).to(dev).view(
        torch.bfloat16).view(T, 1, 64)
    wv = torch.ones((T, 1), dtype=torch.float32, device=dev)
    pt = torch.arange(E // 64, dtype=torch.int32, device=dev).view(1, -1)
    sid = torch.zeros(T, dtype=torch.int32, device=dev)
    nv = torch.full((T,), E, dtype=torch.int32, device=dev)
    idx = csa2.index_topk(q, wv, k_idx, pt, sid, nv, K).cpu().numpy()
    for r in range(T):
        np.testing.assert_array_equal(idx[r], np.arange(K))


@pytest.mark.parametrize("boost", ["sampled", "unsampled"])
def test_topk_streamed_sample_misses(csa2, dev, boost):
    """Rows whose sample misleads the streamed Top-K's threshold: the keys at the sampled
    16-entry segments (one in every ceil(E/16/256)) scaled x8, so the threshold keeps fewer
    than K keys, or every other key scaled x8, so it keeps more than the list holds.  Both
    must fall back to the exact passes and match the oracle."""
    _say("topk_streamed_sample_misses", boost)
    E, K, T = 65600, 512, 66
    nseg = E // 16
    gap = -(-nseg // 256)
    seg = np.zeros(E // 16, bool)
    seg[::gap] = True
    in_sample = np.repeat(seg, 16)
    kf = np.abs(synth.normal_f32(11, 1, 0, E * 64)).reshape(E, 64)
    kf[in_sample if boost == "sampled" else ~in_sample] *= 8.0
    kb = synth.f32_to_bf16_bits(kf)
    qb = synth.f32_to_bf16_bits(np.abs(synth.normal_f32(11, 2, 0, T * 64)).reshape(T, 1, 64))
    wv = np.ones((T, 1), np.float32)
    pt = np.arange(E // 64, dtype=np.int32)[None]
    sid = np.zeros(T, np.int32)
    nv = np.full(T, E, np.int32)
    t16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(
        torch.bfloat16)
    ti = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    idx = csa2.index_topk(t16(qb), ti(wv), t16(kb).view(E // 64, 64, 64), ti(pt), ti(sid),
                          ti(nv), K).cpu().numpy()
    rows = np.array([0, 1, 33, 65])
    _, s_ref = orc.index_topk(K, E // 64, qb, wv, kb, pt, sid, nv, rows=rows, want_scores=True)
    tl.check_topk(idx[rows], s_ref, K, nv, rows=rows)
    assert np.all(np.diff(idx, axis=1) > 0)


def test_topk_chunked_all_equal_scores(csa2, dev):
    """Equal scores over many chunks: the lowest K indices win, in order, also when the
    selection spans several chunks."""
    _say("topk_chunked_all_equal_scores")
    E, K = 70016, 9000
    key = torch.from_numpy(synth.normal_bf16(9, 1, 0, 64).view(np.int16)).to(dev)
    k_idx = key.view(1, 1, 64).expand(E // 64, 64, 64).contiguous().view(torch.bfloat16)
    q = torch.from_numpy(synth.normal_bf16(9, 2, 0, 3 * 64).view(np.int16)).to(dev).view(
        torch.bfloat16).view(3, 1, 64)
    wv = torch.ones((3, 1), dtype=torch.float32, device=dev)
    pt = torch.arange(E // 64, dtype=torch.int32, device=dev).view(1, -1)
    sid = torch.zeros(3, dtype=torch.int32, device=dev)
    nv = torch.tensor([E, 1000, K + 3], dtype=torch.int32, device=dev)
    idx = csa2.index_topk(q, wv, k_idx, pt, sid, nv, K).cpu().numpy()
    np.testing.assert_array_equal(idx[0], np.arange(K))
    np.testing.assert_array_equal(idx[1], np.r_[np.arange(1000), -np.ones(K - 1000, np.int32)])
    np.testing.assert_array_equal(idx[2], np.arange(K))


def test_empty_rows_and_windows(csa2, dev):
    _say("empty_rows_and_windows")
    w = W(B=2, T=3, E=512, K=64, H=16, H_I=2, H_kv=16, seq_id_rows=[0, 1, 0],
          n_vis_rows=[0, 512, 5], swa_start_rows=[0, 0, 0], swa_len_rows=[0, 128, 0])
    d = tl.DeviceWorkload(w, dev)
    res = d.run_layer_group()[0]
    assert np.all(res["idx"][0] == -1)
    np.testing.assert_array_equal(res["idx"][2], np.r_[np.arange(5), -np.ones(59, np.int32)])
    assert np.all(res["o"][0] == 0) and np.all(np.isneginf(res["lse"][0]))
    assert np.all(res["o_swa"][0] == 0) and np.all(np.isneginf(res["lse_swa"][0]))
    assert np.all(res["o_swa"][2] == 0) and np.all(np.isneginf(res["lse_swa"][2]))
    h = tl.HostWorkload(w)
    rows = np.arange(3)
    tl.check_topk(res["idx"], h.scores(0, rows), w.K, w.n_vis())
    tl.check_attn(res, h.attn_on(res["idx"], 0, rows))
    # T = 0 is a no-op
    L = d.layers[0]
    z = csa2.index_topk(L["q_idx"][:0], L["w_idx"][:0], L["k_idx"], d.page_table,
                        d.seq_id[:0], d.n_vis[:0], w.K)
    assert z.shape == (0, w.K)


def _group_case(csa2, dev, w, rows, name, fmt=0):
    _say("layer_group", name, "kv_format", fmt, "rows", len(rows))
    d = tl.DeviceWorkload(w, dev, fmt=fmt)
    res = d.run_layer_group()
    torch.cuda.synchronize()
    h = tl.HostWorkload(w, fmt=fmt)
    ref = h.run_layer_group(rows)
    _, idx_src = orc.resolve_sources(w.modes)
    nb = 0
    for li in range(len(w.modes)):
        if ref[li]["pooled"]:
            nb += _check_pooled_layer(res[li]["idx"], res[0]["idx"], ref[li], w, rows, h,
                                      idx_src[li])
        else:
            nb += tl.check_topk(res[li]["idx"], ref[li]["scores"], w.K, w.n_vis(), rows=rows)
        oref = h.attn_on(res[li]["idx"][rows], li, rows)
        tl.check_attn(res[li], oref, rows=rows)
    # Reuse borrows Reindex's indices; Reindex's differ from Full's (independent indexers)
    if w.modes == [0, 1, 2]:
        np.testing.assert_array_equal(res[2]["idx"], res[1]["idx"])
        assert not np.array_equal(res[1]["idx"], res[0]["idx"])
    return d, res, nb


def _check_pooled_layer(idxp, idx0, ref, w, rows, h, li):
    """Selection idxp of a pooled Reindex layer li (or of a Reuse layer borrowing it).  The
    oracle searched the pool of its own layer-0 selection ref["sel0"]; rows whose GPU
    layer-0 selection idx0 is the same set (all, unless a near-tie moved a boundary entry)
    are compared with that search.  For the other rows the oracle searches the pool of the
    GPU's own layer-0 selection, and the GPU's picks are held to the same rule: min(K, pool)
    picks, all in the pool, ascending, -1 padded, the pool's best up to the score
    tolerance."""
    same = np.array([np.array_equal(idx0[t], ref["sel0"][r]) for r, t in enumerate(rows)])
    assert same.mean() >= 0.75, "too few rows with the oracle's layer-0 selection"
    nb = tl.check_topk_pool(idxp[rows[same]], ref["scores"][same], w.K)
    if (~same).any():
        other = rows[~same]
        _, s_own = h.pool_search(li, other, idx0)
        nb += tl.check_topk_pool(idxp[other], s_own, w.K)
    return nb


def test_layer_group_full_reindex_reuse(csa2, dev):
    w = W(name="group_small", B=4, T=4, E=2048, K=256, H=64, H_I=8, H_kv=64, n_hot=20,
          modes=[0, 1, 2])
    _group_case(csa2, dev, w, np.arange(4), "group_small")


POOL = {
    # name: (workload, K_sel)
    "pool_small_k256": (W(B=2, T=4, E=2048, K=256, H_I=8), 256),
    "pool_ragged_take_all": (W(B=3, T=5, E=1536, K=100, H_I=3, seq_id_rows=[0, 1, 2, 1, 0],
                               n_vis_rows=[1536, 700, 33, 1100, 1]), 64),
    "pool_k_above_pool": (W(B=2, T=3, E=1024, K=300, H_I=4), 32),
    "pool_sel_not_mult8": (W(B=2, T=3, E=4096, K=512, H_I=8, n_vis_rows=[4096, 3001, 2047],
                             seq_id_rows=[0, 1, 0]), 300),
    "pool_sel_1": (W(B=1, T=2, E=512, K=16, H_I=2), 1),
    "pool_2048_on_32k": (W(B=8, T=8, E=32768, K=2048, H_I=8, n_hot=328), 2048),
}


def _pool_parity(csa2, dev, w, K_sel, name, rows=None, empty_row=None):
    _say("index_topk_pool", name)
    rows = np.arange(w.T) if rows is None else rows
    sel = w.selection(K_sel)
    if empty_row is not None:
        sel[empty_row] = -1
    w1 = synth.Workload(**{**w.__dict__, "modes": [0, 3]})
    d = tl.DeviceWorkload(w1, dev)
    L = d.layers[1]
    idx = csa2.index_topk_pool(L["q_idx"], L["w_idx"], L["k_idx"], d.page_table, d.seq_id,
                               d.n_vis, w.K, torch.from_numpy(sel).to(dev))
    torch.cuda.synchronize()
    h = tl.HostWorkload(w1)
    ref, scores = h.pool_search(1, rows, sel)
    idx = idx.cpu().numpy()
    tl.check_topk_pool(idx, scores, w.K, rows=rows)
    return idx, ref


@pytest.mark.parametrize("name", list(POOL))
def test_index_topk_pool_parity(csa2, dev, name):
    w, K_sel = POOL[name]
    _pool_parity(csa2, dev, w, K_sel, name, empty_row=(1 if name == "pool_small_k256" else None))


def test_full_size_pool_64x128k(csa2, dev):
    """Pooled search at the headline decode shape: 64 rows over 32768 entries, K = 2048,
    pools from 2048 selections (16384 key slots per row); the oracle checks every row."""
    w = synth.workload(2)
    idx, _ = _pool_parity(csa2, dev, w, 2048, "pool_" + w.name)
    assert np.all(idx >= 0)


def test_layer_group_pooled_reindex(csa2, dev):
    w = W(name="group_pool", B=4, T=4, E=4096, K=256, H=64, H_I=8, H_kv=64, n_hot=20,
          modes=[0, 3, 2])
    d, res, _ = _group_case(csa2, dev, w, np.arange(4), "group_pool")
    np.testing.assert_array_equal(res[2]["idx"], res[1]["idx"])


def test_index_ignores_keys_past_visible(csa2, dev):
    """The scoring reads whole pages (and, pooled, whole 8-entry blocks), visible or not:
    key rows past a sequence's visible count may hold anything, NaN and huge values
    included, and the selections do not change.  Visible counts end inside a page, inside
    an 8-entry block and at a page edge."""
    _say("index_ignores_keys_past_visible")
    w = W(name="tailpoison", B=3, T=3, E=1536, K=300, H_I=8, seq_id_rows=[0, 1, 2],
          n_vis_rows=[1003, 704, 33], shuffle=True, modes=[0, 3])
    d = tl.DeviceWorkload(w, dev)
    L = d.layers[1]
    sel = torch.from_numpy(w.selection(256)).to(dev)
    args = (L["q_idx"], L["w_idx"], L["k_idx"], d.page_table, d.seq_id, d.n_vis, w.K)

    def run():
        a = csa2.index_topk(*args)
        b = csa2.index_topk_pool(*args, sel)
        torch.cuda.synchronize()
        return a.cpu().numpy(), b.cpu().numpy()

    before = run()
    pt = w.page_table()
    kv = L["k_idx"].view(-1, 64).view(torch.int16)
    rng = np.random.default_rng(5)
    for b, nv in enumerate(w.n_vis()):
        rows = w.physical_rows(b, pt)[int(nv):]
        junk = rng.choice(np.array([0x7fc0, 0xffc0, 0x7f7f, 0xff7f, 0x7f80], np.uint16),
                          size=(rows.size, 64)).view(np.int16)
        kv[torch.from_numpy(rows).to(dev)] = torch.from_numpy(junk).to(dev)
    after = run()
    np.testing.assert_array_equal(after[0], before[0])
    np.testing.assert_array_equal(after[1], before[1])


def test_determinism(csa2, dev):
    _say("determinism")
    w = W(B=4, T=8, E=4096, K=1024, H=64, seq_id_rows=[0, 1, 2, 3, 3, 2, 1, 0])
    d = tl.DeviceWorkload(w, dev)
    a = d.run_layer_group()[0]
    b = d.run_layer_group()[0]
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


def test_side_stream_schedule_matches_sequential(csa2, dev):
    """The SWA branch on the side stream (persistent workgroups beside attention) and the
    same layer group run in sequence on one stream (kernel timing on) give bit-identical
    outputs: the branches share no buffer and the launch shapes are the same."""
    _say("side_stream_vs_sequential")
    w = W(name="sched_t96_b3", B=3, T=96, E=2048, K=512, H=64, H_I=8, H_kv=64,
          seq_id_rows=(np.arange(96) % 3).astype(np.int32), modes=[0, 1, 2])
    d = tl.DeviceWorkload(w, dev)
    a = d.run_layer_group()
    torch.cuda.synchronize()
    csa2.timing_enable(True)
    try:
        b = d.run_layer_group()
        torch.cuda.synchronize()
    finally:
        csa2.timing_enable(False)
        csa2.timing_read()
    for la, lb in zip(a, b):
        for k in la:
            np.testing.assert_array_equal(la[k], lb[k])


def test_layer_group_graph_capture(csa2, dev):
    """The layer group recorded in a HIP graph (through torch's capture): each replay, with
    the outputs cleared eagerly and the device synchronized in between, gives the eager
    call's bits, SWA branch (side stream, forked and joined by events) included."""
    _say("layer_group_graph_capture")
    w = W(name="graph_t16_b2", B=2, T=16, E=2048, K=256, H=64, H_I=8, H_kv=64,
          seq_id_rows=(np.arange(16) % 2).astype(np.int32), modes=[0, 1, 2])
    d = tl.DeviceWorkload(w, dev)
    ref = d.run_layer_group()
    torch.cuda.synchronize()
    descs, g = d.descs(), d.group_args()
    need = csa2.workspace_bytes(csa2.OP_LAYER_GROUP, g)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                      # warm-up on the capture stream
        csa2.layer_group(descs, g, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        csa2.layer_group(descs, g, workspace=ws)
    outs = [k for k in ("o", "lse", "o_swa", "lse_swa")]
    for rep in range(3):
        for L in d.layers:
            for k in outs:
                L[k].zero_()
            if "idx_out" in L:
                L["idx_out"].fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _, idx_src = tl.orc.resolve_sources(w.modes)
        for li, L in enumerate(d.layers):
            np.testing.assert_array_equal(d.layers[idx_src[li]]["idx_out"].cpu().numpy(),
                                          ref[li]["idx"], err_msg=f"replay {rep} layer {li}")
            for k in outs:
                np.testing.assert_array_equal(L[k].cpu().numpy(), ref[li][k],
                                              err_msg=f"replay {rep} layer {li} {k}")


# ---------------------------------------------------------------- full sizes
def test_full_size_decode_64x128k(csa2, dev):
    """The headline decode workload (64 rows, 32768 entries each, K=2048, H=64) in the same
    launch configuration the benchmark times; the oracle checks every row."""
    w = synth.workload(2)
    rows = np.arange(w.T)
    d, res, _ = _group_case(csa2, dev, w, rows, w.name)
    idx = res[0]["idx"]
    assert np.all(np.diff(idx, axis=1) > 0) and idx.min() >= 0 and idx.max() < w.E


def test_full_size_decode_64x128k_e4m3(csa2, dev):
    """The headline decode with the main KV in the E4M3-per-16 format, every row."""
    w = synth.workload(2)
    _group_case(csa2, dev, w, np.arange(w.T), w.name + "_e4m3", fmt=1)


def test_layer_group_e4m3_group_small(csa2, dev):
    w = W(name="group_small_e4m3", B=4, T=4, E=2048, K=256, H=64, H_I=8, H_kv=64, n_hot=20,
          modes=[0, 1, 2])
    _group_case(csa2, dev, w, np.arange(4), "group_small_e4m3", fmt=1)


def test_layer_group_swa_in_scoring_launch(csa2, dev):
    """A small SWA branch (at most a quarter of the scoring's bytes) runs inside the per-row
    scoring's launch: the Full and Reindex layers' branches that way, the Reuse layer's on
    the side stream; ragged windows, an empty window, ragged visible counts."""
    w = W(name="swa_fused", B=3, T=4, E=8192, K=256, H=16, H_I=8, H_kv=16, L_swa=32,
          seq_id_rows=[0, 1, 2, 1], n_vis_rows=[8192, 5000, 777, 6001],
          swa_start_rows=[0, 3, 31, 10], swa_len_rows=[32, 29, 1, 0], modes=[0, 1, 2])
    _group_case(csa2, dev, w, np.arange(4), "swa_fused")


def test_full_size_decode_4x1m(csa2, dev):
    w = synth.workload(4)
    _group_case(csa2, dev, w, np.arange(4), w.name)


def test_full_size_group_32x256k(csa2, dev):
    w = synth.workload(3)
    _group_case(csa2, dev, w, np.arange(w.T), w.name)


def test_full_size_group_pooled_32x256k(csa2, dev):
    """The 32 x 256K group with its Reindex layer searching the Full layer's pool, every
    row."""
    w = synth.workload(3)
    w = synth.Workload(**{**w.__dict__, "name": w.name + "_pool", "modes": [0, 3, 2]})
    _group_case(csa2, dev, w, np.arange(w.T), w.name)


def test_full_size_prefill_4096_sampled(csa2, dev):
    w = synth.workload(5)
    rows = np.unique(np.r_[[0, 1, 2, 3, 4095], np.arange(0, 4096, 64)])
    _group_case(csa2, dev, w, rows, w.name)
