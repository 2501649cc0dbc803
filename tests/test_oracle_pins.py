"""Pins of the CPU oracle against facts fixed outside it: the format definitions, closed
forms, brute force on tiny inputs, textbook special cases and invariants.

Sources: [summary] = picx.dev whiteboard summary of "DeepSeek-V4.1-Flash: Pushing the Limits
of KV Cache Compression"; OCP MX v1.0 = the Microscaling Formats specification that
[summary] Methodology > Architecture Components > 5 names for the FP4 main KV cache.
"""
import os

import numpy as np
import pytest
import torch

import synth
from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(v) for v in line.split()])
    return np.array(rows)


def _bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def _f(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


# ---------------------------------------------------------------- MXFP4 codec
def test_e2m1_table():
    g = _golden("e2m1_codes.txt")
    for code, val in g:
        got = orc.e2m1_decode(int(code))
        assert got == val and np.signbit(got) == np.signbit(val), (code, got, val)


def test_e8m0_decode():
    assert orc.e8m0_decode(127) == 1.0
    assert orc.e8m0_decode(130) == 8.0
    assert orc.e8m0_decode(0) == 2.0 ** -127


def _block_with(values):
    x = np.zeros(512, np.float32)
    x[: len(values)] = values
    return x


def _codes(lat):
    lat = lat.reshape(-1)
    c = np.empty(lat.size * 2, np.int64)
    c[0::2] = lat & 15
    c[1::2] = lat >> 4
    return c


def test_mxfp4_tie_table():
    g = _golden("mxfp4_ties.txt")
    for inp, want in g:
        x = _block_with([inp, 4.0])              # block max in [4, 8): shared exponent 0
        lat, scl = orc.mxfp4_quantize(x[None])
        assert scl[0, 0] == 127
        got = orc.mxfp4_dequantize(lat, scl)[0, 0]
        assert got == want and np.signbit(got) == np.signbit(want), (inp, got, want)


def _brute_codes(x, scale_byte):
    """Nearest E2M1 value by exhaustive search over the 8 magnitudes; a tie goes to the
    even code; the sign is the sign of x."""
    e = int(scale_byte) - 127
    y = np.abs(x.astype(np.float64)) * 2.0 ** (-e)
    d = np.abs(y[:, None] - E2M1_MAGS[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    codes = np.empty(x.size, np.int64)
    for i in range(x.size):
        ks = np.nonzero(cand[i])[0]
        ks_even = [k for k in ks if k % 2 == 0]
        codes[i] = ks_even[0] if ks_even else ks[0]
    return codes | (np.signbit(x).astype(np.int64) << 3)


def _random_blocks(n_rows, seed):
    rng = np.random.default_rng(seed)
    x = synth.normal_f32(seed, 77, 0, n_rows * 512).reshape(n_rows, 512)
    # per-block magnitudes spanning many binades, plus planted grid points and ties
    mult = 2.0 ** rng.integers(-20, 20, size=(n_rows, 16)).astype(np.float32)
    x = (x.reshape(n_rows, 16, 32) * mult[:, :, None]).reshape(n_rows, 512)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0], np.float32)
    for r in range(n_rows):
        blk = rng.integers(0, 16)
        sc = np.float32(2.0 ** rng.integers(-5, 5))
        x[r, blk * 32: blk * 32 + 9] = ties * sc * rng.choice([-1, 1], 9)
        x[r, blk * 32 + 9] = 7.5 * sc           # block max in [4, 8) * sc
    x[0, :32] = 0.0                                # an all-zero block
    x[0, 1] = -0.0
    return x.astype(np.float32)


def test_quantizer_matches_brute_force():
    x = _random_blocks(64, 5)
    lat, scl = orc.mxfp4_quantize(x)
    codes = _codes(lat).reshape(64, 512)
    for r in range(64):
        for b in range(16):
            blk = x[r, b * 32:(b + 1) * 32]
            amax = np.abs(blk.astype(np.float64)).max()
            e = int(scl[r, b]) - 127
            if amax == 0:
                assert e == -127
            else:
                # defining property of the shared exponent floor(log2 amax) - 2
                assert 4.0 * 2.0 ** e <= amax < 8.0 * 2.0 ** e
            np.testing.assert_array_equal(codes[r, b * 32:(b + 1) * 32], _brute_codes(blk, scl[r, b]))


def test_zero_block_keeps_sign():
    x = _block_with([0.0, -0.0, 0.0])
    lat, scl = orc.mxfp4_quantize(x[None])
    assert scl[0, 0] == 0
    c = _codes(lat)
    assert c[0] == 0 and c[1] == 8


def test_sign_symmetry():
    x = _random_blocks(8, 6)
    la, sa = orc.mxfp4_quantize(x)
    lb, sb = orc.mxfp4_quantize(-x)
    np.testing.assert_array_equal(sa, sb)
    np.testing.assert_array_equal(_codes(la) ^ 8, _codes(lb))


def test_roundtrip_idempotent():
    x = _random_blocks(16, 7)
    lat, scl = orc.mxfp4_quantize(x)
    v = orc.mxfp4_dequantize(lat, scl)
    lat2, scl2 = orc.mxfp4_quantize(v.astype(np.float32))
    np.testing.assert_array_equal(orc.mxfp4_dequantize(lat2, scl2), v)


def test_error_bound():
    x = _random_blocks(32, 8).astype(np.float64)
    lat, scl = orc.mxfp4_quantize(x.astype(np.float32))
    v = orc.mxfp4_dequantize(lat, scl)
    e = np.repeat(scl.astype(np.float64) - 127, 32, axis=1)
    y = np.abs(x) * 2.0 ** (-e)
    half_step = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
    bound = np.where(y <= 6, half_step, 2.0) * 2.0 ** e
    assert np.all(np.abs(x - v) <= bound)


def test_page_magnitude_bound_never_clips():
    # [summary] Architecture Components > 5: KV magnitudes stay below sqrt(512) ~ 22.6.
    x = np.zeros((4, 512), np.float32)
    x[:, :32] = np.linspace(-22.6, 22.6, 32, dtype=np.float32)
    x[1, :32] *= 0.75
    lat, scl = orc.mxfp4_quantize(x)
    assert scl[:, 0].max() <= 127 + 2
    v = orc.mxfp4_dequantize(lat, scl)
    y = np.abs(x[:, :32].astype(np.float64)) / 2.0 ** (scl[:, :1].astype(np.float64) - 127)
    assert np.all(y <= 6.0)                        # inside the element range: no saturation
    assert np.all(np.abs(v[:, :32] - x[:, :32]) <= 1.0 * 2.0 ** 2)


def test_nonfinite_rejected():
    x = _block_with([1.0, np.nan])
    with pytest.raises(ValueError):
        orc.mxfp4_quantize(x[None])
    x = _block_with([np.inf])
    with pytest.raises(ValueError):
        orc.mxfp4_quantize(x[None])


# ---------------------------------------------------------------- indexer + Top-K
def _tiny_index_inputs(E=256, H_I=1, seed=3, positive=True):
    q = synth.normal_f32(seed, 1, 0, H_I * 64).reshape(1, H_I, 64)
    k = synth.normal_f32(seed, 2, 0, E * 64).reshape(E, 64)
    if positive:
        q, k = np.abs(q), np.abs(k)
    return _bf16(q), _bf16(k)


def _identity_paging(E):
    P = E // 64
    return np.arange(P, dtype=np.int32)[None, :], np.zeros(1, np.int32), np.array([E], np.int32)


def test_index_single_head_is_plain_dot():
    # H_I = 1, w = 1 and all dots positive: the score is the plain dot product (GEMV).
    E = 256
    qb, kb = _tiny_index_inputs(E)
    pt, sid, nv = _identity_paging(E)
    _, s = orc.index_topk(16, E // 64, qb, np.ones((1, 1), np.float32), kb, pt, sid, nv,
                          want_scores=True)
    ref = _f(kb) @ _f(qb)[0, 0]
    np.testing.assert_allclose(s[0], ref, rtol=1e-13)


def test_index_relu_gates_negative_dots():
    # Two heads with q_2 = -q_1 and unit weights: exactly one head passes the ReLU,
    # so the score is |q_1 . k|.
    E = 128
    qb, kb = _tiny_index_inputs(E, positive=False)
    q2 = np.concatenate([qb, qb ^ np.uint16(0x8000)], axis=1)
    pt, sid, nv = _identity_paging(E)
    _, s = orc.index_topk(8, E // 64, q2, np.ones((1, 2), np.float32), kb, pt, sid, nv,
                          want_scores=True)
    np.testing.assert_allclose(s[0], np.abs(_f(kb) @ _f(qb)[0, 0]), rtol=1e-13)
    # weights scale each head's contribution: w = (2, 0) keeps 2*max(0, d)
    _, s2 = orc.index_topk(8, E // 64, q2, np.array([[2.0, 0.0]], np.float32), kb, pt, sid,
                           nv, want_scores=True)
    np.testing.assert_allclose(s2[0], 2 * np.maximum(0, _f(kb) @ _f(qb)[0, 0]), rtol=1e-13)


def _lexsort_topk(s, K):
    order = np.lexsort((np.arange(s.size), -s))[:K]
    out = np.full(K, -1, np.int32)
    out[: min(K, s.size)] = np.sort(order)
    return out


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(11)
    for n, K in [(1000, 64), (333, 333), (50, 64), (4096, 2048), (1, 1), (0, 8)]:
        s = rng.integers(-5, 6, n).astype(np.float64)    # heavy ties
        np.testing.assert_array_equal(orc.topk_from_scores(s, K), _lexsort_topk(s, K))


def test_topk_all_equal_and_short_rows():
    np.testing.assert_array_equal(orc.topk_from_scores(np.full(100, 3.0), 10), np.arange(10))
    got = orc.topk_from_scores(np.arange(5.0), 8)
    np.testing.assert_array_equal(got, [0, 1, 2, 3, 4, -1, -1, -1])


def test_topk_signed_zero_ties():
    s = np.array([-0.0, 0.0, -0.0, -1.0, 0.0])
    np.testing.assert_array_equal(orc.topk_from_scores(s, 2), [0, 1])


def _small_workload(**kw):
    base = dict(name="t", B=2, T=2, E=512, H=16, H_I=4, K=64, H_kv=16, L_swa=128, seed=31,
                hot="uniform", n_hot=8, shuffle=True)
    base.update(kw)
    return synth.Workload(**base)


def _planes(w, pt=None):
    pt = w.page_table() if pt is None else pt
    lat_l, scl_l = [], []
    for b in range(w.B):
        l, s = orc.mxfp4_quantize(w.latent_seq(b))
        lat_l.append(l)
        scl_l.append(s)
    lat = w.to_physical(lambda b: lat_l[b], pt)
    scl = w.to_physical(lambda b: scl_l[b], pt)
    rope = w.to_physical(w.rope_seq, pt)
    kidx = w.to_physical(w.k_idx_seq, pt)
    return lat, scl, rope, kidx


def test_topk_invariant_to_positive_query_scale():
    w = _small_workload()
    pt = w.page_table()
    _, _, _, kidx = _planes(w, pt)
    q = w.q_idx()
    a = orc.index_topk(w.K, w.P, q, w.w_idx(), kidx, pt, w.seq_id(), w.n_vis())
    q2 = _bf16(_f(q) * 2.0)                       # exact doubling in bf16
    b = orc.index_topk(w.K, w.P, q2, w.w_idx(), kidx, pt, w.seq_id(), w.n_vis())
    np.testing.assert_array_equal(a, b)


def test_hot_entries_rank_first():
    # keys x4 on the hot entries: with positive weights they take the top of the ranking
    w = _small_workload(n_hot=8, K=8, H_I=8)
    pt = w.page_table()
    _, _, _, kidx = _planes(w, pt)
    idx = orc.index_topk(w.K, w.P, w.q_idx(), w.w_idx(), kidx, pt, w.seq_id(), w.n_vis())
    for t in range(w.T):
        hot = set(w.hot_entries(w.seq_id()[t]).tolist())
        assert len(hot & set(idx[t].tolist())) >= 6


def test_page_shuffle_invariance():
    w = _small_workload()
    pt1 = w.page_table()
    pt2 = np.arange(w.n_pages, dtype=np.int32).reshape(w.B, w.P)
    out = []
    for pt in (pt1, pt2):
        lat, scl, rope, kidx = _planes(w, pt)
        idx = orc.index_topk(w.K, w.P, w.q_idx(), w.w_idx(), kidx, pt, w.seq_id(), w.n_vis())
        o, lse = orc.sparse_attn(w.P, w.q(), lat, scl, rope, pt, w.seq_id(), idx)
        out.append((idx, o, lse))
    np.testing.assert_array_equal(out[0][0], out[1][0])
    np.testing.assert_array_equal(out[0][1], out[1][1])
    np.testing.assert_array_equal(out[0][2], out[1][2])


# ---------------------------------------------------------------- attention
def _dense_reference(q_bits, V, R, sm):
    """Softmax attention by torch's scaled_dot_product_attention (float64, CPU) over the
    given keys [n, 576] = [V ; R] and values V."""
    q = torch.from_numpy(_f(q_bits))[None]                          # [1, H, 576]
    k = torch.from_numpy(np.concatenate([V, R], axis=1))[None, None]  # [1, 1, n, 576]
    v = torch.from_numpy(V)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        q.transpose(0, 1)[None], k, v, scale=sm)                    # [1, H, 1, 512]
    logits = (q[0].double() @ k[0, 0].T) * sm
    lse = torch.logsumexp(logits, dim=-1)
    return o[0, :, 0].numpy(), lse.numpy()


def test_attention_dense_when_k_covers_all_visible():
    w = _small_workload(B=1, T=1, E=192, K=256, shuffle=True)
    pt = w.page_table()
    lat, scl, rope, _ = _planes(w, pt)
    idx = np.concatenate([np.arange(192), -np.ones(64)]).astype(np.int32)[None]
    o, lse = orc.sparse_attn(w.P, w.q(), lat, scl, rope, pt, w.seq_id(), idx)
    l, s = orc.mxfp4_quantize(w.latent_seq(0))
    V = orc.mxfp4_dequantize(l, s)
    R = _f(w.rope_seq(0))
    ro, rl = _dense_reference(w.q()[0], V, R, 1 / 24.0)
    np.testing.assert_allclose(o[0], ro, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse[0], rl, rtol=1e-12)


def test_attention_zero_query_is_mean():
    w = _small_workload(B=1, T=1, E=256, K=32)
    pt = w.page_table()
    lat, scl, rope, _ = _planes(w, pt)
    idx = np.arange(0, 256, 8, dtype=np.int32)[None]
    q = np.zeros((1, 16, 576), np.uint16)
    o, lse = orc.sparse_attn(w.P, q, lat, scl, rope, pt, w.seq_id(), idx)
    l, s = orc.mxfp4_quantize(w.latent_seq(0))
    V = orc.mxfp4_dequantize(l, s)[idx[0]]
    np.testing.assert_allclose(o[0], np.broadcast_to(V.mean(0), (16, 512)), rtol=1e-12,
                               atol=1e-14)
    np.testing.assert_allclose(lse[0], np.log(32.0), rtol=1e-14)


def test_attention_single_entry_and_empty():
    w = _small_workload(B=1, T=1, E=128, K=4)
    pt = w.page_table()
    lat, scl, rope, _ = _planes(w, pt)
    idx = np.array([[-1, 77, -1, -1]], np.int32)
    o, lse = orc.sparse_attn(w.P, w.q(), lat, scl, rope, pt, w.seq_id(), idx)
    l, s = orc.mxfp4_quantize(w.latent_seq(0))
    v = orc.mxfp4_dequantize(l, s)[77]
    np.testing.assert_array_equal(o[0], np.broadcast_to(v, (16, 512)))
    key = np.concatenate([v, _f(w.rope_seq(0))[77]])
    np.testing.assert_allclose(lse[0], (_f(w.q()[0]) @ key) / 24.0, rtol=1e-12)
    o, lse = orc.sparse_attn(w.P, w.q(), lat, scl, rope, pt, w.seq_id(),
                             -np.ones((1, 4), np.int32))
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_attention_permutation_invariance_and_split_merge():
    w = _small_workload(B=1, T=1, E=512, K=128)
    pt = w.page_table()
    lat, scl, rope, _ = _planes(w, pt)
    rng = np.random.default_rng(2)
    sel = np.sort(rng.choice(512, 128, replace=False)).astype(np.int32)
    o, lse = orc.sparse_attn(w.P, w.q(), lat, scl, rope, pt, w.seq_id(), sel[None])
    o2, lse2 = orc.sparse_attn(w.P, w.q(), lat, scl, rope, pt, w.seq_id(),
                               rng.permutation(sel)[None])
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-14)
    # log-sum-exp merge of two halves reproduces the whole
    oa, la = orc.sparse_attn(w.P, w.q(), lat, scl, rope, pt, w.seq_id(), sel[None, :64])
    ob, lb = orc.sparse_attn(w.P, w.q(), lat, scl, rope, pt, w.seq_id(), sel[None, 64:])
    m = np.logaddexp(la, lb)
    om = np.exp(la - m)[..., None] * oa + np.exp(lb - m)[..., None] * ob
    np.testing.assert_allclose(m, lse, rtol=1e-13)
    np.testing.assert_allclose(om, o, rtol=1e-10, atol=1e-13)


# ---------------------------------------------------------------- SWA
def test_swa_matches_sdpa_with_gqa():
    w = _small_workload(B=2, T=3, H=8, H_kv=2, L_swa=40)
    q = w.q_swa()
    k, v = w.swa_k(), w.swa_v()
    sid = np.array([1, 0, 1], np.int32)
    st = np.array([0, 5, 30], np.int32)
    ln = np.array([40, 17, 1], np.int32)
    o, lse = orc.swa_attn(q, k, v, sid, st, ln)
    for t in range(3):
        b = sid[t]
        K_ = torch.from_numpy(_f(k[b, st[t]:st[t] + ln[t]])).permute(1, 0, 2)  # [H_kv, n, 128]
        V_ = torch.from_numpy(_f(v[b, st[t]:st[t] + ln[t]])).permute(1, 0, 2)
        K_ = K_.repeat_interleave(4, dim=0)
        V_ = V_.repeat_interleave(4, dim=0)
        Q_ = torch.from_numpy(_f(q[t]))[:, None]                              # [H, 1, 128]
        ref = torch.nn.functional.scaled_dot_product_attention(Q_, K_, V_)
        np.testing.assert_allclose(o[t], ref[:, 0].numpy(), rtol=1e-10, atol=1e-12)
        ref_lse = torch.logsumexp((Q_ @ K_.transpose(1, 2))[:, 0] / np.sqrt(128), dim=-1)
        np.testing.assert_allclose(lse[t], ref_lse.numpy(), rtol=1e-12)
    # window of one token returns that token's value
    np.testing.assert_array_equal(o[2], np.repeat(_f(v[1, 30]), 4, axis=0))


def test_swa_zero_query_is_window_mean():
    w = _small_workload(B=1, T=1, H=4, H_kv=4, L_swa=128)
    v = w.swa_v()
    o, lse = orc.swa_attn(np.zeros((1, 4, 128), np.uint16), w.swa_k(), v, [0], [0], [128])
    np.testing.assert_allclose(o[0], _f(v[0]).mean(0), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[0], np.log(128.0), rtol=1e-14)


# ---------------------------------------------------------------- layer group
def _group_layers(w, pt, modes, same_q=False, same_indexer=False):
    lat, scl, rope, _ = _planes(w, pt)
    layers = []
    for i, m in enumerate(modes):
        li = 0 if same_q else i
        L = {"mode": m, "q": w.q(li), "q_swa": w.q_swa(li), "swa_k": w.swa_k(i),
             "swa_v": w.swa_v(i)}
        if m in (orc.FULL, orc.REINDEX, orc.REINDEX_POOL):
            lj = 0 if same_indexer else i
            L.update(q_idx=w.q_idx(lj), w_idx=w.w_idx(lj),
                     k_idx=w.to_physical(lambda b: w.k_idx_seq(b, lj), pt))
        if m == orc.FULL:
            L.update(kv_lat=lat, kv_scl=scl, kv_rope=rope)
        layers.append(L)
    return layers


def test_layer_group_resolution():
    assert orc.resolve_sources([0, 1, 2]) == ([0, 0, 0], [0, 1, 1])
    assert orc.resolve_sources([0, 2, 1, 2, 0, 2]) == ([0, 0, 0, 0, 4, 4], [0, 0, 2, 2, 4, 4])
    with pytest.raises(ValueError):
        orc.resolve_sources([1, 2])


def test_layer_group_reuse_and_reindex_invariants():
    w = _small_workload()
    pt = w.page_table()
    args = (w.K, w.P, pt, w.seq_id(), w.n_vis(), w.swa_start(), w.swa_len())
    # identical indexer inputs: Reindex reproduces Full's indices; identical queries and
    # SWA caches would make every layer's outputs identical
    layers = _group_layers(w, pt, [orc.FULL, orc.REINDEX, orc.REUSE], same_q=True,
                           same_indexer=True)
    for L in layers:
        L["swa_k"], L["swa_v"] = layers[0]["swa_k"], layers[0]["swa_v"]
    res = orc.layer_group(layers, *args)
    for r in res[1:]:
        for key in ("idx", "o", "lse", "o_swa", "lse_swa"):
            np.testing.assert_array_equal(r[key], res[0][key])
    # distinct indexers: Reuse borrows Reindex's indices and Full's KV
    layers = _group_layers(w, pt, [orc.FULL, orc.REINDEX, orc.REUSE])
    res = orc.layer_group(layers, *args)
    assert not np.array_equal(res[1]["idx"], res[0]["idx"])
    np.testing.assert_array_equal(res[2]["idx"], res[1]["idx"])
    o, lse = orc.sparse_attn(w.P, layers[2]["q"], layers[0]["kv_lat"], layers[0]["kv_scl"],
                             layers[0]["kv_rope"], pt, w.seq_id(), res[1]["idx"])
    np.testing.assert_array_equal(res[2]["o"], o)


# ---------------------------------------------------------------- hierarchical pool
def _pool_golden():
    cases = []
    with open(os.path.join(GOLDEN, "pool_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            nv, sel, pool = (part.split() for part in line.split("|"))
            cases.append((int(nv[0]), np.array([int(v) for v in sel], np.int32),
                          np.array([int(v) for v in pool], np.int32)))
    return cases


def test_pool_blocks_golden():
    cases = _pool_golden()
    assert len(cases) == 7
    for nv, sel, pool in cases:
        np.testing.assert_array_equal(orc.pool_positions(sel, nv), pool)


def test_pool_size_bound_at_the_pages_sizes():
    # 2,048 selected entries -> at most 2,048 blocks x 8 = 16,384 positions; exactly that
    # when every selected entry lies in its own block
    n_vis, K_sel = 131072, 2048
    spread = (64 * np.arange(K_sel) + np.arange(K_sel) % 8).astype(np.int32)
    assert orc.pool_positions(spread, n_vis).size == 16384
    rng = np.random.default_rng(5)
    for _ in range(3):
        sel = np.sort(rng.choice(n_vis, K_sel, replace=False)).astype(np.int32)
        pool = orc.pool_positions(sel, n_vis)
        assert pool.size <= 16384 and pool.size % 8 == 0
        assert np.all(np.diff(pool) > 0) and np.all(np.isin(sel, pool))


def _pool_case(seed=41, K=64, E=512):
    w = _small_workload(K=K, E=E, seed=seed)
    pt = w.page_table()
    _, _, _, kidx = _planes(w, pt)
    return w, pt, kidx


def test_pool_topk_brute_force():
    # selection restricted to the pool: the K best pool positions by (score desc, position
    # asc), ascending, -1 padded; including a pool smaller than K
    w, pt, kidx = _pool_case()
    _, s = orc.index_topk(w.K, w.P, w.q_idx(), w.w_idx(), kidx, pt, w.seq_id(), w.n_vis(),
                          want_scores=True)
    rng = np.random.default_rng(9)
    nv = w.n_vis()
    for K_sel in (32, 3):
        sel = np.full((w.T, K_sel), -1, np.int32)
        for t in range(w.T):
            m = min(K_sel, int(nv[t]))
            sel[t, :m] = np.sort(rng.choice(int(nv[t]), m, replace=False))
        got = orc.index_topk_pool(w.K, w.P, w.q_idx(), w.w_idx(), kidx, pt, w.seq_id(), nv,
                                  sel)
        for t in range(w.T):
            pool = np.array(sorted({8 * (j // 8) + o for j in sel[t] if j >= 0
                                    for o in range(8) if 8 * (j // 8) + o < nv[t]}))
            ref = np.full(w.K, -1, np.int32)
            pick = pool[_lexsort_topk(s[t, pool], w.K)[: min(w.K, pool.size)]]
            ref[: pick.size] = np.sort(pick)
            np.testing.assert_array_equal(got[t], ref)


def test_pool_covering_everything_equals_full_search():
    w, pt, kidx = _pool_case()
    nv = w.n_vis()
    n_blocks = (int(nv.max()) + 7) // 8
    sel = np.tile(8 * np.arange(n_blocks, dtype=np.int32), (w.T, 1))
    sel[sel >= nv[:, None]] = -1
    sel = np.sort(np.where(sel < 0, np.iinfo(np.int32).max, sel), axis=1)
    sel[sel == np.iinfo(np.int32).max] = -1
    a = orc.index_topk(w.K, w.P, w.q_idx(), w.w_idx(), kidx, pt, w.seq_id(), nv)
    b = orc.index_topk_pool(w.K, w.P, w.q_idx(), w.w_idx(), kidx, pt, w.seq_id(), nv, sel)
    np.testing.assert_array_equal(a, b)


def test_layer_group_pooled_reindex():
    w = _small_workload()
    pt = w.page_table()
    args = (w.K, w.P, pt, w.seq_id(), w.n_vis(), w.swa_start(), w.swa_len())
    # the same indexer as the Full layer: the Full selection lies inside its own pool, so
    # the pooled search finds it again
    layers = _group_layers(w, pt, [orc.FULL, orc.REINDEX_POOL, orc.REUSE], same_indexer=True)
    res = orc.layer_group(layers, *args)
    np.testing.assert_array_equal(res[1]["idx"], res[0]["idx"])
    # its own indexer: every pick lies in the pool of the Full selection; Reuse borrows it
    layers = _group_layers(w, pt, [orc.FULL, orc.REINDEX_POOL, orc.REUSE])
    res = orc.layer_group(layers, *args)
    assert not np.array_equal(res[1]["idx"], res[0]["idx"])
    np.testing.assert_array_equal(res[2]["idx"], res[1]["idx"])
    for t in range(w.T):
        pool = orc.pool_positions(res[0]["idx"][t], w.n_vis()[t])
        picks = res[1]["idx"][t]
        assert np.all(np.isin(picks[picks >= 0], pool))


# ---------------------------------------------------------------- FP4 with E4M3 scales / 16
def test_e4m3_golden_and_all_bytes():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e4m3_codes.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) == 11
    for b, v in rows:
        got = orc.e4m3_decode(int(b, 16))
        assert got == float(v) and np.signbit(got) == np.signbit(float(v)), b
    assert np.isnan(orc.e4m3_decode(0x7f)) and np.isnan(orc.e4m3_decode(0xff))
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for b in range(256):
        got = orc.e4m3_decode(b)
        assert (np.isnan(got) and np.isnan(ref[b])) or got == ref[b], hex(b)


def test_e4m3_round_nearest_even_and_saturating():
    grid = np.array([orc.e4m3_decode(b) for b in range(0x7f)])          # 0 .. 448, ascending
    mids = (grid[1:] + grid[:-1]) / 2
    # every midpoint goes to the neighbour with the even mantissa (even byte)
    for k, m in enumerate(mids):
        assert orc.e4m3_round(m) == (k if k % 2 == 0 else k + 1), m
    rng = np.random.default_rng(4)
    v = np.abs(rng.standard_normal(4000)) * 10.0 ** rng.integers(-4, 3, 4000)
    for x in v:
        b = orc.e4m3_round(x)
        if x >= 448:
            assert b == 0x7e
        else:
            assert abs(grid[b] - x) <= np.abs(grid - x).min()
    assert orc.e4m3_round(1e9) == 0x7e and orc.e4m3_round(0.0) == 0


def _e2m1_nearest(y):
    """Brute force: nearest E2M1 magnitude code to y >= 0, ties to the even code."""
    mags = np.array([orc.e2m1_decode(c) for c in range(8)])
    d = np.abs(mags - min(y, 6.0))
    best = np.flatnonzero(d == d.min())
    return int(best[0] if best.size == 1 else best[best % 2 == 0][0])


def test_fp4e4m3_quantizer_brute_force():
    rng = np.random.default_rng(8)
    rows = 6
    x = rng.standard_normal((rows, 512)).astype(np.float32)
    x *= (2.0 ** rng.integers(-12, 6, (rows, 32, 1))).repeat(16, -1).reshape(rows, 512)
    x[0, :16] = 0.0
    x[1, 16:32] = np.float32(1e-6) * rng.standard_normal(16)   # scale rounds to 0
    x[2, 32:48] = [6.0, 0.75, 0.25, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, -0.75, 0, 0, 0, 0, 0, 0]
    lat, scl = orc.fp4e4m3_quantize(x)
    for r in range(rows):
        for b in range(32):
            blk = x[r, 16 * b: 16 * b + 16].astype(np.float64)
            sb = orc.e4m3_round(np.abs(blk).max() / 6.0)
            assert scl[r, b] == sb
            sv = orc.e4m3_decode(sb)
            for i in range(16):
                byte = lat[r, 8 * b + i // 2]
                code = (byte >> 4) if i % 2 else (byte & 15)
                mag = _e2m1_nearest(abs(blk[i]) / sv) if sv > 0 else 0
                assert code == (mag | (8 if np.signbit(blk[i]) else 0)), (r, b, i)


def test_fp4e4m3_range_and_error_bound():
    # the format's largest magnitude is 6 x 448 = 2688, the range the page gives
    top = np.zeros((1, 512), np.float32)
    top[0, 0] = 2688.0
    top[0, 1] = -2688.0
    lat, scl = orc.fp4e4m3_quantize(top)
    assert scl[0, 0] == 0x7e
    np.testing.assert_array_equal(orc.fp4e4m3_dequantize(lat, scl)[0, :2], [2688.0, -2688.0])
    # |x| <= sqrt(512) never reaches the scale's saturation; the error stays within half a
    # grid step at the block's scale, plus the clipping above 6 s
    rng = np.random.default_rng(9)
    x = np.clip(rng.standard_normal((64, 512)) * 8, -22.6, 22.6).astype(np.float32)
    lat, scl = orc.fp4e4m3_quantize(x)
    assert scl.max() < 0x7e
    v = orc.fp4e4m3_dequantize(lat, scl)
    s = np.array([[orc.e4m3_decode(b) for b in row] for row in scl]).repeat(16, axis=1)
    a = np.abs(x.astype(np.float64))
    half = np.where(a < 2 * s, 0.25, np.where(a < 4 * s, 0.5, 1.0)) * s
    err = np.abs(v - x)
    assert np.all(err <= np.maximum(half, a - 6 * s) + 1e-12)


def test_attention_e4m3_planes_dense():
    w = _small_workload(B=1, T=1, E=192, K=256, shuffle=True)
    pt = w.page_table()
    l, s = orc.fp4e4m3_quantize(w.latent_seq(0))
    lat = w.to_physical(lambda b: l, pt)
    scl = w.to_physical(lambda b: s, pt)
    rope = w.to_physical(w.rope_seq, pt)
    idx = np.concatenate([np.arange(192), -np.ones(64)]).astype(np.int32)[None]
    o, lse = orc.sparse_attn(w.P, w.q(), lat, scl, rope, pt, w.seq_id(), idx, fmt=1)
    ro, rl = _dense_reference(w.q()[0], orc.fp4e4m3_dequantize(l, s), _f(w.rope_seq(0)),
                              1 / 24.0)
    np.testing.assert_allclose(o[0], ro, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse[0], rl, rtol=1e-12)


# ---------------------------------------------------------------- KV append (block pooling)
def _append_inputs(n=6, D=576, seed=21):
    c = synth.normal_f32(seed, 1, 0, n * 4 * D).reshape(n, 4, D)
    z = (2.0 * synth.normal_f32(seed, 2, 0, n * 4 * D)).reshape(n, 4, D).astype(np.float32)
    return c, z


def test_kv_pool_equal_logits_is_mean():
    c, z = _append_inputs()
    z[:] = 0.75
    np.testing.assert_allclose(orc.kv_pool(c, z), c.astype(np.float64).mean(axis=1),
                               rtol=1e-14, atol=1e-15)


def test_kv_pool_dominant_token_and_two_token_weights():
    c, z = _append_inputs()
    z[:] = -1e4
    z[:, 2] = 0.0                                   # exp(-1e4) underflows to 0 in fp64
    np.testing.assert_array_equal(orc.kv_pool(c, z), c[:, 2].astype(np.float64))
    # logits log 3 and log 1 on tokens 0 and 1: weights 3/4 and 1/4
    z[:] = -1e4
    z[:, 0] = np.float32(np.log(3.0))
    z[:, 1] = 0.0
    w0 = 1.0 / (1.0 + np.exp(-np.float64(np.float32(np.log(3.0)))))
    ref = w0 * c[:, 0] + (1 - w0) * c[:, 1]
    np.testing.assert_allclose(orc.kv_pool(c, z), ref, rtol=1e-13, atol=1e-15)


def test_kv_pool_shift_and_permutation_invariance_and_convexity():
    c, z = _append_inputs()
    z = (np.round(z * 64) / 64).astype(np.float32)  # exact after adding 7.5
    y = orc.kv_pool(c, z)
    np.testing.assert_allclose(orc.kv_pool(c, z + np.float32(7.5)), y, rtol=1e-14, atol=1e-15)
    perm = [3, 0, 2, 1]
    np.testing.assert_allclose(orc.kv_pool(c[:, perm], z[:, perm]), y, rtol=1e-14, atol=1e-15)
    assert np.all(y <= c.max(axis=1) + 1e-12) and np.all(y >= c.min(axis=1) - 1e-12)


def test_round_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-6, 6, 2000),
                        1.0 + np.arange(16) * 2.0 ** -9, -(1.0 + np.arange(16) * 2.0 ** -9),
                        [0.0, -0.0]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(orc.round_bf16(x.astype(np.float64)), ref)


def test_kv_append_composes_pooling_with_the_cache_formats():
    c, z = _append_inputs()
    ci, zi = _append_inputs(D=64, seed=22)
    out = orc.kv_append(c, z, ci, zi)
    y = orc.kv_pool(c, z)
    lat, scl = orc.mxfp4_quantize(y[:, :512].astype(np.float32))
    np.testing.assert_array_equal(out["lat"], lat)
    np.testing.assert_array_equal(out["scl"], scl)
    np.testing.assert_array_equal(out["rope"], orc.round_bf16(y[:, 512:]))
    np.testing.assert_array_equal(out["k_idx"], orc.round_bf16(orc.kv_pool(ci, zi)))


# ---------------------------------------------------------------- footprint
def test_footprint_structure():
    # one entry = 256 B of E2M1 codes + 16 E8M0 scale bytes + 64 bf16 rope = 400 B
    assert 512 // 2 + 512 // 32 + 64 * 2 == 400
    # 1M-token context at 4:1 compression: 262,144 entries x 400 B = 100 MiB per layer
    assert 262144 * 400 == 100 * 2 ** 20
    assert orc.footprint_bytes_per_token([orc.FULL]) == (400 + 128) / 4
    assert orc.footprint_bytes_per_token([orc.FULL, orc.REINDEX, orc.REUSE]) == 164.0
    assert orc.footprint_bytes_per_token([orc.REUSE]) == 0.0
    # [summary] Results, KV cache compression: 890 B/token against ~3,560 (V4-Flash) and
    # ~389,000 (V1) gives the quoted 1/4 and ~437x
    assert 3560 / 890 == 4.0
    assert round(389000 / 890) == 437


def test_bf16_storage_rounding_matches_torch():
    x = synth.normal_f32(9, 1, 0, 100000) * np.float32(37.0)
    ours = _bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(synth.normal_bf16(9, 1, 0, 1000),
                                  _bf16(synth.normal_f32(9, 1, 0, 1000)))
