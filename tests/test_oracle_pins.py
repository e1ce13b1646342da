"""Pins of the CPU oracle against things other than itself.

Each test ties an oracle function to a closed form, a brute-force scalar loop,
a library routine (torch's float64 scaled_dot_product_attention and
logsumexp, scipy's expit/softmax), a hand-derived golden case, or an exact
invariant of the mathematics.  None of these retypes the oracle's own code.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import mla_oracle as om
from verify_inputs import LATENT, NOPE, PAGE, build_inputs, f32_to_bf16_bits

from probes import needle_case, needle_expected

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ helpers
def small_case(seed, batch=2, heads=3, q_len=4, ctx=(130, 70), bounds=None, q_scale=1.0,
               latent_q=False):
    return build_inputs(batch=batch, heads=heads, q_len=q_len, ctx=np.array(ctx[:batch]),
                        bounds=bounds, seed=seed, q_scale=q_scale, latent_q=latent_q)


def dense_cache_loop(pool_dense, block_table, b, n):
    """Request b's first n cache rows, gathered one token at a time (float64)."""
    rows = []
    for j in range(n):
        page = int(block_table[b, j // PAGE])
        bits = pool_dense[page, j % PAGE].astype(np.uint32) << 16
        rows.append(bits.view(np.float32).astype(np.float64))
    return np.array(rows).reshape(n, LATENT)


def f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)


# ------------------------------------------------------------------ encoding
def test_bf16_decode_known_patterns():
    pats = np.array([0x3F80, 0xC000, 0x4049, 0x0001, 0x8000, 0x7F80, 0xFF80, 0x7F7F], np.uint16)
    want = [1.0, -2.0, 3.140625, 2.0 ** -133, -0.0, math.inf, -math.inf,
            (2 - 2 ** -7) * 2.0 ** 127]
    got = om.bf16_to_f64(pats)
    assert got.tolist() == want
    assert math.copysign(1.0, got[4]) == -1.0
    assert np.isnan(om.bf16_to_f64(np.array([0x7FC0], np.uint16)))[0]


def test_sigmoid_matches_library():
    x = np.concatenate([np.linspace(-40, 40, 801), [-800.0, 800.0, 0.0]])
    np.testing.assert_allclose(om.sigmoid(x), scipy.special.expit(x), rtol=1e-15, atol=0)
    assert om.sigmoid(np.array([0.0]))[0] == 0.5


# ------------------------------------------------------------------ golden
def test_hand_derived_golden_case():
    g = json.load(open(os.path.join(GOLDEN, "hand_three_keys.json")))
    pool = np.full((2, PAGE, LATENT), 0x7FC0, np.uint16)   # NaN everywhere
    pool[1, :3] = 0
    pool[1, 0, 0] = 0x3F80      # c0 = e0
    pool[1, 1, 1] = 0x3F80      # c1 = e1   (c2 = 0)
    bt = np.array(g["block_table"], np.int32)
    bounds = np.array(g["kv_bounds"], np.int32)
    q = np.zeros((1, 3, 1, LATENT), np.uint16)
    q[..., 0] = 0x3F80
    o, lse = oracle.verify_attention_latent(q, pool, bt, bounds, math.log(3.0))
    exp_lse = [float(v) for v in g["expected"]["lse"]]
    for t in range(3):
        if math.isinf(exp_lse[t]):
            assert lse[0, t, 0] == -math.inf
        else:
            assert lse[0, t, 0] == pytest.approx(exp_lse[t], abs=1e-15)
        np.testing.assert_allclose(o[0, t, 0, :3], g["expected"]["o_lat_head"][t], atol=1e-15)
        assert np.all(o[0, t, 0, 3:] == 0)
    w_uv = np.zeros((1, NOPE, LATENT), np.uint16)
    w_uv[0, 0, 0] = 0x3F80
    w_uv[0, 1, 1] = 0x4000
    gate = np.zeros((1, 3, 1, NOPE), np.uint16)
    out = oracle.gated_output(o, w_uv, gate)
    for t in range(3):
        np.testing.assert_allclose(out[0, t, 0, :3], g["expected"]["out_head"][t], atol=1e-15)


# ------------------------------------------------------------------ library routine
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_torch_sdpa_float64(seed):
    rng = np.random.default_rng(100 + seed)
    ctx = np.array([130, 70])
    bounds = rng.integers(0, 131, size=(2, 4)).astype(np.int32)
    bounds[1] = np.minimum(bounds[1], 70)
    bounds[0, 0] = 0
    x = small_case(seed, ctx=ctx, bounds=bounds, q_scale=1536.0 if seed == 2 else 1.0)
    r = oracle.verify_attention_mla(x.q_nope, x.w_uk, x.w_uv, x.gate, x.pool, x.block_table,
                                    x.kv_bounds, x.sm_scale)
    dense = x.pool.dense()
    for b in range(2):
        n = int(bounds[b].max())
        cache = torch.tensor(dense_cache_loop(dense, x.block_table, b, n))
        wk = torch.tensor(f64(x.w_uk))
        wv = torch.tensor(f64(x.w_uv))
        k = torch.einsum("nc,hdc->hnd", cache, wk)             # [H, n, 128]
        v = torch.einsum("nc,hdc->hnd", cache, wv)
        q = torch.tensor(f64(x.q_nope[b])).permute(1, 0, 2)    # [H, T, 128]
        mask = torch.arange(n)[None, :] < torch.tensor(bounds[b])[:, None]   # [T, n]
        o = torch.nn.functional.scaled_dot_product_attention(
            q, k, v, attn_mask=mask, scale=x.sm_scale)          # [H, T, 128]
        s = torch.einsum("htd,hnd->htn", q, k) * x.sm_scale
        lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)   # [H, T]
        for t in range(4):
            if bounds[b, t] == 0:
                assert np.all(r["lse"][b, t] == -np.inf) and np.all(r["o_v"][b, t] == 0)
                continue
            np.testing.assert_allclose(r["o_v"][b, t], o[:, t].numpy(), rtol=1e-10, atol=1e-14)
            np.testing.assert_allclose(r["lse"][b, t], lse[:, t].numpy(), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ brute force
def scalar_decode(q, keys, values, scale):
    """Textbook single-query attention with explicit scalar loops."""
    scores = [scale * sum(qi * ki for qi, ki in zip(q, k)) for k in keys]
    m = max(scores)
    ws = [math.exp(s - m) for s in scores]
    tot = sum(ws)
    out = [sum(w * v[d] for w, v in zip(ws, values)) / tot for d in range(len(values[0]))]
    return out, m + math.log(tot)


def test_each_token_is_a_standalone_decode_bruteforce():
    rng = np.random.default_rng(7)
    ctx = np.array([130, 66])
    bounds = np.array([[127, 128, 129, 130], [63, 64, 65, 66]], np.int32)
    bounds[0, 1] = 65           # non-monotone bound, crossing a page boundary
    x = small_case(11, heads=2, ctx=ctx, bounds=bounds, q_scale=800.0)
    r = oracle.verify_attention_mla(x.q_nope, x.w_uk, x.w_uv, x.gate, x.pool, x.block_table,
                                    x.kv_bounds, x.sm_scale)
    dense = x.pool.dense()
    wk, wv = f64(x.w_uk), f64(x.w_uv)
    for b in range(2):
        for t in range(4):
            L = int(bounds[b, t])
            cache = dense_cache_loop(dense, x.block_table, b, L).tolist()
            for h in range(2):
                # up-project key by key: k[d] = <W[h][d], c>
                keys = [[float(np.dot(wk[h, d], c)) for d in range(NOPE)] for c in cache]
                vals = [[float(np.dot(wv[h, d], c)) for d in range(NOPE)] for c in cache]
                q = f64(x.q_nope[b, t, h]).tolist()
                o_v, lse = scalar_decode(q, keys, vals, x.sm_scale)
                o_lat, _ = scalar_decode(q, keys, cache, x.sm_scale)
                g = 1.0 / (1.0 + math.exp(-float(f64(x.gate[b, t, h, 0]))))
                assert r["lse"][b, t, h] == pytest.approx(lse, rel=1e-12)
                np.testing.assert_allclose(r["o_v"][b, t, h], o_v, rtol=1e-9, atol=1e-13)
                np.testing.assert_allclose(r["o_lat"][b, t, h], o_lat, rtol=1e-9, atol=1e-13)
                assert r["out"][b, t, h, 0] == pytest.approx(g * o_v[0], rel=1e-9, abs=1e-15)
    _ = rng


def test_k0_reduces_to_plain_decode():
    """q_len 1: the verify call is ordinary single-token decode (scipy softmax)."""
    x = build_inputs(batch=3, heads=4, q_len=1, ctx=np.array([1, 64, 200]), seed=5,
                     q_scale=500.0)
    r = oracle.verify_attention_mla(x.q_nope, x.w_uk, x.w_uv, x.gate, x.pool, x.block_table,
                                    x.kv_bounds, x.sm_scale)
    dense = x.pool.dense()
    for b, n in enumerate([1, 64, 200]):
        cache = dense_cache_loop(dense, x.block_table, b, n)
        for h in range(4):
            k = cache @ f64(x.w_uk[h]).T
            v = cache @ f64(x.w_uv[h]).T
            s = x.sm_scale * (k @ f64(x.q_nope[b, 0, h]))
            p = scipy.special.softmax(s)
            np.testing.assert_allclose(r["o_v"][b, 0, h], p @ v, rtol=1e-10, atol=1e-14)
            assert r["lse"][b, 0, h] == pytest.approx(scipy.special.logsumexp(s), rel=1e-13)


# ------------------------------------------------------------------ invariants
def test_absorbed_equals_unabsorbed():
    x = small_case(3, ctx=(130, 90), q_scale=1536.0)
    r = oracle.verify_attention_mla(x.q_nope, x.w_uk, x.w_uv, x.gate, x.pool, x.block_table,
                                    x.kv_bounds, x.sm_scale)
    q_lat = oracle.absorb_query(x.q_nope, x.w_uk)
    o_lat, lse = oracle.verify_attention_latent(q_lat, x.pool, x.block_table, x.kv_bounds,
                                                x.sm_scale, q_is_f64=True)
    np.testing.assert_allclose(lse, r["lse"], rtol=1e-12)
    np.testing.assert_allclose(o_lat, r["o_lat"], rtol=1e-10, atol=1e-15)
    # W_UV after the latent average equals the average of up-projected values
    o_v = np.einsum("hdc,bthc->bthd", f64(x.w_uv), o_lat)
    np.testing.assert_allclose(o_v, r["o_v"], rtol=1e-10, atol=1e-15)
    out = oracle.gated_output(o_lat, x.w_uv, x.gate)
    np.testing.assert_allclose(out, r["out"], rtol=1e-10, atol=1e-15)


def test_split_pages_partition():
    for n in [0, 1, 63, 64, 65, 130, 1000, 8192]:
        for s in [1, 2, 3, 4, 7, 8, 16, 200]:
            ch = oracle.split_pages(n, s)
            assert len(ch) == s
            cover = [j for a, bnd in ch for j in range(a, bnd)]
            assert cover == list(range(n))
            for a, bnd in ch:
                assert a % PAGE == 0 or a == n


@pytest.mark.parametrize("seed", [0, 1])
def test_split_invariance_random_partitions(seed):
    rng = np.random.default_rng(seed)
    x = small_case(20 + seed, ctx=(200, 130), q_scale=1536.0, latent_q=True)
    o_full, lse_full = oracle.verify_attention_latent(x.q_latent, x.pool, x.block_table,
                                                      x.kv_bounds, x.sm_scale)
    q = f64(x.q_latent)
    for b in range(2):
        cache, n = oracle.request_keys(x.pool, x.block_table, x.kv_bounds, b)
        for t in range(4):
            L = oracle.token_bound(x.kv_bounds, b, t, n)
            for _ in range(3):
                cuts = np.sort(rng.integers(0, L + 1, size=rng.integers(1, 6)))
                edges = [0, *cuts.tolist(), L, L]        # includes empty chunks
                edges += [L]
                for h in range(3):
                    parts = [oracle.attend_chunk(q[b, t, h], cache[a:e], x.sm_scale)
                             for a, e in zip(edges[:-1], edges[1:])]
                    o, lse = oracle.lse_merge(parts)
                    if L == 0:
                        assert lse == -np.inf and np.all(o == 0)
                        continue
                    assert lse == pytest.approx(lse_full[b, t, h], rel=1e-12)
                    np.testing.assert_allclose(o, o_full[b, t, h], rtol=1e-10, atol=1e-15)


def test_identity_rows_and_merge():
    bounds = np.array([[0, 5, 0]], np.int32)
    x = build_inputs(batch=1, heads=2, q_len=3, ctx=np.array([5]), bounds=bounds, seed=9)
    r = oracle.verify_attention_mla(x.q_nope, x.w_uk, x.w_uv, x.gate, x.pool, x.block_table,
                                    x.kv_bounds, x.sm_scale)
    for t in (0, 2):
        assert np.all(r["lse"][0, t] == -np.inf)
        for key in ("o_v", "o_lat", "out"):
            assert np.all(r[key][0, t] == 0)
    assert np.all(np.isfinite(r["lse"][0, 1]))
    o = np.arange(4.0)
    merged = oracle.lse_merge([(o, 0.7), (np.zeros(4), -np.inf)])
    assert merged[1] == 0.7 and np.array_equal(merged[0], o)
    empty = oracle.lse_merge([(np.zeros(4), -np.inf)] * 3)
    assert empty[1] == -np.inf and np.all(empty[0] == 0)
    # a whole request with every bound 0 reads no page at all
    x0 = build_inputs(batch=1, heads=1, q_len=2, ctx=np.array([0]),
                      bounds=np.zeros((1, 2), np.int32), seed=1)
    o0, l0 = oracle.verify_attention_latent(x0.q_nope.repeat(4, -1), x0.pool, x0.block_table,
                                            x0.kv_bounds, 1.0)
    assert np.all(l0 == -np.inf) and np.all(o0 == 0)


def test_closed_forms():
    x = build_inputs(batch=1, heads=1, q_len=3, ctx=np.array([100]),
                     bounds=np.array([[100, 1, 37]], np.int32), seed=4, latent_q=True)
    cache, _ = oracle.request_keys(x.pool, x.block_table, x.kv_bounds, 0)
    # q = 0: uniform weights
    qz = np.zeros_like(x.q_latent)
    o, lse = oracle.verify_attention_latent(qz, x.pool, x.block_table, x.kv_bounds, 0.3)
    assert lse[0, 0, 0] == pytest.approx(math.log(100), rel=1e-15)
    assert lse[0, 2, 0] == pytest.approx(math.log(37), rel=1e-15)
    np.testing.assert_allclose(o[0, 0, 0], cache.mean(axis=0), rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(o[0, 2, 0], cache[:37].mean(axis=0), rtol=1e-12, atol=1e-16)
    # L = 1: the single key, lse = its score
    o, lse = oracle.verify_attention_latent(x.q_latent, x.pool, x.block_table, x.kv_bounds, 0.3)
    assert np.array_equal(o[0, 1, 0], cache[0])
    assert lse[0, 1, 0] == pytest.approx(0.3 * float(f64(x.q_latent[0, 1, 0]) @ cache[0]),
                                         rel=1e-14)
    # all keys equal to c: o = c, lse = s + ln L
    pool = np.zeros((2, PAGE, LATENT), np.uint16)
    c = f32_to_bf16_bits(np.linspace(-1, 1, LATENT, dtype=np.float32))
    pool[:] = c
    bt = np.array([[1, 0]], np.int32)
    o, lse = oracle.verify_attention_latent(x.q_latent[:, :1], pool, bt,
                                            np.array([[100]], np.int32), 0.3)
    s = 0.3 * float(f64(x.q_latent[0, 0, 0]) @ f64(c))
    np.testing.assert_allclose(o[0, 0, 0], f64(c), rtol=1e-13)
    assert lse[0, 0, 0] == pytest.approx(s + math.log(100), rel=1e-13)
    # gate 0 halves W_UV o exactly; a huge gate leaves it unchanged
    o_lat = np.random.default_rng(0).standard_normal((1, 1, 2, LATENT))
    w = build_inputs(batch=1, heads=2, q_len=1, ctx=np.array([1]), seed=3).w_uv
    g0 = np.zeros((1, 1, 2, NOPE), np.uint16)
    gbig = np.full((1, 1, 2, NOPE), 0x4780, np.uint16)        # 65536
    ref = np.einsum("hdc,bthc->bthd", f64(w), o_lat)
    assert np.array_equal(oracle.gated_output(o_lat, w, g0), ref * 0.5)
    assert np.array_equal(oracle.gated_output(o_lat, w, gbig), ref)


def test_page_permutation_invariance():
    x = small_case(30, ctx=(190, 130), latent_q=True, q_scale=1536.0)
    o1, l1 = oracle.verify_attention_latent(x.q_latent, x.pool, x.block_table, x.kv_bounds,
                                            x.sm_scale)
    perm = np.random.default_rng(1).permutation(x.pool.num_pages)
    pool2 = x.pool.remap(perm)
    bt2 = np.where(x.block_table >= 0, perm[np.maximum(x.block_table, 0)], -1).astype(np.int32)
    o2, l2 = oracle.verify_attention_latent(x.q_latent, pool2, bt2, x.kv_bounds, x.sm_scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_head_independence():
    x = small_case(40, ctx=(100, 80), q_scale=1536.0)
    r1 = oracle.verify_attention_mla(x.q_nope, x.w_uk, x.w_uv, x.gate, x.pool, x.block_table,
                                     x.kv_bounds, x.sm_scale)
    q2, wk2 = x.q_nope.copy(), x.w_uk.copy()
    q2[:, :, 1] ^= 0x00FF
    wk2[1] ^= 0x0055
    r2 = oracle.verify_attention_mla(q2, wk2, x.w_uv, x.gate, x.pool, x.block_table,
                                     x.kv_bounds, x.sm_scale)
    for h in (0, 2):
        assert np.array_equal(r1["o_v"][:, :, h], r2["o_v"][:, :, h])
        assert np.array_equal(r1["lse"][:, :, h], r2["lse"][:, :, h])
    assert not np.allclose(r1["o_v"][:, :, 1], r2["o_v"][:, :, 1])


def test_nan_poison_never_reaches_outputs():
    x = small_case(50, ctx=(130, 65), q_scale=1536.0)
    dense = x.pool.dense()
    assert np.isnan(f64(dense)).any()        # the pool really is poisoned
    r = oracle.verify_attention_mla(x.q_nope, x.w_uk, x.w_uv, x.gate, dense, x.block_table,
                                    x.kv_bounds, x.sm_scale)
    for key in ("o_v", "o_lat", "out"):
        assert np.all(np.isfinite(r[key]))
    assert not np.isnan(r["lse"]).any()


def test_needle_probe_oracle_exact():
    bounds = np.array([[1, 64, 65, 63], [129, 100, 128, 2], [0, 200, 255, 192]], np.int32)
    x, pool, q, bounds = needle_case(bounds)
    o, lse = oracle.verify_attention_latent(q, pool, x.block_table, bounds, 1.0)
    want = needle_expected(x, bounds)
    for b in range(bounds.shape[0]):
        for t in range(bounds.shape[1]):
            for h in range(2):
                assert np.array_equal(o[b, t, h], want[b, t])
            assert np.all(lse[b, t] == (0.0 if bounds[b, t] > 0 else -np.inf))


# ------------------------------------------------------------------ mutation check
def _pins_pass():
    """Run a cheap subset of the pins; True if all pass."""
    try:
        test_matches_torch_sdpa_float64(0)
        test_closed_forms()
        test_needle_probe_oracle_exact()
        test_hand_derived_golden_case()
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("mutant", ["bound_plus_one", "bound_minus_one", "page_reversed",
                                    "scores_perturbed", "wuk_transposed", "gate_negated",
                                    "no_max_shift_lse"])
def test_planted_oracle_mistakes_are_caught(monkeypatch, mutant):
    """A plausible mistake planted in the oracle must make some pin fail."""
    assert _pins_pass()
    if mutant == "bound_plus_one":
        orig = om.token_bound
        monkeypatch.setattr(om, "token_bound", lambda kb, b, t, n: min(orig(kb, b, t, n) + 1, n))
    elif mutant == "bound_minus_one":
        orig = om.token_bound
        monkeypatch.setattr(om, "token_bound", lambda kb, b, t, n: max(orig(kb, b, t, n) - 1, 0))
    elif mutant == "page_reversed":
        orig = om.request_keys

        def rk(pool, bt, kb, b, decode=None):
            n_pg = -(-int(np.clip(np.max(kb[b]), 0, bt.shape[1] * PAGE)) // PAGE)
            bt2 = bt.copy()
            bt2[b, :n_pg] = bt[b, :n_pg][::-1]
            return orig(pool, bt2, kb, b, decode)
        monkeypatch.setattr(om, "request_keys", rk)
    elif mutant == "scores_perturbed":
        orig = om.softmax_attend
        monkeypatch.setattr(om, "softmax_attend", lambda s, v: orig(s * 1.0001 + 1e-3, v))
    elif mutant == "wuk_transposed":
        orig = om.bf16_to_f64

        def dec(bits):
            a = orig(bits)
            if a.ndim == 3 and a.shape[1:] == (NOPE, LATENT):
                a = a[:, ::-1, :].copy()
            return a
        monkeypatch.setattr(om, "bf16_to_f64", dec)
    elif mutant == "gate_negated":
        orig = om.sigmoid
        monkeypatch.setattr(om, "sigmoid", lambda x: orig(-np.asarray(x)) * 1.0 + 0.0
                            if np.any(np.asarray(x) != 0) else orig(x) * 0.999)
    elif mutant == "no_max_shift_lse":
        orig = om.softmax_attend

        def sa(scores, values):
            o, lse = orig(scores, values)
            return o, lse - np.log(max(scores.shape[-1], 1)) * 1e-3
        monkeypatch.setattr(om, "softmax_attend", sa)
    assert not _pins_pass(), f"planted mistake {mutant} went unnoticed"
