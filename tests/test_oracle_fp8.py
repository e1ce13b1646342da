"""Pins of the oracle's fp8 (OCP E4M3) latent-cache path.

The pages run the serving stack with an fp8 KV cache and note that the
per-token-bound decode kernel they describe still rejects fp8 KV; the format
and the scale convention are not spelled out there, so the reading is: OCP
E4M3 codes (bias 7, no infinities, 0x7F/0xFF NaN) and one per-cache scale,
latent = kv_scale * value(code).  The decoder is pinned to the format
definition (hand-listed values), to torch's float8_e4m3fn conversion, and the
fp8 attention to the already pinned bf16 attention and to the exact way a
scale must enter both the scores and the values.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import mla_oracle as om
from verify_inputs import (FP8_KV_SCALE, PAGE, build_inputs, f32_to_bf16_bits, fp8_cache,
                           make_config)

ALL_CODES = np.arange(256, dtype=np.uint8)


def test_decode_matches_torch_float8_e4m3fn():
    ref = torch.from_numpy(ALL_CODES.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = om.fp8_e4m3_to_f64(ALL_CODES)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x30, 0.5), (0x38, 1.0), (0x39, 1.125), (0x3C, 1.5), (0x40, 2.0), (0x77, 240.0),
    (0x78, 256.0), (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0), (0x81, -(2.0 ** -9)),
])
def test_decode_closed_forms(code, value):
    # (1 + m/8) 2^(e-7) for e > 0, (m/8) 2^-6 for e = 0: values written out by hand
    assert om.fp8_e4m3_to_f64(np.array([code], np.uint8))[0] == value


def test_decode_special_codes_and_order():
    got = om.fp8_e4m3_to_f64(ALL_CODES)
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert np.isnan(got).sum() == 2                     # no infinities, only two NaNs
    assert got[0x80] == 0.0 and math.copysign(1.0, got[0x80]) == -1.0
    pos = got[:0x7F]
    assert np.all(np.diff(pos) > 0)                     # codes 0..0x7E increase strictly
    assert np.array_equal(got[0x80:0xFF], -pos)          # sign bit mirrors
    # every E4M3 value has at most 4 significant bits, so bf16 holds it exactly
    assert np.array_equal(om.bf16_to_f64(f32_to_bf16_bits(pos.astype(np.float32))), pos)


def _bf16_twin(x8):
    """The same batch with a bf16 cache holding exactly kv_scale * value(code)."""
    vals = om.fp8_e4m3_to_f64(x8.pool.pages) * x8.kv_scale
    bits = f32_to_bf16_bits(vals.astype(np.float32))
    assert np.array_equal(om.bf16_to_f64(bits)[~np.isnan(vals)], vals[~np.isnan(vals)])
    pool = type(x8.pool)(x8.pool.num_pages, x8.pool.page_ids, bits)
    return pool


@pytest.mark.parametrize("seed", [0, 1])
def test_fp8_attention_equals_bf16_attention_on_the_decoded_values(seed):
    x = build_inputs(batch=2, heads=3, q_len=4, ctx=np.array([150, 70]), seed=seed, q_scale=300.0)
    x8 = fp8_cache(x, 2.0 ** -7)
    q = oracle.absorb_query(x8.q_nope, x8.w_uk)
    o8, l8 = oracle.verify_attention_latent(q, x8.pool, x8.block_table, x8.kv_bounds, x8.sm_scale,
                                            q_is_f64=True, kv_dtype="fp8", kv_scale=x8.kv_scale)
    o, l = oracle.verify_attention_latent(q, _bf16_twin(x8), x8.block_table, x8.kv_bounds,
                                          x8.sm_scale, q_is_f64=True)
    assert np.allclose(o8, o, rtol=0, atol=1e-14)
    assert np.array_equal(np.isneginf(l8), np.isneginf(l))
    fin = np.isfinite(l)
    assert np.allclose(l8[fin], l[fin], rtol=0, atol=1e-13)
    # the unabsorbed definition agrees as well
    m8 = oracle.verify_attention_mla(x8.q_nope, x8.w_uk, x8.w_uv, x8.gate, x8.pool, x8.block_table,
                                     x8.kv_bounds, x8.sm_scale, kv_dtype="fp8",
                                     kv_scale=x8.kv_scale)
    assert np.allclose(m8["o_lat"], o, rtol=0, atol=1e-13)


def test_scale_enters_scores_and_values():
    """latent = s * v: scores scale by s (same as sm_scale * s) and the output
    by s, so o(s, sm) = s * o(1, sm * s) and lse(s, sm) = lse(1, sm * s)."""
    x8 = fp8_cache(build_inputs(batch=2, heads=2, q_len=3, ctx=np.array([100, 65]), seed=3,
                                q_scale=200.0), 2.0 ** -6)
    q = oracle.absorb_query(x8.q_nope, x8.w_uk)
    args = (q, x8.pool, x8.block_table, x8.kv_bounds)
    for s in (0.37, 2.0 ** -6, 5.0):
        o_s, l_s = oracle.verify_attention_latent(*args, x8.sm_scale, q_is_f64=True,
                                                  kv_dtype="fp8", kv_scale=s)
        o_1, l_1 = oracle.verify_attention_latent(*args, x8.sm_scale * s, q_is_f64=True,
                                                  kv_dtype="fp8", kv_scale=1.0)
        # entries near zero carry cancellation error, so the bound is relative
        # to the output's scale
        assert np.abs(o_s - s * o_1).max() <= 1e-12 * np.abs(o_s).max()
        fin = np.isfinite(l_1)
        assert np.allclose(l_s[fin], l_1[fin], rtol=1e-13)


def test_workload_codes_are_in_the_normal_range():
    """The fp8 workloads (bf16 draws / 2^-8) use codes far from overflow and
    mostly above the subnormal range; unreferenced slots hold the NaN code."""
    x8 = fp8_cache(make_config(2))
    assert x8.kv_scale == FP8_KV_SCALE
    vals = om.fp8_e4m3_to_f64(x8.pool.pages)
    fin = vals[~np.isnan(vals)]
    assert np.abs(fin).max() < 448.0
    assert np.mean(np.abs(fin) < 2.0 ** -6) < 0.01
    n_keys = int(x8.kv_bounds.max(axis=1)[0])
    page0 = x8.pool[np.array([x8.block_table[0, n_keys // PAGE]])][0]
    if n_keys % PAGE:
        assert np.all(page0[n_keys % PAGE:] == 0x7F)


@pytest.mark.parametrize("mutant", ["bias8", "subnormal_as_normal", "scale_dropped"])
def test_planted_fp8_mistakes_are_caught(monkeypatch, mutant):
    """Each plausible mistake in the fp8 path fails one of the pins above."""
    real = om.fp8_e4m3_to_f64
    if mutant == "bias8":
        monkeypatch.setattr(om, "fp8_e4m3_to_f64", lambda c: real(c) / 2.0)
        with pytest.raises(AssertionError):
            test_decode_closed_forms(0x38, 1.0)
    elif mutant == "subnormal_as_normal":
        def bad(c):
            c = np.asarray(c, dtype=np.uint8)
            out = real(c)
            e0 = ((c >> 3) & 0xF) == 0
            return np.where(e0 & ((c & 7) > 0), out + np.sign(out) * 2.0 ** -6, out)
        monkeypatch.setattr(om, "fp8_e4m3_to_f64", bad)
        with pytest.raises(AssertionError):
            test_decode_matches_torch_float8_e4m3fn()
    else:
        def bad_decoder(kv_dtype="bf16", kv_scale=1.0):
            if kv_dtype == "fp8":
                return lambda c: real(c)        # scale dropped from the values
            return om.bf16_to_f64
        monkeypatch.setattr(om, "kv_decoder", bad_decoder)
        with pytest.raises(AssertionError):
            test_scale_enters_scores_and_values()
