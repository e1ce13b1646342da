"""Parity of the fp8 (OCP E4M3) latent-cache path with the float64 oracle.

The cache holds E4M3 codes and one scale (latent = kv_scale * value(code));
the oracle decodes the same codes exactly.  Bars as for the bf16 path:
outputs max-abs <= 1e-2 and relative L2 <= 5e-3, finite LSE within 1e-3,
masked rows exactly (-inf, 0), the needle probe bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import speculative_verify_attention_absorbed_amd as mv
from gpu_util import (assert_close_output, assert_lse, assert_masked_rows_zero, bits_of,
                      bf16_tensor, f64_of, log, round_bf16, sync, upload_fp8)
from probes import needle_case_fp8, needle_expected_fp8
from verify_inputs import build_inputs, fp8_cache, make_config

pytestmark = pytest.mark.gpu


def qlat_bits(x):
    return round_bf16(oracle.absorb_query(x.q_nope, x.w_uk))


def check_fp8(x, d, q_bits, num_splits=None, tile_rows=0, kv_scale=None, what=""):
    s = x.num_splits if num_splits is None else num_splits
    scale = x.kv_scale if kv_scale is None else kv_scale
    out, lse = mv.verify_attn(d["q_latent"], d["pool"], d["block_table"], d["kv_bounds"],
                              x.sm_scale, num_splits=s, tile_rows=tile_rows,
                              kv_dtype=mv.KV_FP8_E4M3, kv_scale=scale)
    sync()
    got, got_lse = f64_of(out), lse.cpu().numpy().astype(np.float64)
    want, want_lse = oracle.verify_attention_latent(q_bits, x.pool, x.block_table, x.kv_bounds,
                                                    x.sm_scale, kv_dtype="fp8", kv_scale=scale)
    assert_lse(got_lse, want_lse, f"{what} lse")
    assert_masked_rows_zero(got, want_lse, f"{what} out_latent")
    assert_close_output(got, want, f"{what} out_latent")
    return out, lse


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
@pytest.mark.parametrize("sharp", [False, True])
def test_fp8_latent_parity_configs(cfg, sharp):
    log(f"fp8 latent parity: config {cfg} sharp={sharp}")
    x = fp8_cache(make_config(cfg, sharp=sharp))
    q = qlat_bits(x)
    check_fp8(x, upload_fp8(x, q), q, what=f"fp8 cfg{cfg}")


def test_fp8_latent_parity_config5():
    log("fp8 latent parity: config 5 (ragged, zero and truncated bounds), S=8")
    x = fp8_cache(make_config(5))
    q = qlat_bits(x)
    check_fp8(x, upload_fp8(x, q), q, what="fp8 cfg5")


@pytest.mark.parametrize("tile", [32, 64, 128])
@pytest.mark.parametrize("cfg,splits", [(3, 4), (2, 8), (4, 2)])
def test_fp8_forced_tiles(cfg, tile, splits):
    log(f"fp8 forced tile: config {cfg} (sharp), tile {tile}, S={splits}")
    x = fp8_cache(make_config(cfg, sharp=True))
    q = qlat_bits(x)
    check_fp8(x, upload_fp8(x, q), q, num_splits=splits, tile_rows=tile, what=f"fp8 tile{tile}")


def test_fp8_odd_bounds_pair_staging():
    """Key rows are staged in pairs: every bound parity, page edges, a single
    key, zero rows and an empty request, on every tile shape and split count."""
    log("fp8 odd/even bounds, page edges, zero rows")
    rng = np.random.default_rng(11)
    b, t, h = 6, 6, 8
    ctx = np.array([201, 1, 0, 333, 64, 130])
    bounds = np.stack([rng.integers(0, c + 1, size=t) for c in ctx]).astype(np.int32)
    bounds[2] = 0
    bounds[4] = [64, 0, 63, 1, 65 - 1, 3]
    bounds[5] = [129, 127, 65, 66, 2, 130]
    x = fp8_cache(build_inputs(batch=b, heads=h, q_len=t, ctx=ctx, bounds=bounds, seed=9,
                               latent_q=True, q_scale=1536.0))
    d = upload_fp8(x)
    for s in (0, 1, 2, 5):
        for tile in (0, 32, 64, 128):
            check_fp8(x, d, x.q_latent, num_splits=s, tile_rows=tile, what=f"S{s} tile{tile}")


@pytest.mark.parametrize("splits", [1, 2, 4])
@pytest.mark.parametrize("tile", [0, 64, 128])
def test_fp8_needle_probe_bit_exact(splits, tile):
    log(f"fp8 needle probe, S={splits}, tile {tile}")
    bounds = np.array([[1, 64, 65, 63], [129, 100, 128, 2], [0, 200, 255, 192],
                       [255, 254, 253, 129]], np.int32)
    x, pool, q, bounds = needle_case_fp8(bounds, heads=2, kv_scale=0.5)
    want = needle_expected_fp8(x, bounds, kv_scale=0.5)
    out, lse = mv.verify_attn(bf16_tensor(q), torch.from_numpy(pool).cuda(),
                              torch.from_numpy(x.block_table).cuda(),
                              torch.from_numpy(bounds).cuda(), 1.0, num_splits=splits,
                              tile_rows=tile, kv_dtype=mv.KV_FP8_E4M3, kv_scale=0.5)
    sync()
    got, lse = f64_of(out), lse.cpu().numpy()
    for bb in range(bounds.shape[0]):
        for t in range(bounds.shape[1]):
            for hh in range(2):
                assert np.array_equal(got[bb, t, hh], want[bb, t]), (bb, t, hh, got[bb, t, hh, :8])
                assert lse[bb, t, hh] == (0.0 if bounds[bb, t] > 0 else -np.inf)


def test_fp8_scale_not_a_power_of_two():
    """A scale with a full mantissa enters the scores and the normaliser in fp32."""
    log("fp8 config 2 (sharp) with kv_scale 0.0037")
    x = fp8_cache(make_config(2, sharp=True))
    q = qlat_bits(x)
    check_fp8(x, upload_fp8(x, q), q, kv_scale=0.0037, what="fp8 scale 0.0037")


def test_fp8_gated_config5():
    """The ragged gated workload on an fp8 cache: the latent oracle, then W_UV
    and the gate in float64."""
    log("fp8 gated: config 5, S=8")
    x = fp8_cache(make_config(5))
    q = qlat_bits(x)
    d = upload_fp8(x, q)
    out, lse, lat = mv.verify_attn_gated(d["q_latent"], d["pool"], d["block_table"],
                                         d["kv_bounds"], d["w_uv"], d["gate"], x.sm_scale,
                                         num_splits=8, want_latent=True,
                                         kv_dtype=mv.KV_FP8_E4M3, kv_scale=x.kv_scale)
    sync()
    o_lat, want_lse = oracle.verify_attention_latent(q, x.pool, x.block_table, x.kv_bounds,
                                                     x.sm_scale, kv_dtype="fp8",
                                                     kv_scale=x.kv_scale)
    want = oracle.gated_output(o_lat, x.w_uv, x.gate)
    assert_lse(lse.cpu().numpy().astype(np.float64), want_lse, "fp8 cfg5 gated lse")
    assert_masked_rows_zero(f64_of(out), want_lse, "fp8 cfg5 gated out")
    assert_close_output(f64_of(out), want, "fp8 cfg5 gated out")
    assert_close_output(f64_of(lat), o_lat, "fp8 cfg5 o_lat")


@pytest.mark.parametrize("cfg,splits", [(1, None), (3, 4)])
def test_fp8_gated_end_to_end(cfg, splits):
    """The gated call on an fp8 cache against the unabsorbed oracle (explicit
    per-head K/V up-projection of the decoded latent).  Stated value spread
    only: the ABI takes q_latent rounded to bf16, which the unabsorbed oracle
    never sees, and with the sharp spread that rounding alone moves the LSE
    by ~1e-2 (the sharp cases are compared against the latent oracle, which
    takes the same bf16 query)."""
    log(f"fp8 gated end to end: config {cfg}")
    x = fp8_cache(make_config(cfg))
    q = qlat_bits(x)
    d = upload_fp8(x, q)
    s = x.num_splits if splits is None else splits
    out, lse, lat = mv.verify_attn_gated(d["q_latent"], d["pool"], d["block_table"],
                                         d["kv_bounds"], d["w_uv"], d["gate"], x.sm_scale,
                                         num_splits=s, want_latent=True,
                                         kv_dtype=mv.KV_FP8_E4M3, kv_scale=x.kv_scale)
    sync()
    r = oracle.verify_attention_mla(x.q_nope, x.w_uk, x.w_uv, x.gate, x.pool, x.block_table,
                                    x.kv_bounds, x.sm_scale, kv_dtype="fp8", kv_scale=x.kv_scale)
    assert_lse(lse.cpu().numpy().astype(np.float64), r["lse"], "fp8 gated lse")
    assert_masked_rows_zero(f64_of(out), r["lse"], "fp8 gated out")
    assert_close_output(f64_of(lat), r["o_lat"], "fp8 o_lat")
    assert_close_output(f64_of(out), r["out"], "fp8 gated out")


def test_fp8_page_permutation_and_repeat_bit_identical():
    log("fp8 page permutation and repeat: config 2 (sharp), bit-identical outputs")
    x = fp8_cache(make_config(2, sharp=True))
    q = qlat_bits(x)
    o1, l1 = check_fp8(x, upload_fp8(x, q), q, num_splits=4)
    o1b, l1b = check_fp8(x, upload_fp8(x, q), q, num_splits=4)
    assert np.array_equal(bits_of(o1), bits_of(o1b)) and torch.equal(l1, l1b)
    perm = np.random.default_rng(3).permutation(x.pool.num_pages)
    x2 = fp8_cache(make_config(2, sharp=True))
    x2.pool = x.pool.remap(perm)
    x2.block_table = np.where(x.block_table >= 0, perm[np.maximum(x.block_table, 0)],
                              -1).astype(np.int32)
    o2, l2 = check_fp8(x2, upload_fp8(x2, q), q, num_splits=4)
    assert np.array_equal(bits_of(o1), bits_of(o2)) and torch.equal(l1, l2)


def test_fp8_long_context_block_table_past_one_split_staging():
    """fp8 cache with a block-table row longer than one split stages in LDS
    (1094 page ids for 70000 keys): each split loads its own slice of the row."""
    log("fp8 long context: B=2 ctx=(70000, 3000) H=8 T=4")
    x = fp8_cache(build_inputs(batch=2, heads=8, q_len=4, ctx=np.array([70000, 3000]), seed=41,
                               latent_q=True, q_scale=1536.0))
    assert x.block_table.shape[1] > 1024
    d = upload_fp8(x)
    for s in (0, 3):
        check_fp8(x, d, x.q_latent, num_splits=s, what=f"fp8 long S{s}")


@pytest.mark.parametrize("heads,q_len", [(8, 8), (64, 1)])
def test_fp8_noncausal_draft_block_equal_bounds(heads, q_len):
    """fp8 cache, every token of a group sharing one bound (the draft block):
    lengths on, just before and just after page boundaries, odd lengths that
    cut a staged key pair, and an empty request."""
    log(f"fp8 non-causal draft block H={heads} T={q_len}")
    ctx = np.array([1024, 1023, 1025, 64, 1, 0, 701, 1535])
    bounds = np.repeat(ctx[:, None], q_len, axis=1).astype(np.int32)
    x = fp8_cache(build_inputs(batch=len(ctx), heads=heads, q_len=q_len, ctx=ctx, bounds=bounds,
                               seed=33, latent_q=True, q_scale=1536.0))
    d = upload_fp8(x)
    for s in (0, 1, 3):
        check_fp8(x, d, x.q_latent, num_splits=s, what=f"fp8 equal bounds S{s}")
