"""Parity of the HIP path (through the C ABI) with the float64 CPU oracle.

Every test prints the case it is about to run, then runs it on cuda:0.
Bars: outputs max-abs <= 1e-2 and relative L2 <= 5e-3; finite LSE within
1e-3; masked rows exactly (-inf, 0); indexing probes bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import speculative_verify_attention_absorbed_amd as mv
from gpu_util import (assert_close_output, assert_lse, assert_masked_rows_zero, bits_of, upload_fp8,
                      bf16_tensor, f64_of, log, rel_l2, round_bf16, sync, upload,
                      upload_dense_pool)
from probes import needle_case, needle_expected
from verify_inputs import SHARP_Q_SCALE, build_inputs, fp8_cache, make_config, ramp_scores

pytestmark = pytest.mark.gpu


def oracle_qlat_bits(x):
    """The ABI input: q_latent = bf16(W_UK^T q_nope) computed in float64."""
    return round_bf16(oracle.absorb_query(x.q_nope, x.w_uk))


def run_latent(x, d, num_splits=None, tile_rows=0):
    s = x.num_splits if num_splits is None else num_splits
    out, lse = mv.verify_attn(d["q_latent"], d["pool"], d["block_table"], d["kv_bounds"],
                              x.sm_scale, num_splits=s, tile_rows=tile_rows)
    sync()
    return f64_of(out), lse.cpu().numpy().astype(np.float64), out


def check_latent(x, d, q_bits, num_splits=None, what="", tile_rows=0):
    got, lse, _ = run_latent(x, d, num_splits, tile_rows)
    want, want_lse = oracle.verify_attention_latent(q_bits, x.pool, x.block_table, x.kv_bounds,
                                                    x.sm_scale)
    assert_lse(lse, want_lse, f"{what} lse")
    assert_masked_rows_zero(got, want_lse, f"{what} out_latent")
    return assert_close_output(got, want, f"{what} out_latent")


# ------------------------------------------------------------------ absorption
@pytest.mark.parametrize("cfg,sharp", [(1, False), (2, False), (2, True), (5, False)])
def test_absorb_q_matches_oracle(cfg, sharp):
    """fp32 accumulation then one bf16 rounding: every element lies within half
    a bf16 ulp plus the fp32 summation bound n * 2^-24 * sum|q_d W_dc| of the
    exact float64 value."""
    log(f"absorb: config {cfg} sharp={sharp}")
    x = make_config(cfg, sharp=sharp)
    d = upload(x)
    q = mv.verify_absorb_q(d["q_nope"], d["w_uk"])
    sync()
    got = f64_of(q)
    want = oracle.absorb_query(x.q_nope, x.w_uk)
    mag = np.einsum("bthd,hdc->bthc", np.abs(oracle.bf16_to_f64(x.q_nope)),
                    np.abs(oracle.bf16_to_f64(x.w_uk)))
    top = np.maximum(np.abs(got), np.abs(want))
    ulp = np.exp2(np.floor(np.log2(np.maximum(top, 1e-38))) - 7)
    allowed = 0.5 * ulp + 128 * 2.0 ** -24 * mag
    excess = np.abs(got - want) - allowed
    assert excess.max() <= 0, f"worst excess {excess.max():.3e}"
    assert rel_l2(got, want) < 5e-3


# ------------------------------------------------------------------ latent ABI
@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
@pytest.mark.parametrize("sharp", [False, True])
def test_latent_parity_configs(cfg, sharp):
    log(f"latent parity: config {cfg} sharp={sharp}")
    x = make_config(cfg, sharp=sharp)
    q_bits = oracle_qlat_bits(x)
    d = upload(x, q_latent_bits=q_bits)
    check_latent(x, d, q_bits, what=f"cfg{cfg}")


def test_latent_parity_config5_full():
    log("latent parity: config 5 (ragged, zero and truncated bounds), S=8")
    x = make_config(5)
    q_bits = oracle_qlat_bits(x)
    d = upload(x, q_latent_bits=q_bits)
    check_latent(x, d, q_bits, what="cfg5")


@pytest.mark.parametrize("cfg", [2, 5])
def test_latent_parity_drifting_scores(cfg):
    """Sharp scores plus a drift of up to ~200 nats along each context
    (ramp_scores): most row tiles meet a score more than 64 (log2) above
    their first unit's maximum, so the item runs the softmax's second pass.
    The drift adds up to ~10 to latent values, so outputs reach that size:
    the max-abs bar applies to outputs divided by their largest magnitude,
    the L2 and LSE bars as stated."""
    log(f"latent parity: config {cfg}, sharp scores drifting along the context")
    x = ramp_scores(make_config(cfg, sharp=True))
    q_bits = oracle_qlat_bits(x)
    d = upload(x, q_latent_bits=q_bits)
    got, lse, _ = run_latent(x, d)
    want, want_lse = oracle.verify_attention_latent(q_bits, x.pool, x.block_table, x.kv_bounds,
                                                    x.sm_scale)
    assert_lse(lse, want_lse, "drift lse")
    assert_masked_rows_zero(got, want_lse, "drift out_latent")
    scale = max(1.0, float(np.abs(want).max()))
    log(f"  output scale {scale:.2f}")
    assert_close_output(got / scale, want / scale, "drift out_latent (scaled)")


@pytest.mark.parametrize("tile", [32, 64, 128])
@pytest.mark.parametrize("cfg,splits", [(3, 4), (2, 8), (4, 2)])
def test_forced_tiles_on_workloads(cfg, tile, splits):
    """Every tile shape on the 8-head workloads (40 or 64 folded rows: one
    partial tile of 128, one or two of 64, two of 32), against the oracle."""
    log(f"forced tile: config {cfg} (sharp), tile {tile}, S={splits}")
    x = make_config(cfg, sharp=True)
    q_bits = oracle_qlat_bits(x)
    d = upload(x, q_latent_bits=q_bits)
    check_latent(x, d, q_bits, num_splits=splits, tile_rows=tile, what=f"tile{tile}")


@pytest.mark.parametrize("splits", [1, 2, 3, 4, 7, 8, 16])
def test_split_invariance(splits):
    log(f"split invariance: config 3 (sharp), S={splits}")
    x = make_config(3, sharp=True)
    q_bits = oracle_qlat_bits(x)
    d = upload(x, q_latent_bits=q_bits)
    check_latent(x, d, q_bits, num_splits=splits, what=f"S={splits}")


@pytest.mark.parametrize("heads,q_len", [(1, 1), (8, 9), (12, 3), (96, 1), (96, 2), (128, 16),
                                         (3, 16), (64, 5)])
def test_fold_shapes(heads, q_len):
    log(f"fold shapes: H={heads} T={q_len}")
    rng = np.random.default_rng(heads * 100 + q_len)
    b = 3
    ctx = rng.integers(q_len, 300, size=b)
    bounds = (ctx[:, None] - (q_len - 1) + np.arange(q_len)[None, :]).astype(np.int32)
    x = build_inputs(batch=b, heads=heads, q_len=q_len, ctx=ctx, bounds=bounds, seed=heads + q_len,
                     latent_q=True, q_scale=1536.0)
    d = upload(x)
    for s in (1, 3):
        for tile in (0, 32, 64, 128):
            check_latent(x, d, x.q_latent, num_splits=s, tile_rows=tile,
                         what=f"H{heads}T{q_len}S{s}tile{tile}")


@pytest.mark.parametrize("batch,splits", [(1, 7), (3, 5), (5, 3), (7, 8), (9, 16), (13, 6)])
def test_combine_rows_by_xcd_cover_every_request(batch, splits):
    # the combine after the contiguous layout takes each request on the die
    # that ran its first split: batch * splits not a multiple of 8 leaves
    # dies with no request and requests straddling two dies' groups
    log(f"combine by die: B={batch} S={splits}")
    rng = np.random.default_rng(batch * 31 + splits)
    ctx = rng.integers(4, 1200, size=batch)
    bounds = (ctx[:, None] - 3 + np.arange(4)[None, :]).astype(np.int32)
    x = build_inputs(batch=batch, heads=8, q_len=4, ctx=ctx, bounds=bounds, seed=batch + splits,
                     latent_q=True, q_scale=1536.0)
    d = upload(x)
    check_latent(x, d, x.q_latent, num_splits=splits, what=f"B{batch}S{splits}")


@pytest.mark.parametrize("batch", [13, 40, 64])
def test_dealt_grid_of_several_rounds(batch):
    # 128-row tiles, four per request, more workgroups than CUs (the dealt
    # layout): ties, a request with no visible key and a padded last slot
    # must still map every (request, split, row tile) exactly once
    log(f"dealt grid: B={batch} H=64 T=8 S=8")
    rng = np.random.default_rng(batch)
    ctx = rng.integers(8, 600, size=batch)
    ctx[::5] = ctx[0]                      # ties
    bounds = (ctx[:, None] - 7 + np.arange(8)[None, :]).astype(np.int32)
    bounds[3] = 0                          # a request with no visible key
    x = build_inputs(batch=batch, heads=64, q_len=8, ctx=ctx, bounds=bounds, seed=batch,
                     latent_q=True, q_scale=1536.0)
    d = upload(x)
    check_latent(x, d, x.q_latent, num_splits=8, what=f"B{batch}")


def test_long_context_block_table_past_one_split_staging():
    """A block-table row longer than one split stages in LDS (1024 page ids):
    each split then loads only its own slice of the row.  70000 keys = 1094
    pages; the library's split count, a forced 2 (547 pages per split) and 3,
    and the rejection of a forced single split (1094 > 1024 pages)."""
    log("long context: B=2 ctx=(70000, 3000) H=8 T=4")
    q_len = 4
    ctx = np.array([70000, 3000])
    x = build_inputs(batch=2, heads=8, q_len=q_len, ctx=ctx, seed=41, latent_q=True, q_scale=1536.0)
    assert x.block_table.shape[1] > 1024
    d = upload(x)
    for s in (0, 2, 3):
        check_latent(x, d, x.q_latent, num_splits=s, what=f"long S{s}")
    with pytest.raises(mv.MlaVerifyError) as e:
        mv.verify_attn(d["q_latent"], d["pool"], d["block_table"], d["kv_bounds"], x.sm_scale,
                       num_splits=1)
    assert e.value.code == -4


@pytest.mark.parametrize("heads,q_len", [(8, 8), (64, 8), (64, 1)])
def test_noncausal_draft_block_equal_bounds(heads, q_len):
    """The drafter's own attention: every token of a group shares
    one bound, so masking is needed only in a request's last page.  Lengths
    land on, just before and just after page boundaries; one request sees
    nothing."""
    log(f"non-causal draft block H={heads} T={q_len}")
    ctx = np.array([1024, 1023, 1025, 64, 1, 0, 700, 1536])
    bounds = np.repeat(ctx[:, None], q_len, axis=1).astype(np.int32)
    x = build_inputs(batch=len(ctx), heads=heads, q_len=q_len, ctx=ctx, bounds=bounds, seed=33,
                     latent_q=True, q_scale=1536.0)
    d = upload(x)
    for s in (0, 1, 3):
        check_latent(x, d, x.q_latent, num_splits=s, what=f"equal bounds S{s}")


def test_random_bounds_zero_rows_and_empty_requests():
    log("random bounds incl. zero rows, an all-zero request, bounds past the table")
    rng = np.random.default_rng(5)
    b, t, h = 5, 6, 8
    ctx = np.array([200, 1, 0, 333, 64])
    bounds = np.stack([rng.integers(0, c + 1, size=t) for c in ctx]).astype(np.int32)
    bounds[2] = 0                          # a request with nothing visible
    bounds[0, 0] = 0
    bounds[4] = [64, 0, 64, 1, 63, 64]
    x = build_inputs(batch=b, heads=h, q_len=t, ctx=ctx, bounds=bounds, seed=9, latent_q=True,
                     q_scale=1536.0)
    d = upload(x)
    for s in (0, 1, 2, 5):
        check_latent(x, d, x.q_latent, num_splits=s, what=f"S{s}")
    for tile in (32, 128):
        check_latent(x, d, x.q_latent, num_splits=2, tile_rows=tile, what=f"S2 tile{tile}")
    # the 128-row kernel writing the outputs itself (one split), the all-zero
    # request included (an item with no unit to stage)
    check_latent(x, d, x.q_latent, num_splits=1, tile_rows=128, what="S1 tile128")
    # bounds beyond max_pages*64 are clamped to it
    big = bounds.copy()
    big[3, 0] = 10_000_000
    x2 = build_inputs(batch=b, heads=h, q_len=t, ctx=ctx, bounds=np.minimum(big, 384),
                      seed=9, latent_q=True, q_scale=1536.0)
    d2 = upload(x2)
    d2["kv_bounds"] = torch.from_numpy(big).cuda()
    out, lse = mv.verify_attn(d2["q_latent"], d2["pool"], d2["block_table"], d2["kv_bounds"],
                              x2.sm_scale, num_splits=1)
    sync()
    want, want_lse = oracle.verify_attention_latent(x2.q_latent, x2.pool, x2.block_table, big,
                                                    x2.sm_scale)
    assert_lse(lse.cpu().numpy().astype(np.float64), want_lse)
    assert_close_output(f64_of(out), want, "clamped bounds")


# ------------------------------------------------------------------ probes
@pytest.mark.parametrize("splits", [1, 2, 4])
def test_needle_probe_bit_exact(splits):
    log(f"needle probe, S={splits}")
    bounds = np.array([[1, 64, 65, 63], [129, 100, 128, 2], [0, 200, 255, 192],
                       [255, 254, 253, 129]], np.int32)
    x, pool, q, bounds = needle_case(bounds, heads=2)
    want = needle_expected(x, bounds)
    out, lse = mv.verify_attn(bf16_tensor(q), upload_dense_pool(pool),
                              torch.from_numpy(x.block_table).cuda(),
                              torch.from_numpy(bounds).cuda(), 1.0, num_splits=splits)
    sync()
    got = f64_of(out)
    lse = lse.cpu().numpy()
    for bb in range(bounds.shape[0]):
        for t in range(bounds.shape[1]):
            for h in range(2):
                assert np.array_equal(got[bb, t, h], want[bb, t]), (bb, t, h, got[bb, t, h, :6])
                assert lse[bb, t, h] == (0.0 if bounds[bb, t] > 0 else -np.inf)


def test_page_permutation_bit_identical():
    log("page permutation: config 2 pages moved, outputs bit-identical")
    x = make_config(2, sharp=True)
    q_bits = oracle_qlat_bits(x)
    d = upload(x, q_latent_bits=q_bits)
    _, lse1, out1 = run_latent(x, d, num_splits=4)
    perm = np.random.default_rng(3).permutation(x.pool.num_pages)
    x2 = make_config(2, sharp=True)
    x2.pool = x.pool.remap(perm)
    x2.block_table = np.where(x.block_table >= 0, perm[np.maximum(x.block_table, 0)],
                              -1).astype(np.int32)
    d2 = upload(x2, q_latent_bits=q_bits)
    _, lse2, out2 = run_latent(x2, d2, num_splits=4)
    assert np.array_equal(bits_of(out1), bits_of(out2))
    assert np.array_equal(lse1, lse2)


def test_deterministic_repeat():
    log("determinism: config 3 run twice")
    x = make_config(3, sharp=True)
    q_bits = oracle_qlat_bits(x)
    d = upload(x, q_latent_bits=q_bits)
    _, l1, o1 = run_latent(x, d)
    _, l2, o2 = run_latent(x, d)
    assert np.array_equal(bits_of(o1), bits_of(o2)) and np.array_equal(l1, l2)


def test_nan_pool_outside_visible_keys_is_ignored():
    log("NaN poison: every unreferenced page and slot past the bounds is NaN")
    x = make_config(2)
    q_bits = oracle_qlat_bits(x)
    d = upload(x, q_latent_bits=q_bits)
    assert torch.isnan(d["pool"].float()).any()
    got, lse, _ = run_latent(x, d)
    assert np.all(np.isfinite(got)) and not np.isnan(lse).any()


# ------------------------------------------------------------------ gated epilogue
def check_gated(x, d, q_bits, num_splits=None, requests=None, what="", tile_rows=0):
    s = x.num_splits if num_splits is None else num_splits
    out, lse, lat = mv.verify_attn_gated(d["q_latent"], d["pool"], d["block_table"],
                                         d["kv_bounds"], d["w_uv"], d["gate"], x.sm_scale,
                                         num_splits=s, want_latent=True, tile_rows=tile_rows)
    sync()
    o_lat, want_lse = oracle.verify_attention_latent(q_bits, x.pool, x.block_table, x.kv_bounds,
                                                     x.sm_scale)
    want = oracle.gated_output(o_lat, x.w_uv, x.gate)
    got = f64_of(out)
    assert_lse(lse.cpu().numpy().astype(np.float64), want_lse, f"{what} lse")
    assert_masked_rows_zero(got, want_lse, f"{what} out")
    assert_close_output(got, want, f"{what} gated out")
    assert_close_output(f64_of(lat), o_lat, f"{what} gated out_latent")


@pytest.mark.parametrize("cfg,splits,tile", [(1, 1, 0), (1, 2, 0), (3, 4, 0), (5, 8, 0),
                                            (1, 2, 128), (3, 4, 32), (5, 0, 0), (5, 8, 64)])
def test_gated_parity(cfg, splits, tile):
    log(f"gated parity: config {cfg}, S={splits}, tile {tile}")
    x = make_config(cfg, sharp=(cfg != 5))
    q_bits = oracle_qlat_bits(x)
    d = upload(x, q_latent_bits=q_bits)
    check_gated(x, d, q_bits, num_splits=splits, what=f"cfg{cfg}", tile_rows=tile)


@pytest.mark.parametrize("splits,heads", [(24, 8), (64, 8), (24, 9), (64, 9)])
def test_gated_many_splits(splits, heads):
    """More than 16 splits per row, so the gated epilogue takes 32 or 64
    lanes per row: 64 folded rows (two 32-row tiles) and 72 (one 128-row
    tile), a 20000-key request beside a short one and one that sees
    nothing."""
    log(f"gated parity: S={splits}, H={heads}, T=8, ctx (20000, 3000, 0)")
    ctx = np.array([20000, 3000, 0])
    bounds = (ctx[:, None] - 7 + np.arange(8)[None, :]).clip(0).astype(np.int32)
    x = build_inputs(batch=3, heads=heads, q_len=8, ctx=ctx, bounds=bounds, seed=61,
                     q_scale=SHARP_Q_SCALE)
    q_bits = oracle_qlat_bits(x)
    d = upload(x, q_latent_bits=q_bits)
    check_gated(x, d, q_bits, num_splits=splits, what=f"S{splits} H{heads}")


@pytest.mark.parametrize("batch,q_len,heads", [(5, 14, 3), (13, 10, 128)])
def test_absorb_q_ragged_tiles(batch, q_len, heads):
    """Row counts that leave a partial 64-row tile, on both column blockings
    (quarters for a small batch, whole rows once the (head, tile) pairs fill
    the GPU: 3 tiles x 128 heads)."""
    log(f"absorb: B={batch} T={q_len} H={heads}")
    x = build_inputs(batch=batch, heads=heads, q_len=q_len, ctx=np.full(batch, 40), seed=31)
    d = upload(x)
    got = bits_of(mv.verify_absorb_q(d["q_nope"], d["w_uk"]))
    sync()
    want = oracle.absorb_query(x.q_nope, x.w_uk)
    # fp32 sum then one bf16 rounding: within half a bf16 ulp plus the fp32
    # summation bound n * 2^-24 * sum|q_d W_dc| of the float64 value
    g = oracle.bf16_to_f64(got)
    mag = np.einsum("bthd,hdc->bthc", np.abs(oracle.bf16_to_f64(x.q_nope)),
                    np.abs(oracle.bf16_to_f64(x.w_uk)))
    top = np.maximum(np.abs(g), np.abs(want))
    ulp = np.exp2(np.floor(np.log2(np.maximum(top, 1e-38))) - 7)
    excess = np.abs(g - want) - (0.5 * ulp + 128 * 2.0 ** -24 * mag)
    assert np.all(excess <= 0), float(excess.max())


# ------------------------------------------------------------------ end to end
@pytest.mark.parametrize("cfg", [1, 2])
def test_end_to_end_against_unabsorbed_oracle(cfg):
    """HIP absorption + HIP attention (+ gated epilogue) against the oracle's
    primary, unabsorbed definition (explicit per-head K/V up-projection)."""
    log(f"end to end vs unabsorbed oracle: config {cfg}")
    x = make_config(cfg)
    d = upload(x)
    q_lat = mv.verify_absorb_q(d["q_nope"], d["w_uk"])
    out_lat, lse = mv.verify_attn(q_lat, d["pool"], d["block_table"], d["kv_bounds"], x.sm_scale)
    out, lse_g, _ = mv.verify_attn_gated(q_lat, d["pool"], d["block_table"], d["kv_bounds"],
                                         d["w_uv"], d["gate"], x.sm_scale)
    sync()
    r = oracle.verify_attention_mla(x.q_nope, x.w_uk, x.w_uv, x.gate, x.pool, x.block_table,
                                    x.kv_bounds, x.sm_scale)
    assert_lse(lse.cpu().numpy().astype(np.float64), r["lse"])
    assert_lse(lse_g.cpu().numpy().astype(np.float64), r["lse"])
    assert_close_output(f64_of(out_lat), r["o_lat"], "o_lat")
    assert_close_output(f64_of(out), r["out"], "gated out")
    assert rel_l2(f64_of(out), r["out"]) < 5e-3


def test_unknown_kv_dtype_raises():
    log("unknown KV dtype is rejected")
    x = make_config(1)
    d = upload(x, q_latent_bits=oracle_qlat_bits(x))
    with pytest.raises(mv.MlaVerifyError, match="MLA_ERR_DTYPE"):
        mv.verify_attn(d["q_latent"], d["pool"], d["block_table"], d["kv_bounds"], x.sm_scale,
                       kv_dtype=5)


# ------------------------------------------------ partials + combine entry points
def library_split_count(n_keys, num_splits, max_pages):
    """The library's split rule for one row tile (the rule the header documents
    for mla_verify_attn_partials): the n_pg pages up to the tile's largest
    bound go to S' = min(S, ceil(n_pg / m)) balanced splits, m = max(1,
    ceil(P / S) // 2); splits s >= S' are empty."""
    n_pg = -(-n_keys // 64)
    m = max(1, (-(-max_pages // num_splits)) // 2)
    return min(num_splits, max(1, -(-n_pg // m)))


ITEM_UNITS = 6   # MLA_VERIFY_ITEM_UNITS


def balanced_chunks(x, splits, tile):
    """Key ranges of every partial slot under the balanced-chunk partition the
    header documents for 128-row tiles on a bf16 cache (split count >= 2):
    request b has U_b = ceil(n_b / 32) units, n_b its largest bound, and
    takes V_b = U_b + F positions (0 if U_b = 0), its units after the first
    F; the requests' positions end to end are cut into chunks of
    C = max(ceil(V / g), ceil(2 P / (S - 1))), g = 8 * floor(32 / row tiles);
    slot j of request b is its part of chunk floor((start_b + F) / C) + j.
    Returns {b: [(k0, k1), ...]} in request keys (before each tile's own
    clip)."""
    b_n, t, h = x.shape
    max_pages = x.block_table.shape[1]
    n_b = np.clip(x.kv_bounds, 0, max_pages * 64).max(axis=1)
    units = [-(-int(n) // 32) for n in n_b]
    spans = [u + ITEM_UNITS if u > 0 else 0 for u in units]
    starts = np.concatenate([[0], np.cumsum(spans)]).astype(int)
    total = int(starts[-1])
    row_tiles = -(-(t * h) // tile)
    groups = 8 * (32 // row_tiles)
    c = max(-(-total // groups), -(-(2 * max_pages) // (splits - 1)))
    g_used = max(1, -(-total // c))
    out = {}
    for bi in range(b_n):
        st, ub = int(starts[bi]) + ITEM_UNITS, units[bi]
        rng = []
        if ub > 0:
            q0, q1 = st // c, (st + ub - 1) // c
            for q in range(q0, q1 + 1):
                lo = q * c
                hi = float("inf") if q == g_used - 1 else lo + c
                rng.append((max(lo, st) - st, min(hi, st + ub) - st))
        assert len(rng) <= splits
        out[bi] = [(a * 32, b_ * 32) for a, b_ in rng]
    return out


def check_partials_and_combine(x, splits, tile_rows=0, requests=None):
    """mla_verify_attn_partials: split s of a row is attention over the keys of
    chunk s of its row tile's partition (clipped to the row's token bound);
    mla_verify_lse_combine of those partials gives the same bits as
    mla_verify_attn with the same split count and tile.  An fp8 cache
    (x.kv_dtype == "fp8", inputs from verify_inputs.fp8_cache) is uploaded as
    its codes and decoded by the oracle with its scale."""
    q_bits = oracle_qlat_bits(x)
    fp8 = getattr(x, "kv_dtype", "bf16") == "fp8"
    d = upload_fp8(x, q_latent_bits=q_bits) if fp8 else upload(x, q_latent_bits=q_bits)
    kv = dict(kv_dtype=mv.KV_FP8_E4M3, kv_scale=x.kv_scale) if fp8 else {}
    decode = oracle.kv_decoder("fp8", x.kv_scale) if fp8 else None
    part_o, part_lse = mv.verify_attn_partials(d["q_latent"], d["pool"], d["block_table"],
                                               d["kv_bounds"], x.sm_scale, num_splits=splits,
                                               tile_rows=tile_rows, **kv)
    out, lse = mv.verify_attn(d["q_latent"], d["pool"], d["block_table"], d["kv_bounds"],
                              x.sm_scale, num_splits=splits, tile_rows=tile_rows, **kv)
    b, t, h = x.shape
    comb, comb_lse = mv.verify_lse_combine(part_o, part_lse)
    sync()
    assert np.array_equal(bits_of(comb), bits_of(out).reshape(b * t * h, 512))
    assert np.array_equal(comb_lse.cpu().numpy(), lse.cpu().numpy().reshape(-1))

    params = mv.VerifyParams.make(b, t, h, x.block_table.shape[1], x.pool.num_pages, x.sm_scale,
                                  splits, tile_rows=tile_rows, **kv)
    tile = mv.verify_tile_rows(params)
    po = f64_of(part_o).reshape(splits, b, t * h, 512)
    pl = part_lse.cpu().numpy().astype(np.float64).reshape(splits, b, t * h)
    q = oracle.bf16_to_f64(q_bits).reshape(b, t * h, 512)
    max_pages = x.block_table.shape[1]
    want_o, want_l, got_o, got_l = [], [], [], []
    n_empty = 0
    balanced = tile == 128 and splits >= 2 and b <= 2000 and max_pages <= 1024
    bal = balanced_chunks(x, splits, tile) if balanced else None
    for bi in (range(b) if requests is None else requests):
        c_b, n_b = oracle.request_keys(x.pool, x.block_table, x.kv_bounds, bi, decode)
        for r0 in range(0, t * h, tile):
            rows = range(r0, min(r0 + tile, t * h))
            # the tile sees the keys up to its own largest bound
            n_tile = max(oracle.token_bound(x.kv_bounds, bi, r // h, n_b) for r in rows)
            if balanced:
                chunks = [(min(k0, n_tile), min(k1, n_tile)) for k0, k1 in bal[bi]]
                chunks += [(n_tile, n_tile)] * (splits - len(chunks))
            else:
                used = library_split_count(n_tile, splits, max_pages)
                chunks = oracle.split_pages(n_tile, used) + [(n_tile, n_tile)] * (splits - used)
            for s, (k0, k1) in enumerate(chunks):
                for r in rows:
                    L = oracle.token_bound(x.kv_bounds, bi, r // h, n_b)
                    hi = min(k1, L)
                    o, l = oracle.attend_chunk(q[bi, r], c_b[k0:max(k0, hi)], x.sm_scale)
                    if l == -np.inf:
                        assert pl[s, bi, r] == -np.inf, (s, bi, r)
                        n_empty += 1
                        continue
                    want_o.append(o)
                    want_l.append(l)
                    got_o.append(po[s, bi, r])
                    got_l.append(pl[s, bi, r])
    assert_close_output(np.array(got_o), np.array(want_o), "partials")
    assert np.abs(np.array(got_l) - np.array(want_l)).max() <= 1e-3
    return n_empty


@pytest.mark.parametrize("cfg,splits,tile", [(3, 4, 0), (2, 5, 0), (2, 5, 64), (3, 3, 128),
                                            (1, 4, 0)])
def test_partials_match_oracle_chunks_and_combine_matches_call(cfg, splits, tile):
    log(f"partials + combine: config {cfg} sharp, S={splits}, tile {tile}")
    check_partials_and_combine(make_config(cfg, sharp=True), splits, tile)


@pytest.mark.parametrize("splits,kv", [(2, "bf16"), (3, "bf16"), (8, "bf16"), (3, "fp8"),
                                       (8, "fp8")])
def test_partials_balanced_chunks_on_128_row_tiles(splits, kv):
    """128-row tiles (64 heads x 8 tokens: four tiles per request) on a bf16
    or an fp8 cache: the balanced-chunk partition, with a request that sees
    nothing, a request whose later tokens see nothing (a tile shorter than
    the request), lengths on and off unit, pair and page edges, and forced
    split counts that bind the chunk size (2, 3) or not (8)."""
    log(f"partials, balanced chunks, S={splits}, {kv} cache")
    ctx = np.array([2000, 0, 33, 1500, 64, 4100, 95, 1])
    bounds = (ctx[:, None] - 7 + np.arange(8)[None, :]).clip(0).astype(np.int32)
    bounds[3, 2:] = 0                      # tiles 1..3 of request 3 see nothing
    bounds[6, :4] = 0
    x = build_inputs(batch=len(ctx), heads=64, q_len=8, ctx=ctx, bounds=bounds, seed=77,
                     latent_q=True, q_scale=1536.0)
    if kv == "fp8":
        x = fp8_cache(x)
    check_partials_and_combine(x, splits, tile_rows=128)


def test_more_than_2000_requests_take_per_tile_splits_on_128_row_tiles():
    """Past 2000 requests the 128-row kernel deals per-tile splits instead of
    balanced chunks: 2001 requests of 72 folded rows (one partial tile each)
    under S = 3, some seeing nothing.  The call against the oracle on every
    row; combine == call bit for bit; the page ranges of a sample of requests'
    partials as the per-tile rule states them."""
    log("2001 requests x 72 rows, S=3, 128-row tiles: per-tile splits")
    rng = np.random.default_rng(2001)
    b, h, t = 2001, 9, 8
    ctx = rng.integers(1, 200, size=b)
    bounds = (ctx[:, None] - (t - 1) + np.arange(t)[None, :]).clip(0).astype(np.int32)
    bounds[::37] = 0                                    # requests that see nothing
    x = build_inputs(batch=b, heads=h, q_len=t, ctx=ctx, bounds=bounds, seed=2001,
                     latent_q=True, q_scale=1536.0)
    params = mv.VerifyParams.make(b, t, h, x.block_table.shape[1], x.pool.num_pages, x.sm_scale, 3)
    assert mv.verify_tile_rows(params) == 128
    check_partials_and_combine(x, 3, tile_rows=0, requests=range(0, b, 97))
    d = upload(x)   # the drawn q_latent
    out, lse = mv.verify_attn(d["q_latent"], d["pool"], d["block_table"], d["kv_bounds"],
                              x.sm_scale, num_splits=3)
    sync()
    want_o, want_lse = oracle.verify_attention_latent(x.q_latent, x.pool, x.block_table,
                                                      x.kv_bounds, x.sm_scale)
    got = f64_of(out)
    assert_lse(lse.cpu().numpy().astype(np.float64), want_lse, "2001 requests lse")
    assert_masked_rows_zero(got, want_lse, "2001 requests out_latent")
    assert_close_output(got, want_o, "2001 requests out_latent")


@pytest.mark.parametrize("splits", [0, 2, 3])
def test_long_block_table_row_on_128_row_tiles(splits):
    """A block-table row longer than a workgroup stages (70000 keys = 1094
    pages) with 72 folded rows per request: the 128-row kernel takes per-tile
    splits, each staging its own slice of the row.  The call against the
    oracle; with S = 2 and 3, also the partials over the per-tile page ranges
    and their combine against the call."""
    log(f"long block-table row, 72 rows, 128-row tiles, S={splits}")
    x = build_inputs(batch=2, heads=9, q_len=8, ctx=np.array([70000, 3000]), seed=43,
                     latent_q=True, q_scale=1536.0)
    assert x.block_table.shape[1] > 1024
    d = upload(x)
    out, lse = mv.verify_attn(d["q_latent"], d["pool"], d["block_table"], d["kv_bounds"],
                              x.sm_scale, num_splits=splits)
    sync()
    want_o, want_lse = oracle.verify_attention_latent(x.q_latent, x.pool, x.block_table,
                                                      x.kv_bounds, x.sm_scale)
    got = f64_of(out)
    assert_lse(lse.cpu().numpy().astype(np.float64), want_lse, f"long row S{splits} lse")
    assert_close_output(got, want_o, f"long row S{splits} out_latent")
    if splits:
        del d
        check_partials_and_combine(x, splits, tile_rows=128)


def test_partials_ragged_batch_takes_fewer_splits_for_short_requests():
    """Requests of 2 to 63 pages under S = 8 with a 64-page block-table
    stride (m = 4): the short ones use 1, 2 or 4 splits, the rest are empty."""
    log("partials + combine: ragged batch, S=8")
    ctx = np.array([100, 300, 900, 2500, 4000, 64 * 63 - 5])
    x = build_inputs(batch=6, heads=8, q_len=8, ctx=ctx, max_pages=64, pool_pages=512,
                     seed=5, gated=False)
    used = [library_split_count(int(c), 8, 64) for c in ctx]
    assert used == [1, 2, 4, 8, 8, 8]
    n_empty = check_partials_and_combine(x, 8, tile_rows=64)
    assert n_empty >= (7 + 6 + 4) * 8 * 8
