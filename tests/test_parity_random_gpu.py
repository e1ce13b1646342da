"""Seeded random shapes through the HIP path, checked against the float64 oracle.

Each case draws its batch, head count, group size, per-request contexts,
per-token bounds (a few fully masked tokens and truncated groups among them),
split count, tile and entry point from its own seed, so that combinations the
named workloads do not reach (odd head counts, groups of up to 16 tokens,
ragged tails of every tile, forced split counts that leave splits empty) are
covered too.  Bars as in test_parity_gpu.py.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import speculative_verify_attention_absorbed_amd as mv
from gpu_util import (assert_close_output, assert_lse, assert_masked_rows_zero, bf16_tensor, f64_of,
                      log, sync, upload)
from verify_inputs import FP8_KV_SCALE, FP8_NAN, build_inputs, fp8_cache

pytestmark = pytest.mark.gpu

HEADS = [1, 3, 5, 8, 12, 16, 24, 64, 96, 128]


def draw_case(seed):
    rng = np.random.default_rng(1000 + seed)
    heads = int(rng.choice(HEADS))
    q_len = int(rng.integers(1, 17))
    rows = heads * q_len
    # keep the oracle's work (batch x rows x keys) to about a second
    max_ctx = int(min(2000, max(q_len + 64, 6_000_000 // (rows * 4))))
    batch = int(rng.integers(1, 1 + max(1, min(12, 6_000_000 // (rows * max_ctx)))))
    ctx = rng.integers(q_len, max_ctx + 1, size=batch)
    bounds = (ctx[:, None] - (q_len - 1) + np.arange(q_len)[None, :]).astype(np.int32)
    flat = bounds.reshape(-1)
    pick = rng.random(flat.size)
    flat[pick < 0.08] = 0                                        # fully masked tokens
    trunc = (pick >= 0.08) & (pick < 0.16)
    flat[trunc] = (flat[trunc] * rng.random(int(trunc.sum()))).astype(np.int32)   # truncated
    splits = int(rng.choice([0, 1, 2, 3, 5, 8, 13]))
    tile = int(rng.choice([0, 0, 32, 64, 128]))
    gated = bool(rng.random() < 0.5)
    kv = "fp8" if rng.random() < 1 / 3 else "bf16"
    want_latent = bool(rng.random() < 0.5)
    return dict(batch=batch, heads=heads, q_len=q_len, ctx=ctx, bounds=bounds, splits=splits,
                tile=tile, gated=gated, kv=kv, want_latent=want_latent)


def upload_case(x):
    """Device inputs; an fp8 cache goes up as its E4M3 codes (NaN code elsewhere)."""
    if x.kv_dtype != "fp8":
        return upload(x)
    dev = torch.device("cuda:0")
    pool = torch.full((x.pool.num_pages, 64, 512), int(FP8_NAN), dtype=torch.uint8, device=dev)
    if x.pool.page_ids.size:
        pool[torch.from_numpy(x.pool.page_ids.astype(np.int64)).to(dev)] = \
            torch.from_numpy(np.ascontiguousarray(x.pool.pages)).to(dev)
    return {"pool": pool, "block_table": torch.from_numpy(x.block_table).to(dev),
            "kv_bounds": torch.from_numpy(x.kv_bounds).to(dev), "w_uv": bf16_tensor(x.w_uv),
            "gate": bf16_tensor(x.gate), "q_latent": bf16_tensor(x.q_latent)}


# MLA_RANDOM_CASES widens the draw (48 cases by default, about half a minute)
@pytest.mark.parametrize("seed", range(int(os.environ.get("MLA_RANDOM_CASES", "48"))))
def test_random_shapes_match_oracle(seed):
    c = draw_case(seed)
    what = (f"seed {seed}: B={c['batch']} H={c['heads']} T={c['q_len']} "
            f"max ctx {int(c['ctx'].max())} S={c['splits']} tile {c['tile']} "
            f"{'gated' if c['gated'] else 'latent'} {c['kv']} cache")
    log(f"random shapes, {what}")
    x = build_inputs(batch=c["batch"], heads=c["heads"], q_len=c["q_len"], ctx=c["ctx"],
                     bounds=c["bounds"], seed=seed, latent_q=True, q_scale=1536.0)
    if c["kv"] == "fp8":
        x = fp8_cache(x, FP8_KV_SCALE)
    d = upload_case(x)
    kv = dict(kv_dtype=mv.KV_FP8_E4M3 if c["kv"] == "fp8" else mv.KV_BF16, kv_scale=x.kv_scale)
    o_lat, want_lse = oracle.verify_attention_latent(x.q_latent, x.pool, x.block_table,
                                                     x.kv_bounds, x.sm_scale, kv_dtype=x.kv_dtype,
                                                     kv_scale=x.kv_scale)
    if c["gated"]:
        out, lse, lat = mv.verify_attn_gated(d["q_latent"], d["pool"], d["block_table"],
                                             d["kv_bounds"], d["w_uv"], d["gate"], x.sm_scale,
                                             num_splits=c["splits"],
                                             want_latent=c["want_latent"], tile_rows=c["tile"],
                                             **kv)
        sync()
        want = oracle.gated_output(o_lat, x.w_uv, x.gate)
        got = f64_of(out)
        assert_lse(lse.cpu().numpy().astype(np.float64), want_lse, f"{what} lse")
        assert_masked_rows_zero(got, want_lse, f"{what} out")
        assert_close_output(got, want, f"{what} gated out")
        if c["want_latent"]:
            assert_close_output(f64_of(lat), o_lat, f"{what} out_latent")
        else:
            assert lat is None
    else:
        out, lse = mv.verify_attn(d["q_latent"], d["pool"], d["block_table"], d["kv_bounds"],
                                  x.sm_scale, num_splits=c["splits"], tile_rows=c["tile"], **kv)
        sync()
        got = f64_of(out)
        assert_lse(lse.cpu().numpy().astype(np.float64), want_lse, f"{what} lse")
        assert_masked_rows_zero(got, want_lse, f"{what} out_latent")
        assert_close_output(got, o_lat, f"{what} out_latent")
