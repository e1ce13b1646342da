"""The C ABI under hipGraph capture, on side streams, and the documented
split partition for two 32-row tiles.

* Capture: the latent call (TP8-share workload) and the gated call (ragged
  gated workload) are captured into a graph after one eager call, replayed
  twice with unrelated eager work in between, and every replay is compared
  with the oracle and with the eager result, bit for bit.  Calls are
  asynchronous and never synchronise or allocate, which is what the first
  page asks of every captured decode bucket ("Kimi K3 support with DSpark
  speculative decoding", "How was it tested?").
* Streams: a call on a side stream, with the binding allocating outputs and
  workspace on that stream; a raw stream handle without a caller workspace is
  rejected.
* Partition: for 56 folded rows the library takes two 32-row tiles; the
  partials of each tile follow the ranges the header documents.
"""
import numpy as np
import pytest
import torch

import oracle
import speculative_verify_attention_absorbed_amd as mv
from gpu_util import (assert_close_output, assert_lse, assert_masked_rows_zero, bits_of, f64_of,
                      log, round_bf16, sync, upload)
from test_parity_gpu import check_partials_and_combine
from verify_inputs import build_inputs, make_config

pytestmark = pytest.mark.gpu


def oracle_qlat_bits(x):
    return round_bf16(oracle.absorb_query(x.q_nope, x.w_uk))


def _graph_case(cfg, gated):
    x = make_config(cfg)
    q_bits = oracle_qlat_bits(x)
    d = upload(x, q_latent_bits=q_bits)
    b, t, h = x.shape
    params = mv.VerifyParams.make(b, t, h, x.block_table.shape[1], x.pool.num_pages, x.sm_scale,
                                  x.num_splits)
    ws_bytes = mv.verify_workspace_size(params, gated)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    lse = torch.empty((b, t, h), dtype=torch.float32, device="cuda")
    out = torch.empty((b, t, h, 128 if gated else 512), dtype=torch.bfloat16, device="cuda")
    lat = torch.empty((b, t, h, 512), dtype=torch.bfloat16, device="cuda") if gated else None

    def call():
        if gated:
            mv.verify_attn_gated(d["q_latent"], d["pool"], d["block_table"], d["kv_bounds"],
                                 d["w_uv"], d["gate"], x.sm_scale, num_splits=x.num_splits,
                                 out=out, lse=lse, out_latent=lat, workspace=ws)
        else:
            mv.verify_attn(d["q_latent"], d["pool"], d["block_table"], d["kv_bounds"], x.sm_scale,
                           num_splits=x.num_splits, out_latent=out, lse=lse, workspace=ws)
    return x, q_bits, call, out, lse, lat


@pytest.mark.parametrize("cfg,gated", [(2, False), (5, True)])
def test_graph_capture_replay_matches_oracle(cfg, gated):
    log(f"graph capture: config {cfg} gated={gated}")
    x, q_bits, call, out, lse, lat = _graph_case(cfg, gated)
    call()                                   # eager (device set-up happens here)
    sync()
    eager = (bits_of(out).copy(), lse.cpu().numpy().copy())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    sync()
    o_lat, want_lse = oracle.verify_attention_latent(q_bits, x.pool, x.block_table, x.kv_bounds,
                                                     x.sm_scale)
    want = oracle.gated_output(o_lat, x.w_uv, x.gate) if gated else o_lat
    replays = []
    for rep in range(2):
        # eager work between replays: poison the outputs, which the replay
        # must overwrite in full
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        if lat is not None:
            lat.fill_(float("nan"))
        sync()
        g.replay()
        sync()
        got = f64_of(out)
        got_lse = lse.cpu().numpy().astype(np.float64)
        assert_lse(got_lse, want_lse, f"replay {rep} lse")
        assert_masked_rows_zero(got, want_lse, f"replay {rep} out")
        assert_close_output(got, want, f"replay {rep} out")
        if lat is not None:
            assert_close_output(f64_of(lat), o_lat, f"replay {rep} out_latent")
        replays.append((bits_of(out).copy(), lse.cpu().numpy().copy()))
    for r in replays:
        assert np.array_equal(r[0], eager[0]), "replay output differs from the eager call"
        assert np.array_equal(r[1], eager[1], equal_nan=False), "replay lse differs from the eager call"


@pytest.mark.parametrize("cfg,gated", [(3, False), (1, True)])
def test_side_stream_call_allocates_on_its_stream(cfg, gated):
    log(f"side stream: config {cfg} gated={gated}")
    x = make_config(cfg, sharp=True)
    q_bits = oracle_qlat_bits(x)
    d = upload(x, q_latent_bits=q_bits)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    if gated:
        out, lse, lat = mv.verify_attn_gated(d["q_latent"], d["pool"], d["block_table"],
                                             d["kv_bounds"], d["w_uv"], d["gate"], x.sm_scale,
                                             num_splits=x.num_splits, want_latent=True, stream=s)
    else:
        out, lse = mv.verify_attn(d["q_latent"], d["pool"], d["block_table"], d["kv_bounds"],
                                  x.sm_scale, num_splits=x.num_splits, stream=s)
    # other work on the current stream meanwhile: allocations there must not
    # reuse the call's workspace
    junk = [torch.full((1 << 20,), 7.0, device="cuda") for _ in range(8)]
    s.synchronize()
    sync()
    del junk
    o_lat, want_lse = oracle.verify_attention_latent(q_bits, x.pool, x.block_table, x.kv_bounds,
                                                     x.sm_scale)
    want = oracle.gated_output(o_lat, x.w_uv, x.gate) if gated else o_lat
    assert_lse(lse.cpu().numpy().astype(np.float64), want_lse)
    assert_close_output(f64_of(out), want, "side stream out")


def test_raw_stream_handle_needs_caller_workspace():
    log("raw stream handle without a workspace is rejected")
    x = make_config(3)
    q_bits = oracle_qlat_bits(x)
    d = upload(x, q_latent_bits=q_bits)
    s = torch.cuda.Stream()
    with pytest.raises(ValueError, match="workspace"):
        mv.verify_attn(d["q_latent"], d["pool"], d["block_table"], d["kv_bounds"], x.sm_scale,
                       num_splits=4, stream=s.cuda_stream)
    # with its own workspace it runs on that stream
    b, t, h = x.shape
    params = mv.VerifyParams.make(b, t, h, x.block_table.shape[1], x.pool.num_pages, x.sm_scale, 4)
    ws = torch.empty(mv.verify_workspace_size(params), dtype=torch.uint8, device="cuda")
    sync()
    out, lse = mv.verify_attn(d["q_latent"], d["pool"], d["block_table"], d["kv_bounds"],
                              x.sm_scale, num_splits=4, stream=s.cuda_stream, workspace=ws)
    s.synchronize()
    o_lat, want_lse = oracle.verify_attention_latent(q_bits, x.pool, x.block_table, x.kv_bounds,
                                                     x.sm_scale)
    assert_lse(lse.cpu().numpy().astype(np.float64), want_lse)
    assert_close_output(f64_of(out), o_lat, "raw stream out")


@pytest.mark.parametrize("splits", [0, 3, 8])
def test_partials_two_32_row_tiles_follow_documented_ranges(splits):
    """56 folded rows (8 heads, 7 tokens): two 32-row tiles, the second 24
    rows; each tile's splits cover the pages up to its own largest bound."""
    log(f"partials, R=56 two tiles, S={splits}")
    rng = np.random.default_rng(56 + splits)
    ctx = rng.integers(300, 1500, size=4)
    bounds = (ctx[:, None] - 6 + np.arange(7)[None, :]).astype(np.int32)
    bounds[1, 4:] = bounds[1, 3]          # a plateau in the second tile's tokens
    x = build_inputs(batch=4, heads=8, q_len=7, ctx=ctx, bounds=bounds, seed=56, latent_q=True,
                     q_scale=1536.0)
    b, t, h = x.shape
    s_used = splits or mv.verify_num_splits(mv.VerifyParams.make(
        b, t, h, x.block_table.shape[1], x.pool.num_pages, x.sm_scale, 0))
    params = mv.VerifyParams.make(b, t, h, x.block_table.shape[1], x.pool.num_pages, x.sm_scale,
                                  s_used)
    assert mv.verify_tile_rows(params) == 32
    check_partials_and_combine(x, s_used)
