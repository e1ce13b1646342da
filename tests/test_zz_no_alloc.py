"""mla_verify_attn_gated_noalloc, the gated call without a workspace argument
(for callers that cannot allocate: hipGraph capture, tight serving loops).

Two calls in a row through the C ABI, the second on a smaller batch, each
against mla_verify_attn_gated with its own workspace (same kernels and plan,
so bit-identical) and against the oracle; the second call finds the first
call's partials in the scratch.  A plan whose workspace exceeds the scratch
is rejected on the host.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import speculative_verify_attention_absorbed_amd as mv
from gpu_util import (assert_close_output, assert_lse, assert_masked_rows_zero, bits_of, f64_of,
                      log, round_bf16, sync, upload)
from verify_inputs import make_config

pytestmark = pytest.mark.gpu


def _case(cfg, sharp, want_latent):
    x = make_config(cfg, sharp=sharp)
    q_bits = round_bf16(oracle.absorb_query(x.q_nope, x.w_uk))
    d = upload(x, q_latent_bits=q_bits)
    b, t, h = x.shape
    dev = torch.device("cuda")
    out = torch.empty((b, t, h, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((b, t, h), dtype=torch.float32, device=dev)
    lat = torch.empty((b, t, h, 512), dtype=torch.bfloat16, device=dev) if want_latent else None
    mv.verify_attn_gated_noalloc(d["q_latent"], d["pool"], d["block_table"], d["kv_bounds"],
                                 d["w_uv"], d["gate"], x.sm_scale, out, lse, out_latent=lat,
                                 num_splits=x.num_splits)
    ref_out, ref_lse, ref_lat = mv.verify_attn_gated(
        d["q_latent"], d["pool"], d["block_table"], d["kv_bounds"], d["w_uv"], d["gate"],
        x.sm_scale, num_splits=x.num_splits, want_latent=want_latent)
    sync()
    assert np.array_equal(bits_of(out), bits_of(ref_out)), "out differs from the workspace call"
    assert np.array_equal(lse.cpu().numpy(), ref_lse.cpu().numpy()), "lse differs"
    o_lat, want_lse = oracle.verify_attention_latent(q_bits, x.pool, x.block_table, x.kv_bounds,
                                                     x.sm_scale)
    want = oracle.gated_output(o_lat, x.w_uv, x.gate)
    got = f64_of(out)
    assert_lse(lse.cpu().numpy().astype(np.float64), want_lse, f"cfg{cfg} lse")
    assert_masked_rows_zero(got, want_lse, f"cfg{cfg} out")
    assert_close_output(got, want, f"cfg{cfg} noalloc out")
    if want_latent:
        assert np.array_equal(bits_of(lat), bits_of(ref_lat))
        assert_close_output(f64_of(lat), o_lat, f"cfg{cfg} noalloc out_latent")


def test_two_calls_second_smaller():
    log("no-alloc gated call: config 2 inputs (8.4 MB of partials), then config 1")
    _case(2, True, True)
    _case(1, False, False)
    _case(2, False, False)


def test_plan_larger_than_scratch_is_rejected_on_host():
    log("no-alloc gated call: a plan needing more than the scratch")
    lib = mv.load_library()
    # 64 requests x 64 heads x 8 tokens with 8 splits: 269 MB of partials
    p = mv.VerifyParams.make(64, 8, 64, 128, 16384, 0.088, 8)
    assert mv.verify_workspace_size(p, True) > mv.STATIC_SCRATCH_BYTES
    fake = ctypes.c_void_p(256)          # aligned, never dereferenced: rejected first
    rc = lib.mla_verify_attn_gated_noalloc(ctypes.byref(p), fake, fake, fake, fake, fake, fake,
                                           fake, fake, None, None)
    assert rc == -5
