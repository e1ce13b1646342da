"""Parity of the KV append and trim kernels (through the C ABI) with the CPU
oracle.  Everything here is integer or bit-pattern work, so the bar is
bit-exact.  Every test prints its case before it touches the GPU."""
import numpy as np
import pytest
import torch

import oracle
from oracle import kv_update as ku
import speculative_verify_attention_absorbed_amd as mv
from gpu_util import (assert_close_output, assert_lse, bf16_tensor, bits_of, dev, f64_of, log,
                      round_bf16, sync, upload)
from verify_inputs import LATENT, PAGE, build_inputs, make_kv_update_inputs

pytestmark = pytest.mark.gpu


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def _append_gpu(x, pool_dev):
    bad = torch.zeros(1, dtype=torch.int32, device=dev())
    mv.verify_kv_append(bf16_tensor(x.new_latent), _i32(x.slots), _i32(x.block_table), pool_dev,
                        bad_slots=bad)
    sync()
    return int(bad.item())


@pytest.mark.parametrize("batch,q_len,max_pages,pool_pages,skip,bad_frac,seed", [
    (16, 8, 25, 512, 0.1, 0.1, 1),     # TP8-share group shape
    (1, 1, 1, 1, 0.0, 0.0, 2),         # smallest
    (33, 16, 4, 200, 0.3, 0.2, 3),     # longest group, ragged batch (tail workgroup)
    (64, 5, 3, 256, 0.0, 0.0, 4),      # every token written
    (7, 4, 2, 30, 1.0, 0.0, 5),        # every token owned elsewhere
    (9, 8, 2, 40, 0.0, 1.0, 6),        # every slot invalid
])
def test_append_matches_oracle(batch, q_len, max_pages, pool_pages, skip, bad_frac, seed):
    log(f"kv_append B={batch} T={q_len} P={max_pages} N={pool_pages} skip={skip} bad={bad_frac} seed={seed}")
    x = make_kv_update_inputs(batch=batch, q_len=q_len, max_pages=max_pages, pool_pages=pool_pages,
                              seed=seed, skip_frac=skip, bad_frac=bad_frac)
    pool = bf16_tensor(x.pool)
    bad = _append_gpu(x, pool)
    want, want_bad = ku.kv_append(x.pool, x.block_table, x.slots, x.new_latent)
    assert bad == want_bad
    assert np.array_equal(bits_of(pool), want)


def test_append_page_ids_out_of_range_are_counted_not_written():
    log("kv_append with block-table entries outside the pool")
    x = make_kv_update_inputs(batch=8, q_len=8, max_pages=3, pool_pages=40, seed=7)
    table = x.block_table.copy()
    table[1, :] = -1
    table[2, :] = 40 + np.arange(3)   # past the pool
    x.block_table = table
    pool = bf16_tensor(x.pool)
    bad = _append_gpu(x, pool)
    want, want_bad = ku.kv_append(x.pool, table, x.slots, x.new_latent)
    assert want_bad == 16 and bad == want_bad
    assert np.array_equal(bits_of(pool), want)


def test_append_duplicate_slots_write_one_of_the_rows():
    log("kv_append with duplicated slots")
    x = make_kv_update_inputs(batch=4, q_len=6, max_pages=2, pool_pages=16, seed=8)
    slots = x.slots.copy()
    slots[:, 3] = slots[:, 1]
    pool = bf16_tensor(x.pool)
    x.slots = slots
    assert _append_gpu(x, pool) == 0
    got = bits_of(pool)
    for b in range(4):
        s = int(slots[b, 1])
        row = got[x.block_table[b, s // PAGE], s % PAGE]
        assert np.array_equal(row, x.new_latent[b, 1]) or np.array_equal(row, x.new_latent[b, 3])
    # every other row matches the oracle (duplicates aside, order does not matter)
    want, _ = ku.kv_append(x.pool, x.block_table, slots, x.new_latent)
    diff = np.argwhere(np.any(got != want, axis=2))
    assert len(diff) <= 4


def test_append_full_size_pool_sampled():
    # the 64 x 8 group of the ragged workload into a 16384-page pool: the
    # written rows are checked one by one, the rest by a seeded sample
    log("kv_append B=64 T=8 P=128 N=16384 (sampled)")
    x = make_kv_update_inputs(batch=64, q_len=8, max_pages=128, pool_pages=16384, seed=9,
                              skip_frac=0.1, bad_frac=0.05, dense_pool=False)
    g = torch.Generator(device=dev()).manual_seed(9)
    pool = (torch.randn((16384, PAGE, LATENT), device=dev(), generator=g) * 0.05).to(torch.bfloat16)
    rng = np.random.default_rng(9)
    sample_pages = torch.from_numpy(rng.integers(0, 16384, size=256)).to(dev())
    sample_rows = torch.from_numpy(rng.integers(0, PAGE, size=256)).to(dev())
    before = pool[sample_pages, sample_rows].clone()
    bad = _append_gpu(x, pool)
    invalid = (x.slots < -1) | (x.slots >= 128 * PAGE)
    assert bad == int(invalid.sum())
    valid = np.argwhere((x.slots >= 0) & ~invalid)
    written = set()
    for b, t in valid:
        s = int(x.slots[b, t])
        page, row = int(x.block_table[b, s // PAGE]), s % PAGE
        written.add((page, row))
        assert np.array_equal(bits_of(pool[page, row]), x.new_latent[b, t]), (b, t)
    after = pool[sample_pages, sample_rows]
    for i in range(256):
        key = (int(sample_pages[i]), int(sample_rows[i]))
        if key not in written:
            assert torch.equal(after[i], before[i]), key


@pytest.mark.parametrize("batch,q_len,max_pages,seed", [
    (1000, 8, 25, 11), (1, 1, 1, 12), (300, 16, 3, 13), (257, 2, 129, 14)])
def test_trim_matches_oracle(batch, q_len, max_pages, seed):
    log(f"kv_trim B={batch} T={q_len} P={max_pages} seed={seed}")
    rng = np.random.default_rng(seed)
    kv_len = rng.integers(-3, max_pages * PAGE + 20, size=batch).astype(np.int32)
    # push a third of the lengths next to a page boundary
    edge = rng.random(batch) < 0.33
    kv_len[edge] = (rng.integers(0, max_pages + 1, size=int(edge.sum())) * PAGE
                    + rng.integers(-2, 3, size=int(edge.sum())))
    accepted = rng.integers(-2, q_len + 2, size=batch).astype(np.int32)
    table = rng.integers(-1, 5000, size=(batch, max_pages)).astype(np.int32)
    t_dev = _i32(table)
    new_len, released = mv.verify_kv_trim(_i32(kv_len), _i32(accepted), t_dev, q_len)
    sync()
    want_len, want_table, want_rel = ku.kv_trim(kv_len, accepted, table, q_len)
    assert np.array_equal(new_len.cpu().numpy(), want_len)
    assert np.array_equal(released.cpu().numpy(), want_rel)
    assert np.array_equal(t_dev.cpu().numpy(), want_table)


def test_trim_in_place_lengths():
    log("kv_trim with new_len aliasing kv_len")
    rng = np.random.default_rng(15)
    kv_len = rng.integers(0, 3 * PAGE, size=64).astype(np.int32)
    accepted = rng.integers(0, 8, size=64).astype(np.int32)
    table = np.arange(64 * 3, dtype=np.int32).reshape(64, 3)
    lens = _i32(kv_len)
    new_len, _ = mv.verify_kv_trim(lens, _i32(accepted), _i32(table), 8, new_len=lens)
    sync()
    assert new_len.data_ptr() == lens.data_ptr()
    want_len, _, _ = ku.kv_trim(kv_len, accepted, table, 8)
    assert np.array_equal(lens.cpu().numpy(), want_len)


def test_append_then_verify_attention_sees_the_group():
    # a verify batch whose group keys are first poisoned in the device pool,
    # then written back by the append kernel from the per-token slot table:
    # the attention must match the oracle on the original cache
    log("kv_append + verify_attn, B=4 H=8 T=8")
    q_len = 8
    ctx = np.array([70, 64, 200, 9])
    x = build_inputs(batch=4, heads=8, q_len=q_len, ctx=ctx, seed=16, gated=False, latent_q=True)
    d = upload(x)
    slots = (ctx[:, None] - q_len + np.arange(q_len)[None, :]).astype(np.int32)
    slots[3, :4] = -1   # owned by another rank: not written (their rows stay as they are)
    group = np.zeros((4, q_len, LATENT), dtype=np.uint16)
    pool_rows = bits_of(d["pool"])
    for b in range(4):
        for t in range(q_len):
            s = int(slots[b, t])
            if s >= 0:
                page, row = int(x.block_table[b, s // PAGE]), s % PAGE
                group[b, t] = pool_rows[page, row]
                d["pool"][page, row] = float("nan")
    bad = torch.zeros(1, dtype=torch.int32, device=dev())
    mv.verify_kv_append(bf16_tensor(group), _i32(slots), d["block_table"], d["pool"], bad_slots=bad)
    out, lse = mv.verify_attn(d["q_latent"], d["pool"], d["block_table"], d["kv_bounds"], x.sm_scale)
    sync()
    assert int(bad.item()) == 0
    want, want_lse = oracle.verify_attention_latent(x.q_latent, x.pool, x.block_table, x.kv_bounds,
                                                    x.sm_scale)
    assert_lse(lse.cpu().numpy().astype(np.float64), want_lse, "lse after append")
    assert_close_output(f64_of(out), want, "out_latent after append")
