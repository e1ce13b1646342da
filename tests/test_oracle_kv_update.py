"""Pins of the KV-update oracle (append by per-token slot table, trim of
rejected tails) against things other than itself: a hand-worked golden case,
the attention oracle's own cache gather, closed forms and invariants."""
import json
import os

import numpy as np
import pytest

from oracle import kv_update as ku
from oracle import mla_oracle as om
from verify_inputs import LATENT, PAGE, f32_to_bf16_bits, make_kv_update_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_append_trim_hand.json")


def _golden():
    with open(GOLDEN) as fh:
        return json.load(fh)


def test_append_golden_hand_case():
    g = _golden()["append"]
    table = np.array(g["block_table"], dtype=np.int32)
    slots = np.array(g["slots"], dtype=np.int32)
    b, t = slots.shape
    pool = np.zeros((g["num_pages"], PAGE, LATENT), dtype=np.uint16)
    latent = np.zeros((b, t, LATENT), dtype=np.float32)
    for bb in range(b):
        for tt in range(t):
            latent[bb, tt, 0] = 10 * bb + tt + 1
    new_pool, bad = ku.kv_append(pool, table, slots, f32_to_bf16_bits(latent))
    assert bad == g["expected_bad"]
    changed = np.argwhere(np.any(new_pool != 0, axis=2))
    want = sorted((p, r) for p, r, _ in g["expected_rows"])
    assert sorted(map(tuple, changed.tolist())) == want
    for p, r, v in g["expected_rows"]:
        assert om.bf16_to_f64(new_pool[p, r, :1])[0] == v
        assert not np.any(new_pool[p, r, 1:])


def test_trim_golden_hand_case():
    g = _golden()["trim"]
    new_len, table, released = ku.kv_trim(np.array(g["kv_len"]), np.array(g["accepted"]),
                                          np.array(g["block_table"], dtype=np.int32), g["q_len"])
    assert new_len.tolist() == g["expected_new_len"]
    assert released.tolist() == g["expected_released"]
    assert table.tolist() == g["expected_block_table"]


def test_appended_tokens_are_the_keys_the_attention_gathers():
    # the attention oracle's own paging (request_keys) must find token t of
    # request b at key position ctx[b] + t after the append
    x = make_kv_update_inputs(batch=3, q_len=5, max_pages=4, pool_pages=24, seed=11)
    pool, bad = ku.kv_append(x.pool, x.block_table, x.slots, x.new_latent)
    assert bad == 0
    bounds = (x.ctx + x.slots.shape[1])[:, None].astype(np.int32)
    for b in range(3):
        keys, n = om.request_keys(pool, x.block_table, bounds, b)
        assert n == x.ctx[b] + 5
        np.testing.assert_array_equal(keys[x.ctx[b]:], om.bf16_to_f64(x.new_latent[b]))
        # the keys before the group are untouched
        before, _ = om.request_keys(x.pool, x.block_table, bounds, b)
        np.testing.assert_array_equal(keys[:x.ctx[b]], before[:x.ctx[b]])


def test_append_skips_minus_one_and_counts_invalid():
    x = make_kv_update_inputs(batch=6, q_len=8, max_pages=3, pool_pages=40, seed=3,
                              skip_frac=0.3, bad_frac=0.3)
    pool, bad = ku.kv_append(x.pool, x.block_table, x.slots, x.new_latent)
    # count invalid entries by the stated rule, independently of the loop
    invalid = (x.slots < -1) | (x.slots >= x.block_table.shape[1] * PAGE)
    assert bad == int(invalid.sum())
    # rows written: exactly the valid slots
    written = int(np.sum(np.any(pool != x.pool, axis=2)))
    valid = int(np.sum((x.slots >= 0) & ~invalid))
    assert written <= valid   # a written row may coincide with the old bits only by chance
    all_skip = np.full_like(x.slots, -1)
    same, bad0 = ku.kv_append(x.pool, x.block_table, all_skip, x.new_latent)
    assert bad0 == 0 and np.array_equal(same, x.pool)


def test_append_is_independent_of_token_order():
    x = make_kv_update_inputs(batch=4, q_len=6, max_pages=3, pool_pages=30, seed=5, skip_frac=0.2)
    a, _ = ku.kv_append(x.pool, x.block_table, x.slots, x.new_latent)
    perm = np.random.default_rng(0).permutation(6)
    b, _ = ku.kv_append(x.pool, x.block_table, x.slots[:, perm], x.new_latent[:, perm])
    assert np.array_equal(a, b)


def test_trim_closed_forms():
    rng = np.random.default_rng(7)
    q_len, pages = 8, 5
    kv = rng.integers(0, pages * PAGE + 1, size=200)
    table = np.arange(200 * pages, dtype=np.int32).reshape(200, pages)
    # everything accepted: nothing changes
    n_all, t_all, r_all = ku.kv_trim(kv, np.full(200, q_len - 1), table, q_len)
    assert np.array_equal(n_all, kv) and np.array_equal(t_all, table) and np.all(r_all == -1)
    # general: a page is released exactly when the page count drops
    acc = rng.integers(0, q_len, size=200)
    new, t2, rel = ku.kv_trim(kv, acc, table, q_len)
    assert np.array_equal(new, np.maximum(0, kv - (q_len - 1 - acc)))
    before = -(-kv // PAGE)
    after = -(-new // PAGE)
    assert np.array_equal(rel != -1, after < before)
    for i in np.flatnonzero(rel != -1):
        assert rel[i] == table[i, after[i]] and t2[i, after[i]] == -1
    assert np.sum(t2 != table) == np.sum(rel != -1)


def test_trim_then_next_group_equals_a_cache_built_without_the_rejected_tail():
    # step n: group G1 appended and verified with `a` accepted drafts; step
    # n+1: group G2 appended after the kept tokens.  The cache the attention
    # then sees must equal one built by appending G1[:1+a] and G2 directly.
    q_len, a = 6, 2
    x = make_kv_update_inputs(batch=2, q_len=q_len, max_pages=4, pool_pages=16, seed=21,
                              ctx=[60, 120])
    g2 = make_kv_update_inputs(batch=2, q_len=q_len, max_pages=4, pool_pages=16, seed=22,
                               ctx=[0, 0]).new_latent
    pool1, _ = ku.kv_append(x.pool, x.block_table, x.slots, x.new_latent)
    length = x.ctx + q_len
    new_len, table, released = ku.kv_trim(length, np.full(2, a), x.block_table, q_len)
    assert np.array_equal(new_len, x.ctx + 1 + a)
    assert released[0] != -1   # request 0 drops back below its second page
    # the next group needs the released page back (a fresh allocation here)
    for b in range(2):
        if released[b] != -1:
            table[b, np.flatnonzero(table[b] == -1)[0]] = released[b]
    slots2 = (new_len[:, None] + np.arange(q_len)[None, :]).astype(np.int32)
    pool2, _ = ku.kv_append(pool1, table, slots2, g2)
    direct_slots = (x.ctx[:, None] + np.arange(1 + a)[None, :]).astype(np.int32)
    direct, _ = ku.kv_append(x.pool, x.block_table, direct_slots, x.new_latent[:, :1 + a])
    direct, _ = ku.kv_append(direct, x.block_table, slots2, g2)
    bounds = (new_len + q_len)[:, None].astype(np.int32)
    for b in range(2):
        k1, n1 = om.request_keys(pool2, table, bounds, b)
        k2, n2 = om.request_keys(direct, x.block_table, bounds, b)
        assert n1 == n2
        np.testing.assert_array_equal(k1, k2)
