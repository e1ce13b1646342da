"""Input builders for indexing probes (no attention arithmetic here)."""
import numpy as np

from verify_inputs import (FP8_NAN, LATENT, PAGE, bf16_bits_to_fp8_codes, build_inputs,
                           f32_to_bf16_bits)

STEP = 1024.0   # score gap between consecutive keys: exp(-1024) is 0 in fp32 and fp64


def bf(v):
    return f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def needle_case(bounds, heads=2, seed=0, pool_pages=None):
    """Needle/decoy probe.  Key j of request b holds
    (STEP*j, 1, b+1, page+1, slot+1, 0, ...) and token t's query is
    (1, -STEP*(L-1), 0, ...), so with sm_scale = 1 the score of key j is
    STEP*(j - L + 1): the last visible key scores exactly 0 and wins with
    weight exactly 1, every earlier key underflows to weight 0, and key L (the
    decoy just past the bound, visible to later tokens) would win if the bound
    were off by one.  Output must equal key L-1 bit for bit and lse must be 0.
    Bounds must stay below 256 so every value is exact in bf16.
    Returns (inputs, dense pool, q_latent bits, bounds).
    """
    bounds = np.asarray(bounds, np.int32)
    assert bounds.max() < 256
    bsz, tlen = bounds.shape
    ctx = np.maximum(bounds.max(axis=1), 1)
    x = build_inputs(batch=bsz, heads=heads, q_len=tlen, ctx=ctx, bounds=bounds, seed=seed,
                     latent_q=True, sm_scale=1.0, pool_pages=pool_pages)
    pool = x.pool.dense()
    for b in range(bsz):
        n = int(bounds[b].max())
        for j in range(n):
            page, slot = int(x.block_table[b, j // PAGE]), j % PAGE
            row = np.zeros(LATENT, np.float32)
            row[:5] = [STEP * j, 1.0, b + 1, page + 1, slot + 1]
            pool[page, slot] = bf(row)
    q = np.zeros((bsz, tlen, heads, LATENT), np.uint16)
    for b in range(bsz):
        for t in range(tlen):
            L = int(bounds[b, t])
            q[b, t, :, 0] = bf(1.0)
            q[b, t, :, 1] = bf(-STEP * max(L - 1, 0))
    return x, pool, q, bounds


def needle_expected(x, bounds):
    """Expected latent output rows of the needle probe (float64)."""
    bsz, tlen = bounds.shape
    want = np.zeros((bsz, tlen, LATENT))
    for b in range(bsz):
        for t in range(tlen):
            L = int(bounds[b, t])
            if L == 0:
                continue
            j = L - 1
            page = int(x.block_table[b, j // PAGE])
            want[b, t, :5] = [STEP * j, 1.0, b + 1, page + 1, j % PAGE + 1]
    return want


def needle_case_fp8(bounds, heads=2, seed=0, kv_scale=0.5):
    """The needle/decoy probe for an fp8 (E4M3) cache.  Key j holds the E4M3
    codes of (1, j // 16, j % 16, b+1, page // 16 + 1, page % 16 + 1,
    slot // 16 + 1, slot % 16 + 1, 0, ...) -- integers up to 16, all exact in
    E4M3 -- and token t's query is (-STEP (L-1), 16 STEP, STEP, 0, ...) / kv_scale,
    so with sm_scale = 1 the score of key j is again STEP (j - L + 1): the
    last visible key wins with weight exactly 1 and the output must be
    kv_scale times its row, bit for bit, with lse 0.  Needs bounds < 256 and
    fewer than 256 pool pages.  Returns (inputs, dense code pool, q_latent
    bits, bounds)."""
    bounds = np.asarray(bounds, np.int32)
    assert bounds.max() < 256
    bsz, tlen = bounds.shape
    ctx = np.maximum(bounds.max(axis=1), 1)
    x = build_inputs(batch=bsz, heads=heads, q_len=tlen, ctx=ctx, bounds=bounds, seed=seed,
                     latent_q=True, sm_scale=1.0)
    assert x.pool.num_pages < 256
    pool = np.full((x.pool.num_pages, PAGE, LATENT), FP8_NAN, np.uint8)
    for b in range(bsz):
        n_pg = -(-int(bounds[b].max()) // PAGE)
        for j in range(n_pg * PAGE):
            page, slot = int(x.block_table[b, j // PAGE]), j % PAGE
            row = np.zeros(LATENT, np.float32)
            row[:8] = [1.0, j // 16, j % 16, b + 1, page // 16 + 1, page % 16 + 1, slot // 16 + 1,
                       slot % 16 + 1]
            pool[page, slot] = bf16_bits_to_fp8_codes(bf(row), 1.0)
    q = np.zeros((bsz, tlen, heads, LATENT), np.uint16)
    for b in range(bsz):
        for t in range(tlen):
            L = int(bounds[b, t])
            q[b, t, :, 0] = bf(-STEP * max(L - 1, 0) / kv_scale)
            q[b, t, :, 1] = bf(16 * STEP / kv_scale)
            q[b, t, :, 2] = bf(STEP / kv_scale)
    return x, pool, q, bounds


def needle_expected_fp8(x, bounds, kv_scale=0.5):
    """Expected latent output rows of the fp8 needle probe (float64)."""
    bsz, tlen = bounds.shape
    want = np.zeros((bsz, tlen, LATENT))
    for b in range(bsz):
        for t in range(tlen):
            L = int(bounds[b, t])
            if L == 0:
                continue
            j = L - 1
            page, slot = int(x.block_table[b, j // PAGE]), j % PAGE
            want[b, t, :8] = kv_scale * np.array([1.0, j // 16, j % 16, b + 1, page // 16 + 1,
                                                  page % 16 + 1, slot // 16 + 1, slot % 16 + 1])
    return want
