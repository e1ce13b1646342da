"""Input builders for indexing probes (no attention arithmetic here)."""
import numpy as np

from verify_inputs import LATENT, PAGE, build_inputs, f32_to_bf16_bits

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
