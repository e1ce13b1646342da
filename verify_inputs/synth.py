"""Seeded synthetic inputs for speculative-verify MLA attention.

This module only draws random data and lays it out; it contains none of the
attention arithmetic.  Both the CPU oracle (``oracle/``) and the HIP path use
it, so that both sides see the same bytes.

Workloads (the shapes follow the verify groups and capture buckets described
in "Kimi K3 support with DSpark speculative decoding", section "What does this
PR do?": draft schedule {16: 7, 32: 4, 64: 0}; the per-token bounds follow the
"Per-token primitive" paragraph of "Kimi K3: DSpark speculative decoding under
Helix CP"):

  1  tiny verify      B=1,  H=8,  T=4,  ctx=256 (4 pages, permuted), gated
  2  TP8 share        B=16, H=8,  T=8,  ctx ~ U{1024..1536}, pool 4096 pages
  3  split 4          B=32, H=8,  T=5,  ctx ~ U{1024..1536}, pool 4096, S=4
  4  plain decode     B=64, H=64, T=1,  ctx ~ U{1024..1536}, pool 4096
  5  ragged, gated    B=64, H=64, T=8,  ctx ~ round(exp U[ln 128, ln 8192]),
                      pool 16384, 10% of tokens bound 0, 10% truncated, S=8

Conventions:
  * bf16 tensors are numpy ``uint16`` bit patterns (round-to-nearest-even
    from float32).
  * ``ctx`` counts the cache including the group's own k+1 tokens, so token t
    of a group of T sees ``ctx - (T-1) + t`` keys.
  * Unreferenced pool pages and cache slots past a request's last visible key
    hold a quiet NaN (0x7FC0); block-table entries past a request's pages are
    -1.  A correct kernel never lets them reach an output.
  * Draw order (fixed): ctx -> bounds -> page assignment -> q_nope -> W_UK ->
    W_UV -> gate -> latent values of referenced pages -> (optional) direct
    q_latent.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

LATENT = 512          # latent rank of the compressed KV
PAGE = 64             # tokens per KV page
NOPE = 128            # per-head q_nope / value dim
BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)      # OCP E4M3 NaN code
# Scale of the fp8 cache workloads: latent = FP8_KV_SCALE * E4M3 value.  A
# power of two, so dividing the bf16 draws by it is exact; the draws (std
# 1/sqrt(512) ~ 0.044) then sit at codes of magnitude ~11 (E4M3 covers up to
# 448), far above the subnormal range.
FP8_KV_SCALE = 2.0 ** -8

CONFIG_SEEDS = {1: 0, 2: 1, 3: 2, 4: 3, 5: 4}


@dataclasses.dataclass
class ConfigSpec:
    batch: int
    heads: int
    q_len: int
    pool_pages: int
    max_pages: int          # block-table row stride
    ctx: str                # "fixed256", "uniform", "loguniform"
    splits: int             # 0 = library's choice
    gated: bool
    zero_frac: float = 0.0
    trunc_frac: float = 0.0


CONFIGS = {
    1: ConfigSpec(1, 8, 4, 4, 4, "fixed256", 0, True),
    2: ConfigSpec(16, 8, 8, 4096, 24, "uniform", 0, False),
    3: ConfigSpec(32, 8, 5, 4096, 24, "uniform", 4, False),
    4: ConfigSpec(64, 64, 1, 4096, 24, "uniform", 0, False),
    5: ConfigSpec(64, 64, 8, 16384, 128, "loguniform", 8, True, 0.1, 0.1),
}


@dataclasses.dataclass
class VerifyInputs:
    """One verify batch.  bf16 arrays are uint16 bit patterns."""
    q_nope: np.ndarray       # [B, T, H, 128] bf16
    w_uk: np.ndarray         # [H, 128, 512] bf16
    w_uv: np.ndarray         # [H, 128, 512] bf16
    gate: np.ndarray         # [B, T, H, 128] bf16
    pool: "SparsePool"       # [N_pool, 64, 512] bf16 (referenced pages stored)
    block_table: np.ndarray  # [B, max_pages] int32, -1 past a request's pages
    kv_bounds: np.ndarray    # [B, T] int32 visible-key counts
    ctx: np.ndarray          # [B] int64 tokens in each request's cache
    sm_scale: float
    num_splits: int
    gated: bool
    q_latent: np.ndarray | None = None   # [B, T, H, 512] bf16, direct draw
    kv_dtype: str = "bf16"               # "bf16", or "fp8" (pool holds E4M3 codes)
    kv_scale: float = 1.0                # fp8: latent = kv_scale * code value

    @property
    def shape(self):
        b, t, h, _ = self.q_nope.shape
        return b, t, h


class SparsePool:
    """A [num_pages, 64, 512] page pool of which only referenced pages are
    stored; every other page reads as NaN.  Indexing with an integer page-id
    array returns the dense pages, like a numpy array would.  Elements are
    bf16 bit patterns (uint16) or, for an fp8 cache, E4M3 codes (uint8)."""

    def __init__(self, num_pages: int, page_ids: np.ndarray, pages: np.ndarray):
        self.num_pages = int(num_pages)
        self.page_ids = np.asarray(page_ids, dtype=np.int64)
        self.pages = pages
        self.slot = np.full(self.num_pages, -1, dtype=np.int64)
        self.slot[self.page_ids] = np.arange(self.page_ids.size)
        self.shape = (self.num_pages, PAGE, LATENT)
        self.dtype = np.dtype(pages.dtype)
        self.fill = FP8_NAN if self.dtype == np.uint8 else BF16_NAN

    def __getitem__(self, idx):
        idx = np.asarray(idx, dtype=np.int64)
        if np.any((idx < 0) | (idx >= self.num_pages)):
            raise IndexError("page id outside the pool")
        s = self.slot[idx]
        out = np.full(idx.shape + (PAGE, LATENT), self.fill, dtype=self.dtype)
        have = s >= 0
        out[have] = self.pages[s[have]]
        return out

    def dense(self) -> np.ndarray:
        out = np.full(self.shape, self.fill, dtype=self.dtype)
        out[self.page_ids] = self.pages
        return out

    def remap(self, perm: np.ndarray) -> "SparsePool":
        """The same pages stored at ids ``perm[old_id]``."""
        return SparsePool(self.num_pages, np.asarray(perm)[self.page_ids], self.pages)


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even) and return the bit pattern."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32)
    # uint32 wrap-around only happens for NaN inputs, which are overwritten below
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_bits_to_f32(u) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (data plumbing only)."""
    u = np.ascontiguousarray(np.asarray(u, dtype=np.uint16))
    return (u.astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(rng, shape, std):
    return f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


def _draw_ctx(rng, spec: ConfigSpec) -> np.ndarray:
    if spec.ctx == "fixed256":
        return np.full(spec.batch, 256, dtype=np.int64)
    if spec.ctx == "uniform":
        return rng.integers(1024, 1536, size=spec.batch, endpoint=True).astype(np.int64)
    if spec.ctx == "loguniform":
        u = rng.uniform(math.log(128), math.log(8192), size=spec.batch)
        return np.rint(np.exp(u)).astype(np.int64)
    raise ValueError(spec.ctx)


def _draw_bounds(rng, spec: ConfigSpec, ctx: np.ndarray) -> np.ndarray:
    b, t = spec.batch, spec.q_len
    causal = ctx[:, None] - (t - 1) + np.arange(t)[None, :]
    bounds = causal.copy()
    n_tok = b * t
    if spec.zero_frac > 0:
        n_zero = int(round(spec.zero_frac * n_tok))
        zero_idx = rng.choice(n_tok, size=n_zero, replace=False)
        bounds.reshape(-1)[zero_idx] = 0
    if spec.trunc_frac > 0:
        n_trunc = int(round(spec.trunc_frac * n_tok))
        flat = bounds.reshape(-1)
        cand = np.array([i for i in range(n_tok) if (i % t) >= 1 and flat[i] != 0])
        pick = rng.choice(cand, size=min(n_trunc, cand.size), replace=False)
        for i in np.sort(pick):
            bi, ti = divmod(int(i), t)
            earlier = int(rng.integers(0, ti))
            flat[i] = causal[bi, earlier]
    return bounds.astype(np.int32)


def _assign_pages(rng, pool_pages, max_pages, n_pages):
    total = int(n_pages.sum())
    if total > pool_pages:
        raise ValueError(f"{total} pages requested from a pool of {pool_pages}")
    if int(n_pages.max(initial=0)) > max_pages:
        raise ValueError("a request needs more pages than the block-table stride")
    picks = rng.choice(pool_pages, size=total, replace=False).astype(np.int32)
    table = np.full((n_pages.size, max_pages), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(n_pages):
        table[b, :n] = picks[off:off + n]
        off += n
    return table


def build_inputs(*, batch, heads, q_len, ctx, bounds=None, pool_pages=None, max_pages=None,
                 seed=0, gated=True, num_splits=0, q_scale=1.0, latent_q=False,
                 sm_scale=None, permute_single=False) -> VerifyInputs:
    """General builder used by the named workloads and by small test cases.

    ``ctx`` is an int array [B]; ``bounds`` an int array [B, T] (defaults to
    the causal group bounds ctx-(T-1)+t).  Pages needed per request are
    ceil(max(bounds[b]) / 64); only those are referenced.
    """
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx, dtype=np.int64).reshape(batch)
    if bounds is None:
        bounds = (ctx[:, None] - (q_len - 1) + np.arange(q_len)[None, :]).astype(np.int32)
    bounds = np.asarray(bounds, dtype=np.int32).reshape(batch, q_len)
    return _finish(rng, batch, heads, q_len, ctx, bounds, pool_pages, max_pages, gated,
                   num_splits, q_scale, latent_q, sm_scale, permute_single)


def _finish(rng, batch, heads, q_len, ctx, bounds, pool_pages, max_pages, gated, num_splits,
            q_scale, latent_q, sm_scale, permute_single=False):
    n_keys = np.clip(bounds.max(axis=1), 0, None).astype(np.int64)
    n_pages = (n_keys + PAGE - 1) // PAGE
    if max_pages is None:
        max_pages = max(1, int(n_pages.max(initial=0)))
    if pool_pages is None:
        pool_pages = max(1, int(n_pages.sum()) * 2)
    if permute_single:
        # the tiny workload: block_table is a random permutation of the pool
        assert batch == 1 and int(n_pages[0]) == pool_pages == max_pages
        table = rng.permutation(pool_pages).astype(np.int32)[None, :]
    else:
        table = _assign_pages(rng, pool_pages, max_pages, n_pages)
    std = 1.0 / math.sqrt(LATENT)
    q_nope = _normal_bf16(rng, (batch, q_len, heads, NOPE), std * q_scale)
    w_uk = _normal_bf16(rng, (heads, NOPE, LATENT), std)
    w_uv = _normal_bf16(rng, (heads, NOPE, LATENT), std)
    gate = _normal_bf16(rng, (batch, q_len, heads, NOPE), 1.0)
    ids, pages = [], []
    for b in range(batch):
        n = int(n_keys[b])
        if n == 0:
            continue
        vals = _normal_bf16(rng, (n, LATENT), std)
        npg = int(n_pages[b])
        padded = np.full((npg * PAGE, LATENT), BF16_NAN, dtype=np.uint16)
        padded[:n] = vals
        ids.append(table[b, :npg])
        pages.append(padded.reshape(npg, PAGE, LATENT))
    pool = SparsePool(pool_pages,
                      np.concatenate(ids) if ids else np.zeros(0, np.int32),
                      np.concatenate(pages) if pages else np.zeros((0, PAGE, LATENT), np.uint16))
    q_latent = None
    if latent_q:
        # direct draw with the spread an absorbed query has (std sqrt(128)/512)
        q_latent = _normal_bf16(rng, (batch, q_len, heads, LATENT),
                                math.sqrt(NOPE) / LATENT * q_scale)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(NOPE)
    return VerifyInputs(q_nope, w_uk, w_uv, gate, pool, table, bounds.astype(np.int32), ctx,
                        float(sm_scale), int(num_splits), bool(gated), q_latent)


# Factor on q_nope that makes the scaled scores' spread about 3 (instead of
# ~0.002 for the stated N(0,1)/sqrt(512) draws), so softmax is far from uniform.
SHARP_Q_SCALE = 1536.0


def make_config(n: int, seed: int | None = None, *, sharp: bool = False,
                latent_q: bool = False) -> VerifyInputs:
    """One of the five named workloads, drawn from ``seed`` (default: its own)."""
    spec = CONFIGS[n]
    rng = np.random.default_rng(CONFIG_SEEDS[n] if seed is None else seed)
    ctx = _draw_ctx(rng, spec)
    bounds = _draw_bounds(rng, spec, ctx)
    return _finish(rng, spec.batch, spec.heads, spec.q_len, ctx, bounds, spec.pool_pages,
                   spec.max_pages, spec.gated, spec.splits,
                   SHARP_Q_SCALE if sharp else 1.0, latent_q, None,
                   permute_single=(spec.ctx == "fixed256"))


def ramp_scores(inp: VerifyInputs, rise: float = 200.0, seed: int = 7) -> VerifyInputs:
    """The same batch with scores that drift along each request's context.

    Key j of a request with n visible keys gets ``(j / n) * r`` times one
    seeded random unit vector u added to its latent row, with
    ``r = rise / (sm_scale * sigma)`` and sigma the spread of an absorbed
    query's projection on u implied by the draws (sqrt(128)/512 times the
    query scale).  A query whose projection is one sigma above zero then sees
    its scores rise by ``rise`` nats from the first key to the last; half the
    queries rise, half fall.  (Stress input for the softmax's reference
    handling; the drift is in the cache, so every row of a request sees it.)
    """
    q_scale = float(np.std(bf16_bits_to_f32(inp.q_nope))) * math.sqrt(LATENT) or 1.0
    sigma = math.sqrt(NOPE) / LATENT * q_scale
    r = rise / (inp.sm_scale * sigma)
    u = np.random.default_rng(seed).standard_normal(LATENT)
    u /= np.linalg.norm(u)
    pages = bf16_bits_to_f32(inp.pool.pages).copy()          # [n_pages, 64, 512]
    slot = inp.pool.slot
    n_keys = np.clip(inp.kv_bounds.max(axis=1), 0, None)
    for b in range(inp.block_table.shape[0]):
        n = int(n_keys[b])
        if n == 0:
            continue
        j = np.arange(n)
        s = slot[inp.block_table[b, j // PAGE]]
        pages[s, j % PAGE] += ((j / n) * r)[:, None].astype(np.float32) * u[None, :].astype(np.float32)
    out = dataclasses.replace(inp)
    out.pool = SparsePool(inp.pool.num_pages, inp.pool.page_ids, f32_to_bf16_bits(pages))
    return out


def bf16_bits_to_fp8_codes(bits, kv_scale: float) -> np.ndarray:
    """E4M3 codes of bf16 values divided by ``kv_scale``: round to nearest
    even, NaN stays NaN (code 0x7F).  The encoding is torch's float8_e4m3fn
    conversion on the CPU; values are clipped to +-448 first so nothing maps
    to NaN by overflow.  (Input plumbing: it writes the cache an fp8 serving
    stack would hold; the attention reads the codes.)"""
    import torch

    x = bf16_bits_to_f32(bits).astype(np.float64) / float(kv_scale)
    nan = np.isnan(x)
    x = np.clip(np.where(nan, 0.0, x), -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    codes[nan] = FP8_NAN
    return codes


def fp8_cache(inp: VerifyInputs, kv_scale: float = FP8_KV_SCALE) -> VerifyInputs:
    """The same verify batch with its latent cache stored as fp8 E4M3 codes
    (``kv_scale`` times the code's value approximates each bf16 latent).
    Unreferenced pages and slots past the last visible key stay NaN."""
    pool = inp.pool
    pages = bf16_bits_to_fp8_codes(pool.pages, kv_scale)
    out = dataclasses.replace(inp, pool=SparsePool(pool.num_pages, pool.page_ids, pages))
    out.kv_dtype, out.kv_scale = "fp8", float(kv_scale)
    return out


def referenced_kv_bytes(inp: VerifyInputs) -> int:
    """Bytes of KV a kernel must read: one latent row (1 KiB in bf16, 512 B in
    fp8) per visible key of each request."""
    n = np.clip(inp.kv_bounds.max(axis=1), 0, inp.block_table.shape[1] * PAGE)
    return int(n.sum()) * LATENT * (1 if inp.kv_dtype == "fp8" else 2)


@dataclasses.dataclass
class KvUpdateInputs:
    """One verify step's cache update.  bf16 arrays are uint16 bit patterns."""
    pool: np.ndarray         # [N, 64, 512] bf16, dense
    block_table: np.ndarray  # [B, P] int32, -1 past a request's pages
    ctx: np.ndarray          # [B] int64 keys before the group
    slots: np.ndarray        # [B, T] int32 write positions (-1 skip, some invalid)
    new_latent: np.ndarray   # [B, T, 512] bf16
    accepted: np.ndarray     # [B] int32 accepted drafts (some outside [0, T-1])


def make_kv_update_inputs(*, batch, q_len, max_pages, pool_pages, seed, skip_frac=0.0,
                          bad_frac=0.0, ctx=None, dense_pool=True) -> KvUpdateInputs:
    """A seeded cache update: request b holds ``ctx[b]`` keys (uniform in
    [0, max_pages*64 - q_len] unless given) and its group of ``q_len`` tokens
    goes to positions ctx[b] .. ctx[b] + q_len - 1.  Each slot is replaced by
    -1 with probability ``skip_frac`` (owned elsewhere) and by an invalid
    value (>= max_pages*64 or below -1) with probability ``bad_frac``.  Pages
    are distinct across requests, so valid slots never collide.  With
    ``dense_pool=False`` no pool is drawn (``pool`` is None)."""
    rng = np.random.default_rng(seed)
    limit = max_pages * PAGE - q_len
    if ctx is None:
        ctx = rng.integers(0, limit + 1, size=batch)
    ctx = np.asarray(ctx, dtype=np.int64).reshape(batch)
    n_pages = (ctx + q_len + PAGE - 1) // PAGE
    assert int(n_pages.sum()) <= pool_pages, "pool too small for distinct pages"
    perm = rng.permutation(pool_pages)
    table = np.full((batch, max_pages), -1, dtype=np.int32)
    at = 0
    for b in range(batch):
        table[b, :n_pages[b]] = perm[at:at + n_pages[b]]
        at += int(n_pages[b])
    slots = (ctx[:, None] + np.arange(q_len)[None, :]).astype(np.int64)
    u = rng.random((batch, q_len))
    bad_vals = np.where(rng.random((batch, q_len)) < 0.5,
                        rng.integers(max_pages * PAGE, max_pages * PAGE + 1000, size=(batch, q_len)),
                        rng.integers(-1000, -1, size=(batch, q_len)))
    slots = np.where(u < skip_frac, -1, np.where(u < skip_frac + bad_frac, bad_vals, slots))
    new_latent = _normal_bf16(rng, (batch, q_len, LATENT), 1.0 / np.sqrt(LATENT))
    accepted = rng.integers(-1, q_len + 1, size=batch).astype(np.int32)
    # the pool is drawn last, so the other arrays do not depend on dense_pool
    pool = _normal_bf16(rng, (pool_pages, PAGE, LATENT), 1.0 / np.sqrt(LATENT)) if dense_pool else None
    return KvUpdateInputs(pool, table, ctx, slots.astype(np.int32), new_latent, accepted)
