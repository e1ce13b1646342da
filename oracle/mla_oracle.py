"""CPU oracle for speculative-verify attention of gated NoPE MLA.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this module; the product path never calls it.
It shares no code with the HIP library and imports nothing from it.

Everything is computed in float64 with NumPy, as the plain definition of the
method, with no blocking or fusion:

* "Kimi K3 support with DSpark speculative decoding", section "What does this
  PR do?": gated NoPE MLA with absorbed projections; each decode step becomes
  a verify of k drafted tokens.  Absorption is an exact reassociation, so the
  primary definition here is the *unabsorbed* attention: per head, keys and
  values are up-projected from the compressed latent (K_h = C W_UK[h]^T,
  V_h = C W_UV[h]^T) and the no-RoPE query q_nope attends over them.
* "Kimi K3: DSpark speculative decoding under Helix CP", first commit message
  ("Per-token primitive", "CuTe DSL MLA decode") and "Changes": every verify
  token has its own attention bound (the number of visible keys, the token's
  position + 1 on one GPU) that replaces the implicit causal bound, and a
  token with no visible key yields the (-inf, 0) identity (LSE = -inf,
  output 0).  The third commit message: such rows must never average
  arbitrary pool bytes.
* Same page, commit "fold_sq padding rows" / "reduction kernel": the
  merge of partial results by their softmax statistics (the LSE combine).
* vLLM "specialized_decode.drafter.model" module docstring: LSE combine
  followed by W_UV; the gate multiplies the W_UV output.

Readings where the pages are silent (each is listed in the design notes):
gate = elementwise sigmoid over the 128-d per-head output; sm_scale is passed
explicitly; the LSE is a natural logarithm; kv_bounds are clamped to
[0, max_pages*64]; slots past a request's largest bound are never read.

Every function here is pinned by tests in tests/test_oracle_*.py against
closed forms, brute force, a library attention routine and invariants.
"""
from __future__ import annotations

import numpy as np

PAGE = 64
LATENT = 512


# ----------------------------------------------------------------- encoding
def bf16_to_f64(bits) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) exactly into float64.

    A bf16 value is the top half of an IEEE float32, so shifting the pattern
    into the high 16 bits of a 32-bit word gives the float32 with the same
    value; widening float32 -> float64 is exact.
    """
    u = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).astype(np.uint32)
    return (u << np.uint32(16)).view(np.float32).astype(np.float64)


def fp8_e4m3_to_f64(codes) -> np.ndarray:
    """Decode OCP FP8 E4M3 codes (uint8) exactly into float64.

    Bit fields, most significant first: sign (1), exponent (4, bias 7),
    mantissa (3).  Exponent field 0 is subnormal: (m / 8) * 2^-6.  Otherwise
    the value is (1 + m / 8) * 2^(e - 7).  The format has no infinities: only
    the all-ones exponent with all-ones mantissa (0x7F, 0xFF) is NaN, so
    0x7E = 1.75 * 2^8 = 448 is the largest finite value.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def kv_decoder(kv_dtype: str = "bf16", kv_scale: float = 1.0):
    """The function that turns stored latent-cache elements into float64.

    bf16: the exact value of each bit pattern.  fp8 (E4M3): kv_scale times the
    exact value of each code (one scale for the whole cache; the latent serves
    as key and as value, so both uses see the same scaled value).
    """
    if kv_dtype == "bf16":
        return bf16_to_f64
    if kv_dtype == "fp8":
        scale = float(kv_scale)
        return lambda codes: fp8_e4m3_to_f64(codes) * scale
    raise ValueError(kv_dtype)


def sigmoid(x) -> np.ndarray:
    """1 / (1 + e^-x) in float64, evaluated without overflow."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


# ----------------------------------------------------------------- paging
def request_keys(pool, block_table, kv_bounds, b, decode=None) -> tuple[np.ndarray, int]:
    """The latent cache rows request b can see, in logical order.

    Logical token j of request b lives in page block_table[b, j // 64] at slot
    j % 64.  Only the first n_b = max_t bound tokens are gathered, so pages
    past ceil(n_b / 64) and slots past n_b are never read.  ``decode`` turns
    the stored elements into float64 (default: bf16 bit patterns).
    Returns (C_b [n_b, 512] float64, n_b).
    """
    decode = bf16_to_f64 if decode is None else decode
    max_pages = block_table.shape[1]
    n_b = int(np.clip(np.max(kv_bounds[b]), 0, max_pages * PAGE))
    if n_b == 0:
        return np.zeros((0, LATENT)), 0
    n_pages = -(-n_b // PAGE)
    pages = pool[np.asarray(block_table[b, :n_pages], dtype=np.int64)]
    rows = np.asarray(pages).reshape(n_pages * PAGE, LATENT)[:n_b]
    return decode(rows), n_b


def token_bound(kv_bounds, b, t, n_b) -> int:
    """Visible-key count of token t of request b, clamped to [0, n_b]."""
    return int(np.clip(kv_bounds[b, t], 0, n_b))


# ----------------------------------------------------------------- attention
def softmax_attend(scores: np.ndarray, values: np.ndarray):
    """Softmax-weighted sum of ``values`` rows for every row of ``scores``.

    scores [..., L] (already scaled), values [L, d].  Returns (o [..., d],
    lse [...]) with lse = log sum_j exp(scores_j) (natural log).  For L = 0 it
    returns the identity (o = 0, lse = -inf).
    """
    if scores.shape[-1] == 0:
        return (np.zeros(scores.shape[:-1] + (values.shape[-1],)),
                np.full(scores.shape[:-1], -np.inf))
    m = scores.max(axis=-1, keepdims=True)
    w = np.exp(scores - m)
    total = w.sum(axis=-1, keepdims=True)
    lse = (m + np.log(total))[..., 0]
    p = w / total
    return p @ values, lse


def absorb_query(q_nope, w_uk) -> np.ndarray:
    """q_latent[b,t,h,:] = W_UK[h]^T q_nope[b,t,h,:]  (128 -> 512), float64.

    With k_nope = W_UK[h] c for a latent c, <q_nope, k_nope> = <q_latent, c>:
    this is the absorbed projection.
    """
    q = bf16_to_f64(q_nope)
    w = bf16_to_f64(w_uk)
    return np.einsum("bthd,hdc->bthc", q, w)


def verify_attention_latent(q_latent, pool, block_table, kv_bounds, sm_scale,
                            q_is_f64: bool = False, kv_dtype: str = "bf16", kv_scale: float = 1.0):
    """The latent-space (absorbed) definition the C-ABI computes.

    For every request b, token t, head h with bound L = kv_bounds[b, t]:
      s_j   = sm_scale * <q_latent[b,t,h], C_b[j]>       for j < L
      lse   = log sum_j exp(s_j)                         (-inf when L = 0)
      o_lat = sum_j softmax(s)_j C_b[j]                  (0 when L = 0)
    C_b holds the decoded cache rows (``kv_decoder``: bf16, or fp8 E4M3 codes
    times kv_scale).
    Returns (o_lat [B,T,H,512] float64, lse [B,T,H] float64).
    """
    q = q_latent if q_is_f64 else bf16_to_f64(q_latent)
    decode = kv_decoder(kv_dtype, kv_scale)
    bsz, tlen, heads, _ = q.shape
    o = np.zeros((bsz, tlen, heads, LATENT))
    lse = np.full((bsz, tlen, heads), -np.inf)
    for b in range(bsz):
        c_b, n_b = request_keys(pool, block_table, kv_bounds, b, decode)
        for t in range(tlen):
            L = token_bound(kv_bounds, b, t, n_b)
            if L == 0:
                continue
            scores = sm_scale * (q[b, t] @ c_b[:L].T)          # [H, L]
            o[b, t], lse[b, t] = softmax_attend(scores, c_b[:L])
    return o, lse


def verify_attention_mla(q_nope, w_uk, w_uv, gate, pool, block_table, kv_bounds, sm_scale,
                         requests=None, kv_dtype: str = "bf16", kv_scale: float = 1.0):
    """Unabsorbed gated NoPE MLA over the paged latent cache (primary definition).

    Per request b and head h the latent rows are up-projected explicitly:
      K_h = C_b W_UK[h]^T,  V_h = C_b W_UV[h]^T               [n_b, 128]
    and per token t with bound L:
      s_j   = sm_scale * <q_nope[b,t,h], K_h[j]>               j < L
      o_v   = sum_j softmax(s)_j V_h[j]                        [128]
      o_lat = sum_j softmax(s)_j C_b[j]                        [512]
      out   = sigmoid(gate[b,t,h]) * o_v                       [128]
    with the (-inf, 0) identity for L = 0.  ``requests`` restricts the work to
    a subset of b (other entries stay at the identity / NaN-free zeros).  The
    cache rows C_b are decoded by ``kv_decoder(kv_dtype, kv_scale)``.
    Returns a dict with o_v, o_lat, lse, out (float64).
    """
    decode = kv_decoder(kv_dtype, kv_scale)
    qn = bf16_to_f64(q_nope)
    wk = bf16_to_f64(w_uk)
    wv = bf16_to_f64(w_uv)
    g = sigmoid(bf16_to_f64(gate)) if gate is not None else None
    bsz, tlen, heads, dn = qn.shape
    res = {
        "o_v": np.zeros((bsz, tlen, heads, dn)),
        "o_lat": np.zeros((bsz, tlen, heads, LATENT)),
        "lse": np.full((bsz, tlen, heads), -np.inf),
    }
    for b in (range(bsz) if requests is None else requests):
        c_b, n_b = request_keys(pool, block_table, kv_bounds, b, decode)
        for h in range(heads):
            k_h = c_b @ wk[h].T
            v_h = c_b @ wv[h].T
            for t in range(tlen):
                L = token_bound(kv_bounds, b, t, n_b)
                if L == 0:
                    continue
                s = sm_scale * (k_h[:L] @ qn[b, t, h])
                m = s.max()
                w = np.exp(s - m)
                total = w.sum()
                p = w / total
                res["lse"][b, t, h] = m + np.log(total)
                res["o_v"][b, t, h] = p @ v_h[:L]
                res["o_lat"][b, t, h] = p @ c_b[:L]
    res["out"] = res["o_v"] * g if g is not None else None
    return res


def gated_output(o_lat, w_uv, gate) -> np.ndarray:
    """out[b,t,h] = sigmoid(gate[b,t,h]) * (W_UV[h] o_lat[b,t,h])   (512 -> 128)."""
    wv = bf16_to_f64(w_uv)
    o_v = np.einsum("hdc,bthc->bthd", wv, np.asarray(o_lat, dtype=np.float64))
    return sigmoid(bf16_to_f64(gate)) * o_v


# ----------------------------------------------------------------- split-KV
def attend_chunk(q_row, c_rows, sm_scale):
    """Partial result of one query row over one chunk of keys: (o, lse).

    An empty chunk returns the identity (o = 0, lse = -inf).
    """
    if c_rows.shape[0] == 0:
        return np.zeros(c_rows.shape[1]), -np.inf
    o, lse = softmax_attend(sm_scale * (c_rows @ q_row), c_rows)
    return o, float(lse)


def lse_merge(partials):
    """Merge partial (o_s, lse_s) results of disjoint key chunks.

    lse = log sum_s exp(lse_s); o = sum_s exp(lse_s - lse) o_s.
    Chunks with lse_s = -inf carry no weight; if every chunk is empty the
    result is the identity (o = 0, lse = -inf), never NaN.
    """
    lses = np.array([float(l) for _, l in partials])
    dim = np.asarray(partials[0][0]).shape
    finite = np.isfinite(lses)
    if not finite.any():
        return np.zeros(dim), -np.inf
    m = lses[finite].max()
    w = np.where(finite, np.exp(np.where(finite, lses - m, 0.0)), 0.0)
    total = w.sum()
    lse = m + np.log(total)
    o = np.zeros(dim)
    for (o_s, _), w_s in zip(partials, w):
        if w_s > 0:
            o = o + (w_s / total) * np.asarray(o_s, dtype=np.float64)
    return o, lse


def split_pages(n_keys: int, num_splits: int):
    """The contiguous, page-aligned key chunks used for split-KV.

    With n_pg = ceil(n_keys / 64) pages, chunk c covers pages
    [floor(c n_pg / S), floor((c+1) n_pg / S)); its key range is clipped to
    n_keys.  A chunk may be empty.  Returns a list of (start, stop) keys.
    """
    n_pg = -(-n_keys // PAGE)
    out = []
    for c in range(num_splits):
        p0 = (c * n_pg) // num_splits
        p1 = ((c + 1) * n_pg) // num_splits
        out.append((min(p0 * PAGE, n_keys), min(p1 * PAGE, n_keys)))
    return out
