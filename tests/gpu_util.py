"""Helpers for the GPU parity tests: upload seeded inputs, compare results."""
import math

import numpy as np
import torch

from verify_inputs import FP8_NAN, LATENT, PAGE, VerifyInputs, f32_to_bf16_bits

# acceptance bar for floating-point outputs and LSE
MAX_ABS = 1e-2
REL_L2 = 5e-3
LSE_ABS = 1e-3
# per-row bar (every (b, t, h) row against its own oracle row): the global
# relative L2 above is a norm over all rows, under which one wrong row among
# thousands can hide; bf16 outputs, bf16 softmax weights and bf16 partials
# give each row about 2e-3 to 3e-3, so 1e-2 still fails a row that is off
# by a few per cent
ROW_REL_L2 = 1e-2


def dev():
    return torch.device("cuda:0")


def bf16_tensor(bits: np.ndarray, device=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device or dev())


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def upload_pool(x: VerifyInputs, device=None) -> torch.Tensor:
    """Dense device pool: referenced pages from the generator, NaN elsewhere."""
    device = device or dev()
    pool = torch.full((x.pool.num_pages, PAGE, LATENT), float("nan"), dtype=torch.bfloat16,
                      device=device)
    if x.pool.page_ids.size:
        ids = torch.from_numpy(x.pool.page_ids.astype(np.int64)).to(device)
        pool[ids] = bf16_tensor(x.pool.pages, device)
    return pool


def upload_dense_pool(pool_bits: np.ndarray, device=None) -> torch.Tensor:
    return bf16_tensor(pool_bits, device)


def upload(x: VerifyInputs, device=None, q_latent_bits=None):
    device = device or dev()
    d = {
        "pool": upload_pool(x, device),
        "block_table": torch.from_numpy(x.block_table).to(device),
        "kv_bounds": torch.from_numpy(x.kv_bounds).to(device),
        "q_nope": bf16_tensor(x.q_nope, device),
        "w_uk": bf16_tensor(x.w_uk, device),
        "w_uv": bf16_tensor(x.w_uv, device),
        "gate": bf16_tensor(x.gate, device),
    }
    ql = q_latent_bits if q_latent_bits is not None else x.q_latent
    if ql is not None:
        d["q_latent"] = bf16_tensor(ql, device)
    return d


def round_bf16(a64: np.ndarray) -> np.ndarray:
    """Host-side RNE rounding of float64 values to bf16 bits (via float32)."""
    return f32_to_bf16_bits(np.asarray(a64, dtype=np.float32))


def row_rel_l2(got: np.ndarray, want: np.ndarray) -> np.ndarray:
    """Relative L2 error of every row (last axis = the row's values).  A row
    whose oracle value is exactly zero (no visible key) must be exactly zero:
    its entry is the absolute L2 of the result then."""
    g = got.reshape(-1, got.shape[-1])
    w = want.reshape(-1, want.shape[-1])
    num = np.linalg.norm(g - w, axis=1)
    den = np.linalg.norm(w, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def assert_close_output(got: np.ndarray, want: np.ndarray, what: str, mask_rows=None):
    """Acceptance bar on outputs: max-abs <= 1e-2 and relative L2 <= 5e-3
    over the whole output, and relative L2 <= 1e-2 on every row.  Prints the
    measured errors."""
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    diff = got - want
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    denom = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(diff)) / denom if denom > 0 else float(np.linalg.norm(diff))
    rows = row_rel_l2(got, want) if diff.size else np.zeros(1)
    worst = int(np.argmax(rows))
    log(f"  {what}: max abs {max_abs:.3e}, rel L2 {rel:.3e}, worst row rel L2 {rows[worst]:.3e} "
        f"(row {worst} of {rows.size})")
    assert max_abs <= MAX_ABS, f"{what}: max abs error {max_abs:.3e}"
    assert rel <= REL_L2, f"{what}: relative L2 error {rel:.3e}"
    assert rows[worst] <= ROW_REL_L2, f"{what}: row {worst} relative L2 error {rows[worst]:.3e}"
    return max_abs, rel


def assert_lse(got: np.ndarray, want: np.ndarray, what="lse"):
    """Finite LSEs within 1e-3; masked rows exactly -inf."""
    inf_w = np.isneginf(want)
    assert np.array_equal(np.isneginf(got), inf_w), f"{what}: -inf pattern differs"
    assert not np.isnan(got).any(), f"{what}: NaN"
    fin = ~inf_w
    if fin.any():
        err = float(np.abs(got[fin] - want[fin]).max())
        log(f"  {what}: max abs error {err:.3e} over {int(fin.sum())} finite rows")
        assert err <= LSE_ABS, f"{what}: max abs error {err:.3e}"


def assert_masked_rows_zero(out: np.ndarray, lse_want: np.ndarray, what="out"):
    rows = np.isneginf(lse_want)
    if rows.any():
        assert np.all(out[rows] == 0), f"{what}: masked rows are not exactly 0"


def sync():
    torch.cuda.synchronize()


def log(msg):
    print(msg, flush=True)


def rel_l2(a, b):
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / n) if n > 0 else float(np.linalg.norm(a - b))


def sm_scale():
    return 1.0 / math.sqrt(128)


def upload_fp8(x, q_latent_bits=None):
    """Device inputs with the pool as E4M3 codes (uint8), NaN code elsewhere."""
    dev = torch.device("cuda:0")
    pool = torch.full((x.pool.num_pages, PAGE, LATENT), int(FP8_NAN), dtype=torch.uint8, device=dev)
    if x.pool.page_ids.size:
        ids = torch.from_numpy(x.pool.page_ids.astype(np.int64)).to(dev)
        pool[ids] = torch.from_numpy(np.ascontiguousarray(x.pool.pages)).to(dev)
    d = {
        "pool": pool,
        "block_table": torch.from_numpy(x.block_table).to(dev),
        "kv_bounds": torch.from_numpy(x.kv_bounds).to(dev),
        "w_uv": bf16_tensor(x.w_uv),
        "gate": bf16_tensor(x.gate),
    }
    ql = q_latent_bits if q_latent_bits is not None else x.q_latent
    d["q_latent"] = bf16_tensor(ql)
    return d
