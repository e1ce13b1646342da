"""MI355X-native speculative-verify attention for gated NoPE MLA (absorbed projections).

Thin Python binding over the C ABI in ``include/mla_verify.h``: it checks and
marshals torch tensors (device memory) and the current HIP stream into the
library's plain-pointer entry points.  Every step of the computation runs in
the library's HIP kernels; there is no fallback path.  If
``libmla_verify.so`` has not been built, every call raises.

Entry points (same names as the C ABI, without the ``mla_`` prefix):
    verify_attn(...)        -> (out_latent [B,T,H,512] bf16, lse [B,T,H] f32)
    verify_attn_gated(...)  -> (out [B,T,H,128] bf16, lse, out_latent or None)
    verify_attn_gated_noalloc(...) -> the same into caller-given outputs, with the
                            library's static device scratch instead of a workspace
    verify_absorb_q(...)    -> q_latent [B,T,H,512] bf16
    verify_kv_append(...)   -> None (writes the group's latents into the pool by slot table)
    verify_kv_trim(...)     -> (new_len [B] i32, released_page [B] i32); block_table updated
    verify_attn_partials(...) -> (part_o [S,B*T*H,512] bf16, part_lse [S,B*T*H] f32)
    verify_lse_combine(...) -> (out_latent [rows,512] bf16, lse [rows] f32)
    verify_check / verify_num_splits / verify_tile_rows / verify_workspace_size / status_string
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os

__all__ = [
    "MlaVerifyError", "VerifyParams", "lib_path", "load_library", "verify_check",
    "verify_num_splits", "verify_tile_rows", "verify_workspace_size", "verify_attn",
    "verify_attn_gated", "verify_attn_gated_noalloc",
    "verify_absorb_q", "verify_attn_partials", "verify_lse_combine", "verify_kv_append",
    "verify_kv_trim", "status_string",
    "EXPORTED_SYMBOLS",
]

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_FILE = os.path.join(_PKG_DIR, "libmla_verify.so")

MLA_OK = 0
STATUS = {0: "MLA_OK", -1: "MLA_ERR_NULL", -2: "MLA_ERR_SHAPE", -3: "MLA_ERR_DTYPE",
          -4: "MLA_ERR_ARG", -5: "MLA_ERR_WORKSPACE", -6: "MLA_ERR_DEVICE", -7: "MLA_ERR_HIP"}
KV_BF16, KV_FP8_E4M3 = 0, 1
LATENT, PAGE, NOPE = 512, 64, 128

EXPORTED_SYMBOLS = [
    "mla_verify_check", "mla_verify_num_splits", "mla_verify_tile_rows", "mla_verify_workspace_size",
    "mla_verify_attn", "mla_verify_attn_partials", "mla_verify_lse_combine",
    "mla_verify_attn_gated", "mla_verify_attn_gated_noalloc", "mla_verify_absorb_q",
    "mla_verify_kv_append", "mla_verify_kv_trim", "mla_verify_status_string",
]
STATIC_SCRATCH_BYTES = 64 << 20     # MLA_VERIFY_STATIC_SCRATCH_BYTES


class MlaVerifyError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = status_string(code) if _LIB is not None else STATUS.get(code, "?")
        super().__init__(f"{where}: {STATUS.get(code, code)} ({msg})")


class VerifyParams(ctypes.Structure):
    """Mirror of ``mla_verify_params``."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("q_len", ctypes.c_int32), ("num_heads", ctypes.c_int32),
        ("latent_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("max_pages_per_req", ctypes.c_int32), ("num_pool_pages", ctypes.c_int32),
        ("num_splits", ctypes.c_int32), ("sm_scale", ctypes.c_float), ("kv_dtype", ctypes.c_int32),
        ("tile_rows", ctypes.c_int32), ("kv_scale", ctypes.c_float),
    ]

    @classmethod
    def make(cls, batch, q_len, num_heads, max_pages_per_req, num_pool_pages, sm_scale,
             num_splits=0, latent_dim=LATENT, page_size=PAGE, kv_dtype=KV_BF16, tile_rows=0,
             kv_scale=1.0):
        return cls(int(batch), int(q_len), int(num_heads), int(latent_dim), int(page_size),
                   int(max_pages_per_req), int(num_pool_pages), int(num_splits), float(sm_scale),
                   int(kv_dtype), int(tile_rows), float(kv_scale))


_LIB = None


def lib_path() -> str:
    return _LIB_FILE


def load_library():
    """Load ``libmla_verify.so`` (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(_LIB_FILE):
        raise RuntimeError(f"{_LIB_FILE} is missing: build it with "
                           "`python -m speculative_verify_attention_absorbed_amd._build`")
    lib = ctypes.CDLL(_LIB_FILE)
    P = ctypes.POINTER(VerifyParams)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.mla_verify_check.argtypes = [P]
    lib.mla_verify_check.restype = ctypes.c_int
    lib.mla_verify_num_splits.argtypes = [P, ctypes.c_int]
    lib.mla_verify_num_splits.restype = ctypes.c_int
    lib.mla_verify_tile_rows.argtypes = [P, ctypes.c_int]
    lib.mla_verify_tile_rows.restype = ctypes.c_int
    lib.mla_verify_workspace_size.argtypes = [P, ctypes.c_int, ctypes.POINTER(sz)]
    lib.mla_verify_workspace_size.restype = ctypes.c_int
    lib.mla_verify_attn.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.mla_verify_attn.restype = ctypes.c_int
    lib.mla_verify_attn_gated.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.mla_verify_attn_gated.restype = ctypes.c_int
    lib.mla_verify_attn_gated_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.mla_verify_attn_gated_noalloc.restype = ctypes.c_int
    lib.mla_verify_attn_partials.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    lib.mla_verify_attn_partials.restype = ctypes.c_int
    lib.mla_verify_lse_combine.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp]
    lib.mla_verify_lse_combine.restype = ctypes.c_int
    lib.mla_verify_absorb_q.argtypes = [P, vp, vp, vp, vp]
    lib.mla_verify_absorb_q.restype = ctypes.c_int
    i = ctypes.c_int
    lib.mla_verify_kv_append.argtypes = [i, i, i, i, vp, vp, vp, vp, vp, vp]
    lib.mla_verify_kv_append.restype = ctypes.c_int
    lib.mla_verify_kv_trim.argtypes = [i, i, i, vp, vp, vp, vp, vp, vp]
    lib.mla_verify_kv_trim.restype = ctypes.c_int
    lib.mla_verify_status_string.argtypes = [ctypes.c_int]
    lib.mla_verify_status_string.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def status_string(code: int) -> str:
    return load_library().mla_verify_status_string(int(code)).decode()


def _check(rc: int, where: str):
    if rc != MLA_OK:
        raise MlaVerifyError(rc, where)


def verify_check(params: VerifyParams) -> int:
    return load_library().mla_verify_check(ctypes.byref(params))


def verify_num_splits(params: VerifyParams, gated: bool = False) -> int:
    rc = load_library().mla_verify_num_splits(ctypes.byref(params), int(bool(gated)))
    if rc < 0:
        raise MlaVerifyError(rc, "mla_verify_num_splits")
    return rc


def verify_tile_rows(params: VerifyParams, gated: bool = False) -> int:
    rc = load_library().mla_verify_tile_rows(ctypes.byref(params), int(bool(gated)))
    if rc < 0:
        raise MlaVerifyError(rc, "mla_verify_tile_rows")
    return rc


def verify_workspace_size(params: VerifyParams, gated: bool = False) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().mla_verify_workspace_size(ctypes.byref(params), int(bool(gated)),
                                                    ctypes.byref(out)), "mla_verify_workspace_size")
    return int(out.value)


# ---------------------------------------------------------------- tensor glue
def _torch():
    import torch
    return torch


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _dev_tensor(t, name, shape, dtypes):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live in GPU memory (got {t.device})")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _bf16_types():
    torch = _torch()
    return (torch.bfloat16, torch.int16, torch.uint16)


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _alloc_on(stream):
    """Context in which this module allocates outputs and workspaces: the
    stream the kernels run on.  torch's caching allocator then returns a
    freed block to that stream's pool only, so it is not handed to other
    work while the call's kernels may still use it.  A raw stream handle has
    no torch stream to allocate on; calls given one must bring their own
    workspace (checked by the callers)."""
    torch = _torch()
    if stream is None or not hasattr(stream, "cuda_stream"):
        return contextlib.nullcontext()
    return torch.cuda.stream(stream)


def _raw_stream(stream):
    return stream is not None and not hasattr(stream, "cuda_stream")


def _params_from(q_latent, pool, block_table, sm_scale, num_splits, kv_dtype, tile_rows=0,
                 kv_scale=1.0):
    b, t, h, d = q_latent.shape
    return VerifyParams.make(b, t, h, block_table.shape[1], pool.shape[0], sm_scale, num_splits,
                             latent_dim=d, page_size=pool.shape[1] if pool.dim() == 3 else PAGE,
                             kv_dtype=kv_dtype, tile_rows=tile_rows, kv_scale=kv_scale)


def _pool_types(kv_dtype):
    """Element types accepted for the latent cache: bf16, or 8-bit codes."""
    torch = _torch()
    if int(kv_dtype) == KV_FP8_E4M3:
        return tuple(t for t in (torch.uint8, getattr(torch, "float8_e4m3fn", None)) if t is not None)
    return _bf16_types()


def _workspace(params, gated, workspace, device, stream=None):
    """The call's workspace: the caller's, or one allocated on the call's
    stream (a raw stream handle requires the caller's)."""
    torch = _torch()
    need = verify_workspace_size(params, gated)
    if need == 0:
        return None, 0
    if workspace is None:
        if _raw_stream(stream):
            raise ValueError("a raw stream handle needs a caller-owned workspace of "
                             f"{need} bytes (verify_workspace_size)")
        with _alloc_on(stream):
            workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    nbytes = workspace.numel() * workspace.element_size()
    return workspace, nbytes


def verify_attn(q_latent, latent_kv_pages, block_table, kv_bounds, sm_scale, *, num_splits=0,
                out_latent=None, lse=None, workspace=None, stream=None, kv_dtype=KV_BF16,
                tile_rows=0, kv_scale=1.0):
    """``mla_verify_attn``: returns (out_latent, lse).  Outputs and workspace are
    allocated with torch when not given (allocation happens here, outside the
    library)."""
    torch = _torch()
    params = _params_from(q_latent, latent_kv_pages, block_table, sm_scale, num_splits, kv_dtype,
                          tile_rows, kv_scale)
    _check(verify_check(params), "mla_verify_attn")
    b, t, h, d = q_latent.shape
    bf = _bf16_types()
    _dev_tensor(q_latent, "q_latent", (b, t, h, LATENT), bf)
    _dev_tensor(latent_kv_pages, "latent_kv_pages", (latent_kv_pages.shape[0], PAGE, LATENT),
                _pool_types(kv_dtype))
    _dev_tensor(block_table, "block_table", (b, block_table.shape[1]), (torch.int32,))
    _dev_tensor(kv_bounds, "kv_bounds", (b, t), (torch.int32,))
    dev = q_latent.device
    with _alloc_on(stream):
        if out_latent is None:
            out_latent = torch.empty((b, t, h, LATENT), dtype=torch.bfloat16, device=dev)
        if lse is None:
            lse = torch.empty((b, t, h), dtype=torch.float32, device=dev)
    _dev_tensor(out_latent, "out_latent", (b, t, h, LATENT), bf)
    _dev_tensor(lse, "lse", (b, t, h), (torch.float32,))
    workspace, nbytes = _workspace(params, False, workspace, dev, stream)
    rc = load_library().mla_verify_attn(
        ctypes.byref(params), _ptr(q_latent), _ptr(latent_kv_pages), _ptr(block_table),
        _ptr(kv_bounds), _ptr(out_latent), _ptr(lse), _ptr(workspace), ctypes.c_size_t(nbytes),
        _stream(stream))
    _check(rc, "mla_verify_attn")
    return out_latent, lse


def verify_attn_gated(q_latent, latent_kv_pages, block_table, kv_bounds, w_uv, gate_logits,
                      sm_scale, *, num_splits=0, out=None, lse=None, out_latent=None,
                      want_latent=False, workspace=None, stream=None, kv_dtype=KV_BF16,
                      tile_rows=0, kv_scale=1.0):
    """``mla_verify_attn_gated``: returns (out, lse, out_latent or None)."""
    torch = _torch()
    params = _params_from(q_latent, latent_kv_pages, block_table, sm_scale, num_splits, kv_dtype,
                          tile_rows, kv_scale)
    _check(verify_check(params), "mla_verify_attn_gated")
    b, t, h, d = q_latent.shape
    bf = _bf16_types()
    _dev_tensor(q_latent, "q_latent", (b, t, h, LATENT), bf)
    _dev_tensor(latent_kv_pages, "latent_kv_pages", (latent_kv_pages.shape[0], PAGE, LATENT),
                _pool_types(kv_dtype))
    _dev_tensor(block_table, "block_table", (b, block_table.shape[1]), (torch.int32,))
    _dev_tensor(kv_bounds, "kv_bounds", (b, t), (torch.int32,))
    _dev_tensor(w_uv, "w_uv", (h, NOPE, LATENT), bf)
    _dev_tensor(gate_logits, "gate_logits", (b, t, h, NOPE), bf)
    dev = q_latent.device
    with _alloc_on(stream):
        if out is None:
            out = torch.empty((b, t, h, NOPE), dtype=torch.bfloat16, device=dev)
        if lse is None:
            lse = torch.empty((b, t, h), dtype=torch.float32, device=dev)
        if out_latent is None and want_latent:
            out_latent = torch.empty((b, t, h, LATENT), dtype=torch.bfloat16, device=dev)
    _dev_tensor(out, "out", (b, t, h, NOPE), bf)
    _dev_tensor(lse, "lse", (b, t, h), (torch.float32,))
    if out_latent is not None:
        _dev_tensor(out_latent, "out_latent", (b, t, h, LATENT), bf)
    workspace, nbytes = _workspace(params, True, workspace, dev, stream)
    rc = load_library().mla_verify_attn_gated(
        ctypes.byref(params), _ptr(q_latent), _ptr(latent_kv_pages), _ptr(block_table),
        _ptr(kv_bounds), _ptr(w_uv), _ptr(gate_logits), _ptr(out), _ptr(lse), _ptr(out_latent),
        _ptr(workspace), ctypes.c_size_t(nbytes), _stream(stream))
    _check(rc, "mla_verify_attn_gated")
    return out, lse, out_latent


def verify_attn_gated_noalloc(q_latent, latent_kv_pages, block_table, kv_bounds, w_uv,
                              gate_logits, sm_scale, out, lse, *, out_latent=None, num_splits=0,
                              stream=None, kv_dtype=KV_BF16, tile_rows=0, kv_scale=1.0):
    """``mla_verify_attn_gated_noalloc``: writes (out, lse, out_latent if given).
    Every output is the caller's; the library allocates nothing, and its
    static scratch is shared by all calls on a GPU (overlapping calls race)."""
    torch = _torch()
    params = _params_from(q_latent, latent_kv_pages, block_table, sm_scale, num_splits, kv_dtype,
                          tile_rows, kv_scale)
    _check(verify_check(params), "mla_verify_attn_gated_noalloc")
    b, t, h, d = q_latent.shape
    bf = _bf16_types()
    _dev_tensor(q_latent, "q_latent", (b, t, h, LATENT), bf)
    _dev_tensor(latent_kv_pages, "latent_kv_pages", (latent_kv_pages.shape[0], PAGE, LATENT),
                _pool_types(kv_dtype))
    _dev_tensor(block_table, "block_table", (b, block_table.shape[1]), (torch.int32,))
    _dev_tensor(kv_bounds, "kv_bounds", (b, t), (torch.int32,))
    _dev_tensor(w_uv, "w_uv", (h, NOPE, LATENT), bf)
    _dev_tensor(gate_logits, "gate_logits", (b, t, h, NOPE), bf)
    _dev_tensor(out, "out", (b, t, h, NOPE), bf)
    _dev_tensor(lse, "lse", (b, t, h), (torch.float32,))
    if out_latent is not None:
        _dev_tensor(out_latent, "out_latent", (b, t, h, LATENT), bf)
    rc = load_library().mla_verify_attn_gated_noalloc(
        ctypes.byref(params), _ptr(q_latent), _ptr(latent_kv_pages), _ptr(block_table),
        _ptr(kv_bounds), _ptr(w_uv), _ptr(gate_logits), _ptr(out), _ptr(lse), _ptr(out_latent),
        _stream(stream))
    _check(rc, "mla_verify_attn_gated_noalloc")
    return out, lse, out_latent


def verify_attn_partials(q_latent, latent_kv_pages, block_table, kv_bounds, sm_scale, *,
                         num_splits=0, part_o=None, part_lse=None, stream=None,
                         kv_dtype=KV_BF16, tile_rows=0, kv_scale=1.0):
    """``mla_verify_attn_partials``: returns (part_o [S, B*T*H, 512] bf16,
    part_lse [S, B*T*H] f32) with S = verify_num_splits(params)."""
    torch = _torch()
    params = _params_from(q_latent, latent_kv_pages, block_table, sm_scale, num_splits, kv_dtype,
                          tile_rows, kv_scale)
    _check(verify_check(params), "mla_verify_attn_partials")
    b, t, h, d = q_latent.shape
    bf = _bf16_types()
    _dev_tensor(q_latent, "q_latent", (b, t, h, LATENT), bf)
    _dev_tensor(latent_kv_pages, "latent_kv_pages", (latent_kv_pages.shape[0], PAGE, LATENT),
                _pool_types(kv_dtype))
    _dev_tensor(block_table, "block_table", (b, block_table.shape[1]), (torch.int32,))
    _dev_tensor(kv_bounds, "kv_bounds", (b, t), (torch.int32,))
    s = verify_num_splits(params)
    rows = b * t * h
    dev = q_latent.device
    with _alloc_on(stream):
        if part_o is None:
            part_o = torch.empty((s, rows, LATENT), dtype=torch.bfloat16, device=dev)
        if part_lse is None:
            part_lse = torch.empty((s, rows), dtype=torch.float32, device=dev)
    _dev_tensor(part_o, "part_o", (s, rows, LATENT), bf)
    _dev_tensor(part_lse, "part_lse", (s, rows), (torch.float32,))
    rc = load_library().mla_verify_attn_partials(
        ctypes.byref(params), _ptr(q_latent), _ptr(latent_kv_pages), _ptr(block_table),
        _ptr(kv_bounds), _ptr(part_o), _ptr(part_lse), _stream(stream))
    _check(rc, "mla_verify_attn_partials")
    return part_o, part_lse


def verify_lse_combine(part_o, part_lse, *, out_latent=None, lse=None, stream=None):
    """``mla_verify_lse_combine``: merges [S, rows, 512] partials into
    (out_latent [rows, 512] bf16, lse [rows] f32)."""
    torch = _torch()
    bf = _bf16_types()
    if part_o.dim() != 3 or part_lse.dim() != 2:
        raise ValueError("part_o must be [S, rows, 512] and part_lse [S, rows]")
    s, rows, _ = part_o.shape
    _dev_tensor(part_o, "part_o", (s, rows, LATENT), bf)
    _dev_tensor(part_lse, "part_lse", (s, rows), (torch.float32,))
    dev = part_o.device
    with _alloc_on(stream):
        if out_latent is None:
            out_latent = torch.empty((rows, LATENT), dtype=torch.bfloat16, device=dev)
        if lse is None:
            lse = torch.empty((rows,), dtype=torch.float32, device=dev)
    _dev_tensor(out_latent, "out_latent", (rows, LATENT), bf)
    _dev_tensor(lse, "lse", (rows,), (torch.float32,))
    rc = load_library().mla_verify_lse_combine(int(s), int(rows), _ptr(part_o), _ptr(part_lse),
                                               _ptr(out_latent), _ptr(lse), _stream(stream))
    _check(rc, "mla_verify_lse_combine")
    return out_latent, lse


def verify_absorb_q(q_nope, w_uk, *, q_latent=None, stream=None):
    """``mla_verify_absorb_q``: q_latent = W_UK[h]^T q_nope, bf16."""
    torch = _torch()
    b, t, h, dn = q_nope.shape
    bf = _bf16_types()
    _dev_tensor(q_nope, "q_nope", (b, t, h, NOPE), bf)
    _dev_tensor(w_uk, "w_uk", (h, NOPE, LATENT), bf)
    if q_latent is None:
        with _alloc_on(stream):
            q_latent = torch.empty((b, t, h, LATENT), dtype=torch.bfloat16, device=q_nope.device)
    _dev_tensor(q_latent, "q_latent", (b, t, h, LATENT), bf)
    params = VerifyParams.make(b, t, h, 1, 1, 1.0 / math.sqrt(NOPE))
    rc = load_library().mla_verify_absorb_q(ctypes.byref(params), _ptr(q_nope), _ptr(w_uk),
                                            _ptr(q_latent), _stream(stream))
    _check(rc, "mla_verify_absorb_q")
    return q_latent


def verify_kv_append(new_latent, slots, block_table, latent_kv_pages, *, bad_slots=None, stream=None):
    """``mla_verify_kv_append``: for every (b, t) with 0 <= slots[b, t] < P*64,
    latent_kv_pages[block_table[b, slot // 64], slot % 64] = new_latent[b, t]
    (in place).  ``bad_slots`` (int32 [1], optional) counts out-of-range
    entries; -1 entries are skipped silently."""
    torch = _torch()
    bf = _bf16_types()
    if new_latent.dim() != 3 or block_table.dim() != 2 or latent_kv_pages.dim() != 3:
        raise ValueError("new_latent must be [B, T, 512], block_table [B, P], pool [N, 64, 512]")
    b, t, _ = new_latent.shape
    p = block_table.shape[1]
    n = latent_kv_pages.shape[0]
    _dev_tensor(new_latent, "new_latent", (b, t, LATENT), bf)
    _dev_tensor(slots, "slots", (b, t), (torch.int32,))
    _dev_tensor(block_table, "block_table", (b, p), (torch.int32,))
    _dev_tensor(latent_kv_pages, "latent_kv_pages", (n, PAGE, LATENT), bf)
    if bad_slots is not None:
        _dev_tensor(bad_slots, "bad_slots", (1,), (torch.int32,))
    rc = load_library().mla_verify_kv_append(int(b), int(t), int(p), int(n), _ptr(new_latent), _ptr(slots),
                                             _ptr(block_table), _ptr(latent_kv_pages), _ptr(bad_slots),
                                             _stream(stream))
    _check(rc, "mla_verify_kv_append")


def verify_kv_trim(kv_len, accepted, block_table, q_len, *, new_len=None, released_page=None, stream=None):
    """``mla_verify_kv_trim``: drops the rejected tail of every request's group
    (block_table is updated in place).  Returns (new_len, released_page)."""
    torch = _torch()
    if block_table.dim() != 2:
        raise ValueError("block_table must be [B, P]")
    b, p = block_table.shape
    i32 = (torch.int32,)
    _dev_tensor(kv_len, "kv_len", (b,), i32)
    _dev_tensor(accepted, "accepted", (b,), i32)
    _dev_tensor(block_table, "block_table", (b, p), i32)
    with _alloc_on(stream):
        if new_len is None:
            new_len = torch.empty((b,), dtype=torch.int32, device=kv_len.device)
        if released_page is None:
            released_page = torch.empty((b,), dtype=torch.int32, device=kv_len.device)
    _dev_tensor(new_len, "new_len", (b,), i32)
    _dev_tensor(released_page, "released_page", (b,), i32)
    rc = load_library().mla_verify_kv_trim(int(b), int(q_len), int(p), _ptr(kv_len), _ptr(accepted),
                                           _ptr(new_len), _ptr(block_table), _ptr(released_page),
                                           _stream(stream))
    _check(rc, "mla_verify_kv_trim")
    return new_len, released_page
