"""Host-side checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments before any HIP call (these run
without a GPU)."""
import ctypes
import math
import os
import re

import pytest

import speculative_verify_attention_absorbed_amd as mv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mv.lib_path()):
        from speculative_verify_attention_absorbed_amd import _build
        _build.build()
    return mv.load_library()


def header_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(mla_\w+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported(lib):
    declared = header_functions()
    assert set(declared) == set(mv.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


def good(**kw):
    base = dict(batch=16, q_len=8, num_heads=8, max_pages_per_req=24, num_pool_pages=4096,
                sm_scale=1 / math.sqrt(128))
    base.update(kw)
    return mv.VerifyParams.make(**base)


def test_check_accepts_valid(lib):
    assert mv.verify_check(good()) == 0
    assert mv.verify_check(good(q_len=16, num_heads=128)) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(latent_dim=576), -2), (dict(page_size=32), -2), (dict(q_len=0), -2),
    (dict(q_len=17), -2), (dict(num_heads=0), -2), (dict(num_heads=129), -2), (dict(batch=0), -2),
    (dict(kv_dtype=7), -3), (dict(kv_dtype=-1), -3),
    (dict(kv_dtype=1, kv_scale=0.0), -4), (dict(kv_dtype=1, kv_scale=-0.5), -4),
    (dict(kv_dtype=1, kv_scale=float("nan")), -4), (dict(kv_dtype=1, kv_scale=float("inf")), -4),
    (dict(sm_scale=0.0), -4), (dict(sm_scale=-1.0), -4), (dict(sm_scale=float("nan")), -4),
    (dict(sm_scale=float("inf")), -4), (dict(num_splits=-1), -4), (dict(num_splits=65), -4),
    (dict(max_pages_per_req=0), -4), (dict(num_pool_pages=0), -4),
    (dict(tile_rows=16), -4), (dict(tile_rows=96), -4), (dict(tile_rows=-1), -4),
])
def test_check_rejects(lib, kw, code):
    assert mv.verify_check(good(**kw)) == code


def test_null_params(lib):
    assert lib.mla_verify_check(None) == -1
    assert lib.mla_verify_workspace_size(ctypes.byref(good()), 0, None) == -1


def test_fp8_kv_takes_a_scale(lib):
    # an fp8 cache plans like a bf16 one; its scale must be finite and positive
    p = good(kv_dtype=mv.KV_FP8_E4M3, kv_scale=2.0 ** -8)
    assert mv.verify_check(p) == 0
    assert mv.verify_workspace_size(p) == mv.verify_workspace_size(good())
    assert mv.verify_num_splits(p) == mv.verify_num_splits(good())
    with pytest.raises(mv.MlaVerifyError, match="MLA_ERR_ARG"):
        mv.verify_workspace_size(good(kv_dtype=mv.KV_FP8_E4M3, kv_scale=0.0))
    # the bf16 path ignores the field
    assert mv.verify_check(good(kv_scale=-3.0)) == 0


def test_split_plan_and_workspace(lib):
    # forced split counts are honoured; direct (unsplit, ungated) needs no workspace
    p1 = good(num_splits=1)
    assert mv.verify_num_splits(p1) == 1 and mv.verify_workspace_size(p1) == 0
    rows = 16 * 8 * 8
    p4 = good(num_splits=4)
    assert mv.verify_num_splits(p4) == 4
    assert mv.verify_workspace_size(p4) == 4 * rows * (512 * 2 + 4)   # bf16 partials + fp32 LSEs
    # the gated path always stages partials
    assert mv.verify_workspace_size(p1, gated=True) == rows * (512 * 2 + 4)
    # automatic choice: one workgroup per CU, at least one split per 16 pages
    # of the longest request, never more splits than pages (or than 64)
    for b, t, h, pmax in [(16, 8, 8, 24), (64, 1, 64, 24), (1, 4, 8, 4), (64, 8, 64, 128),
                          (1, 1, 1, 1), (512, 8, 64, 24), (2, 16, 128, 2000)]:
        p = good(batch=b, q_len=t, num_heads=h, max_pages_per_req=pmax)
        s = mv.verify_num_splits(p)
        tiles = b * -(-(t * h) // mv.verify_tile_rows(p))
        want = max(256 // tiles, -(-pmax // 16), 1)
        assert s == min(want, pmax, 64), (b, t, h, pmax, s)


def test_status_strings(lib):
    for code in range(-7, 1):
        assert mv.status_string(code)
    assert mv.status_string(-99) == "unknown status"


def test_entry_points_validate_before_any_hip_call(lib):
    """Bad arguments come back as error codes, with no device touched."""
    p = good()
    fake = ctypes.c_void_p(0x1000)
    z = ctypes.c_void_p(0)
    args = [fake] * 6
    # NULL pointers
    assert lib.mla_verify_attn(ctypes.byref(p), z, *args[1:], z, 0, z) == -1
    assert lib.mla_verify_attn_gated(ctypes.byref(p), fake, fake, fake, fake, z, fake, fake, fake,
                                     z, fake, 1 << 30, z) == -1
    assert lib.mla_verify_absorb_q(ctypes.byref(p), z, fake, fake, z) == -1
    # misaligned pointer
    odd = ctypes.c_void_p(0x1002)
    assert lib.mla_verify_attn(ctypes.byref(good(num_splits=1)), odd, *args[1:], z, 0, z) == -4
    # workspace too small (split plan needs partials)
    p4 = good(num_splits=4)
    assert lib.mla_verify_attn(ctypes.byref(p4), *args, z, 0, z) == -5
    assert lib.mla_verify_attn(ctypes.byref(p4), *args, fake, 16, z) == -5
    assert lib.mla_verify_attn_gated(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake,
                                     fake, z, z, 0, z) == -5
    # partial-only and combine entry points
    assert lib.mla_verify_attn_partials(ctypes.byref(p), fake, fake, fake, fake, z, fake, z) == -1
    assert lib.mla_verify_attn_partials(ctypes.byref(p), fake, odd, fake, fake, fake, fake, z) == -4
    assert lib.mla_verify_attn_partials(ctypes.byref(good(page_size=32)), fake, fake, fake, fake,
                                        fake, fake, z) == -2
    assert lib.mla_verify_lse_combine(0, 8, fake, fake, fake, fake, z) == -4
    assert lib.mla_verify_lse_combine(65, 8, fake, fake, fake, fake, z) == -4
    assert lib.mla_verify_lse_combine(4, 0, fake, fake, fake, fake, z) == -4
    assert lib.mla_verify_lse_combine(4, 8, fake, z, fake, fake, z) == -1
    assert lib.mla_verify_lse_combine(4, 8, fake, fake, odd, fake, z) == -4
    # bad params take precedence over everything else
    assert lib.mla_verify_attn(ctypes.byref(good(latent_dim=576)), z, *args[1:], z, 0, z) == -2
    assert lib.mla_verify_attn(None, *args, z, 0, z) == -1


def test_kv_update_entry_points_validate_before_any_hip_call(lib):
    """KV append / trim: bad sizes and pointers come back as error codes."""
    i = ctypes.c_int
    lib.mla_verify_kv_append.argtypes = [i, i, i, i] + [ctypes.c_void_p] * 6
    lib.mla_verify_kv_trim.argtypes = [i, i, i] + [ctypes.c_void_p] * 6
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1002)
    z = ctypes.c_void_p(0)
    ok4 = [fake] * 4
    # sizes
    assert lib.mla_verify_kv_append(0, 8, 4, 16, *ok4, z, z) == -2
    assert lib.mla_verify_kv_append(2, 0, 4, 16, *ok4, z, z) == -2
    assert lib.mla_verify_kv_append(2, 17, 4, 16, *ok4, z, z) == -2
    assert lib.mla_verify_kv_append(2, 8, 0, 16, *ok4, z, z) == -4
    assert lib.mla_verify_kv_append(2, 8, 4, 0, *ok4, z, z) == -4
    assert lib.mla_verify_kv_append(2, 8, 1 << 25, 16, *ok4, z, z) == -4
    # pointers: NULL, misaligned, and a misaligned counter
    assert lib.mla_verify_kv_append(2, 8, 4, 16, z, fake, fake, fake, z, z) == -1
    assert lib.mla_verify_kv_append(2, 8, 4, 16, fake, fake, fake, z, z, z) == -1
    assert lib.mla_verify_kv_append(2, 8, 4, 16, fake, odd, fake, fake, z, z) == -4
    assert lib.mla_verify_kv_append(2, 8, 4, 16, *ok4, ctypes.c_void_p(0x1001), z) == -4
    assert lib.mla_verify_kv_trim(0, 8, 4, *[fake] * 5, z) == -2
    assert lib.mla_verify_kv_trim(2, 17, 4, *[fake] * 5, z) == -2
    assert lib.mla_verify_kv_trim(2, 8, 0, *[fake] * 5, z) == -4
    assert lib.mla_verify_kv_trim(2, 8, 4, fake, fake, z, fake, fake, z) == -1
    assert lib.mla_verify_kv_trim(2, 8, 4, fake, fake, fake, odd, fake, z) == -4


def test_tile_rows_forced_and_resolved(lib):
    # forced tiles are honoured for any head fold; 0 resolves to one of 32/64/128
    for t in (32, 64, 128):
        assert mv.verify_tile_rows(good(tile_rows=t)) == t
        assert mv.verify_tile_rows(good(q_len=1, num_heads=4, tile_rows=t)) == t
    assert mv.verify_tile_rows(good()) in (32, 64, 128)
    assert mv.verify_tile_rows(good(q_len=16, num_heads=128)) in (32, 64, 128)
    assert lib.mla_verify_tile_rows(ctypes.byref(good(tile_rows=48)), 0) == -4
    assert lib.mla_verify_tile_rows(None, 0) == -1
    # the workspace follows the split count only, whatever the tile
    for t in (32, 64, 128):
        assert mv.verify_workspace_size(good(num_splits=4, tile_rows=t)) == \
            4 * 16 * 8 * 8 * (512 * 2 + 4)


def _gpu_visible():
    """Whether HIP sees any device (counting devices does not start work on one)."""
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return False
    n = ctypes.c_int(0)
    return hip.hipGetDeviceCount(ctypes.byref(n)) == 0 and n.value > 0


@pytest.mark.skipif(_gpu_visible(), reason="needs a host with no GPU visible")
def test_every_compute_entry_point_reports_no_device(lib):
    """With every argument valid, a host that sees no GPU gets MLA_ERR_DEVICE
    from every entry point that launches work (the pointers are never used:
    the device check comes after the host checks and before any launch)."""
    buf = ctypes.create_string_buffer(1 << 16)
    a = ctypes.c_void_p((ctypes.addressof(buf) + 255) & ~255)
    p = ctypes.byref(good(batch=1, q_len=4, num_heads=8, max_pages_per_req=4, num_pool_pages=8))
    big = ctypes.c_size_t(1 << 30)
    calls = {
        "mla_verify_attn": lambda: lib.mla_verify_attn(p, a, a, a, a, a, a, a, big, None),
        "mla_verify_attn_gated": lambda: lib.mla_verify_attn_gated(p, a, a, a, a, a, a, a, a, a, a, big, None),
        "mla_verify_attn_gated_noalloc": lambda: lib.mla_verify_attn_gated_noalloc(p, a, a, a, a, a, a, a, a, a,
                                                                                   None),
        "mla_verify_attn_partials": lambda: lib.mla_verify_attn_partials(p, a, a, a, a, a, a, None),
        "mla_verify_lse_combine": lambda: lib.mla_verify_lse_combine(4, 32, a, a, a, a, None),
        "mla_verify_absorb_q": lambda: lib.mla_verify_absorb_q(p, a, a, a, None),
        "mla_verify_kv_append": lambda: lib.mla_verify_kv_append(1, 4, 4, 8, a, a, a, a, a, None),
        "mla_verify_kv_trim": lambda: lib.mla_verify_kv_trim(1, 4, 4, a, a, a, a, a, None),
    }
    for name, call in calls.items():
        assert call() == -6, name   # MLA_ERR_DEVICE
    assert "no GPU" in mv.status_string(-6)
