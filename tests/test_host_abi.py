"""Host-side checks of the C-ABI library that need no GPU.

The library must load and export every function include/dlrm_mi355x.h
declares.  Argument validation runs on the host before any HIP call, so the
error paths (NULL pointers, inconsistent shapes, unsupported sizes, missing
workspace) can be exercised here without a device; no compute call is made.
"""
import ctypes
import os
import re

import pytest

import dlrm_embedding_interaction_amd as dl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dlrm_mi355x.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[a-z_][\w\s\*]*?\b(dlrm_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return dl.load()


def test_header_declares_the_hot_path_calls():
    names = declared_functions()
    for n in ("dlrm_embbag_sum", "dlrm_interact_lower_tri", "dlrm_linear_bias_act", "dlrm_forward",
              "dlrm_forward_fused", "dlrm_forward_layered"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def test_status_strings_and_abi_version(lib):
    assert lib.dlrm_abi_version() == dl.ABI_VERSION
    for code in range(7):
        s = lib.dlrm_status_string(code).decode()
        assert s.startswith("DLRM_")
    assert b"unknown" in lib.dlrm_status_string(99)


def _model(ln_bot, ln_top, T, D, rows=100):
    keep = dl._i64s(ln_bot), dl._i64s(ln_top), dl._i64s([rows] * T)
    fake = dl._vp * 64
    ptrs = fake(*([4096] * 64))  # never dereferenced: validation fails or only sizes are read
    m = dl._Model(len(ln_bot), ctypes.cast(keep[0], dl._i64p), len(ln_top), ctypes.cast(keep[1], dl._i64p), T, D,
                  ctypes.cast(keep[2], dl._i64p), ptrs, ptrs, ptrs, ptrs, ptrs, None)
    return m, (keep, ptrs)


def _round_up(v, a):
    return (v + a - 1) // a * a


@pytest.mark.parametrize("B,ln_bot,ln_top,T,D", [
    (8, [4, 32, 16], [22, 32, 1], 3, 16),
    (2048, [13, 512, 256, 64], [70, 512, 256, 1], 3, 64),
    (2048, [13, 512, 256, 64], [592, 512, 256, 1], 32, 64),
    (65536, [13, 512, 256, 128], [479, 1024, 1024, 512, 256, 1], 26, 128),
    (5, [3, 4], [10, 1], 3, 4),
])
def test_workspace_bytes_formula(lib, B, ln_bot, ln_top, T, D):
    m, keep = _model(ln_bot, ln_top, T, D)
    P = (T + 1) * T // 2
    ldR = _round_up(D + P, 4)
    hidden = ln_bot[1:-1] + ln_top[1:-1]
    ldH = _round_up(max(hidden) if hidden else 0, 4)
    want = _round_up(B * ldR * 4, 256) + 2 * _round_up(B * ldH * 4, 256)
    assert lib.dlrm_forward_workspace_bytes(ctypes.byref(m), B) == want


@pytest.mark.parametrize("ln_bot,ln_top,T,D,B", [
    ([13, 8, 4], [9, 8, 1], 3, 4, 16),      # ln_top[0] != D + P
    ([13, 8, 4], [10, 8, 2], 3, 4, 16),     # last top width != 1
    ([13, 8, 5], [10, 8, 1], 3, 4, 16),     # last bottom width != D
    ([4], [10, 8, 1], 3, 4, 16),            # no bottom layer
    ([13, 8, 4], [10, 8, 1], 3, 4, 0),      # empty batch
])
def test_invalid_models_are_rejected(lib, ln_bot, ln_top, T, D, B):
    m, keep = _model(ln_bot, ln_top, T, D)
    assert lib.dlrm_forward_workspace_bytes(ctypes.byref(m), B) == 0
    one = dl._ptrs([])
    for fn in (lib.dlrm_forward, lib.dlrm_forward_layered):
        rc = fn(ctypes.byref(m), B, 4096, one, dl._i64s([1] * T), one, 8, 4096, 4096, 1 << 30, None)
        assert rc == dl.DLRM_E_SHAPE
    rc = lib.dlrm_forward_fused(ctypes.byref(m), B, 4096, one, dl._i64s([1] * T), one, 8, 4096, None)
    assert rc == dl.DLRM_E_SHAPE


def test_mini_dlrm_shape_from_the_pages_is_valid(lib):
    # dlrm_megakernel.rs unit test shape_invariants: ln_bot [13,8,4], m_spa 4, 3 tables, ln_top [10,8,1]
    m, keep = _model([13, 8, 4], [10, 8, 1], 3, 4)
    assert lib.dlrm_forward_workspace_bytes(ctypes.byref(m), 2048) > 0


def test_forward_rejects_missing_or_small_workspace(lib):
    m, keep = _model([13, 8, 4], [10, 8, 1], 3, 4)
    need = lib.dlrm_forward_workspace_bytes(ctypes.byref(m), 16)
    fake = (dl._vp * 3)(4096, 4096, 4096)
    n = dl._i64s([16, 16, 16])
    assert lib.dlrm_forward(ctypes.byref(m), 16, 4096, fake, n, fake, 8, 4096, None, need, None) == dl.DLRM_E_WORKSPACE
    assert lib.dlrm_forward(ctypes.byref(m), 16, 4096, fake, n, fake, 8, 4096, 4096, need - 1, None) == dl.DLRM_E_WORKSPACE
    assert lib.dlrm_forward(ctypes.byref(m), 16, 4096, fake, n, fake, 8, 4096, 4096 + 16, need, None) == dl.DLRM_E_WORKSPACE
    assert lib.dlrm_forward(None, 16, 4096, fake, n, fake, 8, 4096, 4096, need, None) == dl.DLRM_E_NULL
    assert lib.dlrm_forward(ctypes.byref(m), 16, None, fake, n, fake, 8, 4096, 4096, need, None) == dl.DLRM_E_NULL


def test_layered_forward_rejects_missing_or_small_workspace(lib):
    m, keep = _model([13, 8, 4], [10, 8, 1], 3, 4)
    need = lib.dlrm_forward_workspace_bytes(ctypes.byref(m), 16)
    fake = (dl._vp * 3)(4096, 4096, 4096)
    n = dl._i64s([16, 16, 16])
    f = lib.dlrm_forward_layered
    assert f(ctypes.byref(m), 16, 4096, fake, n, fake, 8, 4096, None, need, None) == dl.DLRM_E_WORKSPACE
    assert f(ctypes.byref(m), 16, 4096, fake, n, fake, 8, 4096, 4096, need - 1, None) == dl.DLRM_E_WORKSPACE
    assert f(ctypes.byref(m), 16, 4096, fake, n, fake, 8, 4096, 4096 + 16, need, None) == dl.DLRM_E_WORKSPACE


@pytest.mark.parametrize("ln_bot,ln_top,T,D,why", [
    ([13, 8, 12], [18, 8, 1], 3, 12, "rows shorter than 16"),
    ([13, 8, 33], [39, 8, 1], 3, 33, "rows not a multiple of 4"),
    ([13, 8, 260], [266, 8, 1], 3, 260, "rows longer than 256"),
    ([13] + [16] * 9, [22, 8, 1], 3, 16, "nine bottom layers"),
    ([13, 8, 64], [64 + 2080, 8, 1], 64, 64, "LDS above 160 KiB"),
])
def test_fused_forward_rejects_models_outside_its_limits(lib, ln_bot, ln_top, T, D, why):
    """Checked on the host before any launch, so no device is needed."""
    m, keep = _model(ln_bot, ln_top, T, D)
    fake = (dl._vp * T)(*([4096] * T))
    n = dl._i64s([16] * T)
    rc = lib.dlrm_forward_fused(ctypes.byref(m), 16, 4096, fake, n, fake, 8, 4096, None)
    assert rc == dl.DLRM_E_UNSUPPORTED, why


def _packed_floats(ln):
    n = 0
    for k, o in zip(ln[:-1], ln[1:]):
        if o > 128:
            f = ((o + 31) // 32) * ((k + 7) // 8) * 256
        else:
            f = ((o + 15) // 16) * ((k + 15) // 16) * 256
        n += (f + 63) // 64 * 64
    return n


@pytest.mark.parametrize("ln_bot,ln_top,T,D", [
    ([13, 512, 256, 64], [70, 512, 256, 1], 3, 64),
    ([13, 512, 256, 64], [592, 512, 256, 1], 32, 64),
    ([4, 32, 16], [22, 32, 1], 3, 16),
    ([3, 37, 16], [22, 1], 3, 16),
    ([5, 129, 128, 16], [22, 161, 97, 1], 3, 16),
])
def test_pack_weights_bytes_formula(lib, ln_bot, ln_top, T, D):
    """Every layer but the one-output last: for N <= 128 outputs ceil(N/16) x
    ceil(K/16) tiles of 256 floats, for N > 128 ceil(N/32) x ceil(K/8); each
    layer rounded up to 256 bytes; then the tail of the last layer's weights and
    bias and the hidden biases, each rounded up to 4 floats."""
    m, keep = _model(ln_bot, ln_top, T, D)
    r4 = lambda v: (v + 3) // 4 * 4
    tail = r4(ln_top[-2]) + 4 + sum(r4(n) for n in ln_bot[1:]) + sum(r4(n) for n in ln_top[1:-1])
    want = 4 * (_packed_floats(ln_bot) + _packed_floats(ln_top[:-1]) + (tail + 63) // 64 * 64)
    assert lib.dlrm_pack_weights_bytes(ctypes.byref(m)) == want


def test_pack_weights_argument_errors(lib):
    m, keep = _model([13, 8, 16], [22, 8, 1], 3, 16)
    need = lib.dlrm_pack_weights_bytes(ctypes.byref(m))
    assert need > 0
    f = lib.dlrm_pack_weights
    assert f(None, 4096, need, None) == dl.DLRM_E_NULL
    assert f(ctypes.byref(m), None, need, None) == dl.DLRM_E_NULL
    assert f(ctypes.byref(m), 4096, need - 1, None) == dl.DLRM_E_WORKSPACE
    assert f(ctypes.byref(m), 4096 + 16, need, None) == dl.DLRM_E_WORKSPACE
    bad, keep2 = _model([13, 8, 12], [18, 8, 1], 3, 12)
    assert lib.dlrm_pack_weights_bytes(ctypes.byref(bad)) == 0
    assert f(ctypes.byref(bad), 4096, 1 << 20, None) == dl.DLRM_E_UNSUPPORTED


def test_forward_path_choice(lib):
    """Layered without packed weights; with them the single launch up to batch
    8192 (up to 4096 with 24-32 tables and rows a multiple of 16, 1024..2048
    with more tables); 0 for invalid input.  Host only."""
    m, keep = _model([13, 512, 256, 64], [70, 512, 256, 1], 3, 64)
    assert lib.dlrm_forward_path(ctypes.byref(m), 2048) == 1
    m.packed_w = 4096
    assert lib.dlrm_forward_path(ctypes.byref(m), 2048) == 2
    assert lib.dlrm_forward_path(ctypes.byref(m), 8192) == 2
    assert lib.dlrm_forward_path(ctypes.byref(m), 8193) == 1
    assert lib.dlrm_forward_path(ctypes.byref(m), 0) == 0
    assert lib.dlrm_forward_path(None, 16) == 0
    m16, keep16 = _model([13, 512, 256, 64], [64 + 136, 512, 256, 1], 16, 64)
    m16.packed_w = 4096
    assert lib.dlrm_forward_path(ctypes.byref(m16), 16) == 2
    assert lib.dlrm_forward_path(ctypes.byref(m16), 256) == 2
    assert lib.dlrm_forward_path(ctypes.byref(m16), 8192) == 2
    assert lib.dlrm_forward_path(ctypes.byref(m16), 8193) == 1
    m32, keep32 = _model([13, 512, 256, 64], [64 + 528, 512, 256, 1], 32, 64)
    m32.packed_w = 4096
    assert lib.dlrm_forward_path(ctypes.byref(m32), 16) == 2
    assert lib.dlrm_forward_path(ctypes.byref(m32), 128) == 2
    assert lib.dlrm_forward_path(ctypes.byref(m32), 256) == 2
    assert lib.dlrm_forward_path(ctypes.byref(m32), 512) == 2
    assert lib.dlrm_forward_path(ctypes.byref(m32), 1024) == 2
    assert lib.dlrm_forward_path(ctypes.byref(m32), 4096) == 2
    assert lib.dlrm_forward_path(ctypes.byref(m32), 4097) == 1
    m40, keep40 = _model([13, 512, 256, 64], [64 + 820, 512, 256, 1], 40, 64)
    m40.packed_w = 4096
    assert lib.dlrm_forward_path(ctypes.byref(m40), 512) == 1
    assert lib.dlrm_forward_path(ctypes.byref(m40), 2048) == 2
    assert lib.dlrm_forward_path(ctypes.byref(m40), 4096) == 1
    big, keep3 = _model([13, 64], [70, 1024, 1024, 1], 3, 64)
    big.packed_w = 4096
    assert lib.dlrm_forward_path(ctypes.byref(big), 64) == 1   # 5 MB of weights


def test_fused_forward_needs_packed_weights(lib):
    m, keep = _model([13, 8, 16], [22, 8, 1], 3, 16)
    fake = (dl._vp * 3)(4096, 4096, 4096)
    n = dl._i64s([16, 16, 16])
    assert lib.dlrm_forward_fused(ctypes.byref(m), 16, 4096, fake, n, fake, 8, 4096, None) == dl.DLRM_E_NULL
    m.packed_w = 4096 + 4
    assert lib.dlrm_forward_fused(ctypes.byref(m), 16, 4096, fake, n, fake, 8, 4096, None) == dl.DLRM_E_SHAPE


def test_fused_forward_argument_errors(lib):
    m, keep = _model([13, 8, 16], [22, 8, 1], 3, 16)
    fake = (dl._vp * 3)(4096, 4096, 4096)
    n = dl._i64s([16, 16, 16])
    f = lib.dlrm_forward_fused
    assert f(None, 16, 4096, fake, n, fake, 8, 4096, None) == dl.DLRM_E_NULL
    assert f(ctypes.byref(m), 16, None, fake, n, fake, 8, 4096, None) == dl.DLRM_E_NULL
    assert f(ctypes.byref(m), 16, 4096, fake, n, fake, 8, None, None) == dl.DLRM_E_NULL
    assert f(ctypes.byref(m), 0, 4096, fake, n, fake, 8, 4096, None) == dl.DLRM_E_SHAPE


def test_linear_argument_errors(lib):
    f = lib.dlrm_linear_bias_act
    assert f(4, 4, 4, None, 4, 4096, None, 0, 4096, 4, None) == dl.DLRM_E_NULL
    assert f(0, 4, 4, 4096, 4, 4096, None, 0, 4096, 4, None) == dl.DLRM_E_SHAPE
    assert f(4, 4, 8, 4096, 4, 4096, None, 0, 4096, 4, None) == dl.DLRM_E_SHAPE   # ld_x < K
    assert f(4, 8, 4, 4096, 4, 4096, None, 0, 4096, 4, None) == dl.DLRM_E_SHAPE   # ld_y < N
    assert f(4, 4, 4, 4096, 4, 4096, None, 7, 4096, 4, None) == dl.DLRM_E_SHAPE   # unknown activation


def test_embbag_argument_errors(lib):
    f = lib.dlrm_embbag_sum
    p = (dl._vp * 65)(*([4096] * 65))
    n = dl._i64s([1] * 65)
    assert f(65, 4, 4, p, n, p, n, p, 8, 4096, None) == dl.DLRM_E_UNSUPPORTED
    assert f(0, 4, 4, p, n, p, n, p, 8, 4096, None) == dl.DLRM_E_SHAPE
    assert f(2, 4, 2048, p, n, p, n, p, 8, 4096, None) == dl.DLRM_E_UNSUPPORTED  # dim above 1024
    assert f(2, 4, 4, p, n, p, n, p, 8, None, None) == dl.DLRM_E_NULL
    z = (dl._vp * 2)(4096, None)
    assert f(2, 4, 4, z, n, p, n, p, 8, 4096, None) == dl.DLRM_E_NULL
    neg = dl._i64s([1, -1])
    assert f(2, 4, 4, p, n, p, neg, p, 8, 4096, None) == dl.DLRM_E_SHAPE
    for width in (0, 2, 16):
        assert f(2, 4, 4, p, n, p, n, p, width, 4096, None) == dl.DLRM_E_SHAPE   # index width not 4 or 8
    big = dl._i64s([1 << 31, 1])
    assert f(2, 4, 4, p, n, p, big, p, 4, 4096, None) == dl.DLRM_E_UNSUPPORTED  # int32 cannot count that far


def test_stacked_bag_argument_errors(lib):
    f = lib.dlrm_embbag_sum_stacked
    p = (dl._vp * 2)(4096, 4096)
    n = dl._i64s([4, 4])
    base = dl._i64s([0, 100])
    rows = dl._i64s([100, 50])
    assert f(2, 4, 4, None, base, rows, p, n, p, 8, 4096, None) == dl.DLRM_E_NULL
    assert f(2, 4, 4, 4096, None, rows, p, n, p, 8, 4096, None) == dl.DLRM_E_NULL
    assert f(2, 4, 4, 4096, dl._i64s([0, -1]), rows, p, n, p, 8, 4096, None) == dl.DLRM_E_SHAPE
    assert f(2, 4, 4, 4096, base, dl._i64s([100, 0]), p, n, p, 8, 4096, None) == dl.DLRM_E_SHAPE
    assert f(2, 4, 4, 4096, base, rows, p, n, p, 3, 4096, None) == dl.DLRM_E_SHAPE
    assert f(65, 4, 4, 4096, base, rows, p, n, p, 8, 4096, None) == dl.DLRM_E_UNSUPPORTED


def test_forward_rejects_other_index_widths(lib):
    m, keep = _model([13, 8, 4], [10, 8, 1], 3, 4)
    need = lib.dlrm_forward_workspace_bytes(ctypes.byref(m), 16)
    fake = (dl._vp * 3)(4096, 4096, 4096)
    n = dl._i64s([16, 16, 16])
    for width in (0, 2, 16):
        assert lib.dlrm_forward(ctypes.byref(m), 16, 4096, fake, n, fake, width, 4096, 4096, need,
                                None) == dl.DLRM_E_SHAPE
        assert lib.dlrm_forward_layered(ctypes.byref(m), 16, 4096, fake, n, fake, width, 4096, 4096, need,
                                        None) == dl.DLRM_E_SHAPE
        assert lib.dlrm_forward_fused(ctypes.byref(m), 16, 4096, fake, n, fake, width, 4096,
                                      None) == dl.DLRM_E_SHAPE


def test_stacked_model_needs_its_row_bases(lib):
    """With emb_w NULL the tables come from emb_stacked and emb_row_base."""
    m, keep = _model([13, 8, 4], [10, 8, 1], 3, 4)
    need = lib.dlrm_forward_workspace_bytes(ctypes.byref(m), 16)
    fake = (dl._vp * 3)(4096, 4096, 4096)
    n = dl._i64s([16, 16, 16])
    m.emb_w = None
    assert lib.dlrm_forward(ctypes.byref(m), 16, 4096, fake, n, fake, 8, 4096, 4096, need, None) == dl.DLRM_E_NULL
    m.emb_stacked = 4096
    assert lib.dlrm_forward(ctypes.byref(m), 16, 4096, fake, n, fake, 8, 4096, 4096, need, None) == dl.DLRM_E_NULL
    bad = dl._i64s([0, -5, 10])
    m.emb_row_base = ctypes.cast(bad, dl._i64p)
    assert lib.dlrm_forward(ctypes.byref(m), 16, 4096, fake, n, fake, 8, 4096, 4096, need, None) == dl.DLRM_E_SHAPE


def test_general_bag_argument_errors(lib):
    f = lib.dlrm_embbag
    p = (dl._vp * 2)(4096, 4096)
    n = dl._i64s([4, 4])
    ok = dl._BagOptions(0, 0, 8, 0)
    assert f(2, 4, 4, p, n, p, n, p, None, 4096, None) == dl.DLRM_E_NULL          # no options
    assert f(2, 4, 4, p, n, p, n, p, ctypes.byref(dl._BagOptions(3, 0, 8, 0)), 4096, None) == dl.DLRM_E_SHAPE
    assert f(2, 4, 4, p, n, p, n, p, ctypes.byref(dl._BagOptions(0, 0, 2, 0)), 4096, None) == dl.DLRM_E_SHAPE
    wts = (dl._vp * 2)(4096, 4096)
    mean_w = dl._BagOptions(1, 0, 8, 0, None, ctypes.cast(wts, ctypes.POINTER(dl._vp)))
    assert f(2, 4, 4, p, n, p, n, p, ctypes.byref(mean_w), 4096, None) == dl.DLRM_E_SHAPE   # weights need sum
    assert f(65, 4, 4, p, n, p, n, p, ctypes.byref(ok), 4096, None) == dl.DLRM_E_UNSUPPORTED
    assert f(2, 4, 4, p, n, p, n, p, ctypes.byref(ok), None, None) == dl.DLRM_E_NULL


def test_interact_argument_errors(lib):
    f = lib.dlrm_interact_lower_tri
    assert f(4, 3, 16, None, 16, 4096, 4096, 22, 1, None) == dl.DLRM_E_NULL
    assert f(4, 3, 16, 4096, 8, 4096, 4096, 22, 1, None) == dl.DLRM_E_SHAPE     # ld_x < dim
    assert f(4, 3, 16, 4096, 16, 4096, 4096, 21, 1, None) == dl.DLRM_E_SHAPE    # ld_out < D + P
    assert f(4, 3, 16, 4096, 16, 4096, 4096, 5, 0, None) == dl.DLRM_E_SHAPE     # ld_out < P
    assert f(4, 64, 1024, 4096, 1024, 4096, 4096, 4096, 0, None) == dl.DLRM_E_UNSUPPORTED  # LDS


def test_fused_bag_interaction_argument_errors(lib):
    f = lib.dlrm_embbag_interact
    p = (dl._vp * 3)(4096, 4096, 4096)
    n = dl._i64s([4, 4, 4])
    assert f(3, 4, 16, p, n, p, n, p, 8, None, 16, 4096, 22, 1, None) == dl.DLRM_E_NULL
    assert f(3, 4, 16, p, n, p, n, p, 8, 4096, 8, 4096, 22, 1, None) == dl.DLRM_E_SHAPE
    assert f(3, 4, 16, p, n, p, n, p, 8, 4096, 16, 4096, 21, 1, None) == dl.DLRM_E_SHAPE
    assert f(3, 4, 16, p, n, p, n, p, 8, 4096, 16, 4096, 5, 0, None) == dl.DLRM_E_SHAPE
    assert f(65, 4, 16, p, n, p, n, p, 8, 4096, 16, 4096, 4096, 0, None) == dl.DLRM_E_UNSUPPORTED
    assert f(3, 4, 16, p, n, p, n, p, 5, 4096, 16, 4096, 22, 1, None) == dl.DLRM_E_SHAPE    # index width


def test_pair_map_and_check_argument_errors(lib):
    assert lib.dlrm_pair_index_map(1, 4096, 4096, None) == dl.DLRM_E_SHAPE
    assert lib.dlrm_pair_index_map(4, None, 4096, None) == dl.DLRM_E_NULL
    p = (dl._vp * 2)(4096, 4096)
    n = dl._i64s([1, 1])
    assert lib.dlrm_embbag_check_indices(2, 4, n, p, n, p, 8, None, None) == dl.DLRM_E_NULL
    assert lib.dlrm_embbag_check_indices(0, 4, n, p, n, p, 8, 4096, None) == dl.DLRM_E_SHAPE
    assert lib.dlrm_embbag_check_indices(2, 4, n, p, n, p, 6, 4096, None) == dl.DLRM_E_SHAPE


def test_probe_argument_errors(lib):
    assert lib.dlrm_probe_sink_floats() > 0
    assert lib.dlrm_probe_read_stream(None, 1024, 4096, None) == dl.DLRM_E_NULL
    assert lib.dlrm_probe_read_stream(4096, 1022, 4096, None) == dl.DLRM_E_SHAPE     # not a multiple of 4
    assert lib.dlrm_probe_read_stream(4100, 1024, 4096, None) == dl.DLRM_E_SHAPE     # not 16-byte aligned
    g = lib.dlrm_probe_gather_rows
    assert g(None, 100, 64, 4096, 10, 4096, None) == dl.DLRM_E_NULL
    assert g(4096, 100, 48, 4096, 10, 4096, None) == dl.DLRM_E_SHAPE                # not a power of two
    assert g(4096, 100, 8, 4096, 10, 4096, None) == dl.DLRM_E_SHAPE
    assert g(4096, 0, 64, 4096, 10, 4096, None) == dl.DLRM_E_SHAPE
    l2 = lib.dlrm_probe_l2_stream
    assert l2(None, 1024, 256, 4096, None) == dl.DLRM_E_NULL
    assert l2(4096, 1024, 0, 4096, None) == dl.DLRM_E_SHAPE
    assert l2(4096, 1026, 256, 4096, None) == dl.DLRM_E_SHAPE


def test_noalloc_forward_checks_before_any_launch(lib):
    """Invalid models give dlrm_forward's own error codes; a workspace beyond the
    static array is refused; neither touches the device."""
    assert lib.dlrm_forward_noalloc_max_bytes() == 64 << 20
    fake = (dl._vp * 3)(4096, 4096, 4096)
    n = dl._i64s([16, 16, 16])
    bad, keep = _model([13, 8, 5], [10, 8, 1], 3, 4)
    f = lib.dlrm_forward_noalloc
    assert f(ctypes.byref(bad), 16, 4096, fake, n, fake, 8, 4096, None) == dl.DLRM_E_SHAPE
    assert f(None, 16, 4096, fake, n, fake, 8, 4096, None) == dl.DLRM_E_NULL
    big, keep2 = _model([13, 512, 256, 128], [479, 1024, 1024, 512, 256, 1], 26, 128)
    assert lib.dlrm_forward_workspace_bytes(ctypes.byref(big), 65536) > (64 << 20)
    fake26 = (dl._vp * 26)(*([4096] * 26))
    n26 = dl._i64s([65536 * 20] * 26)
    assert f(ctypes.byref(big), 65536, 4096, fake26, n26, fake26, 8, 4096, None) == dl.DLRM_E_UNSUPPORTED
