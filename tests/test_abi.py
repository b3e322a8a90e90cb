"""The C ABI on the host: the library loads, exports every symbol the header
declares, sizes its workspace, and rejects bad arguments before touching the
GPU (none of these calls launch anything)."""
import ctypes
import os
import re

import pytest

import sparse_moe_layer_fp32_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(moe_\w+)\s*\(", text, re.M)))


def test_header_symbols_exported():
    lib = moe.load_library()
    names = header_functions()
    assert {"moe_route", "moe_permute", "moe_forward", "moe_workspace_size",
            "moe_last_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(moe.EXPORTED)


def test_config_struct_layout():
    # int64 + 5 int32 + float + int32 + 2 floats, natural alignment
    assert ctypes.sizeof(moe.moe_config) == 48
    assert moe.moe_config.routed_scaling.offset == 28


def full(T):
    return moe.make_config(T)


def test_workspace_size_grows_with_tokens():
    s0, s1, s2 = (moe.moe_workspace_size(full(T)) for T in (0, 64, 8192))
    assert 0 < s0 < s1 < s2
    # at least the bf16 intermediates: h [(P + T) * I] and o [(P + T) * H]
    P, T = 8192 * 8, 8192
    assert s2 >= (P + T) * 1280 * 2 + (P + T) * 4096 * 2
    # workspace view regions lie inside the workspace and do not overlap
    cfg = full(8192)
    regions = sorted(moe.moe_workspace_view(cfg, i) for i in range(7))
    for (a, na), (b, _) in zip(regions, regions[1:]):
        assert a + na <= b
    assert regions[-1][0] + regions[-1][1] <= s2


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(top_k=289), moe.MOE_ERR_INVALID_ARG),
    (dict(hidden=0), moe.MOE_ERR_INVALID_ARG),
    (dict(inter_shared=-64), moe.MOE_ERR_INVALID_ARG),
    (dict(num_experts=2048, top_k=8), moe.MOE_ERR_UNSUPPORTED),
    (dict(top_k=33), moe.MOE_ERR_UNSUPPORTED),
    (dict(hidden=4000), moe.MOE_ERR_UNSUPPORTED),
    (dict(inter=1000), moe.MOE_ERR_UNSUPPORTED),
    (dict(tokens=2**28), moe.MOE_ERR_UNSUPPORTED),
])
def test_invalid_configs(kw, status):
    args = dict(tokens=64)
    args.update(kw)
    cfg = moe.make_config(**args)
    assert moe.load_library().moe_workspace_size(ctypes.byref(cfg)) == 0
    lib = moe.load_library()
    st = lib.moe_forward(ctypes.byref(cfg), *([None] * 13), 0, None)
    assert st == status, moe.moe_last_error()
    assert moe.moe_last_error()


def test_null_pointers_and_small_workspace():
    lib = moe.load_library()
    cfg = full(64)
    need = moe.moe_workspace_size(cfg)
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    st = lib.moe_forward(ctypes.byref(cfg), None, fake, None, fake, fake, fake, fake, fake, fake,
                         fake, None, None, fake, need, None)
    assert st == moe.MOE_ERR_INVALID_ARG and "NULL" in moe.moe_last_error()
    st = lib.moe_forward(ctypes.byref(cfg), fake, fake, None, fake, fake, fake, None, fake, fake,
                         fake, None, None, fake, need, None)
    assert st == moe.MOE_ERR_INVALID_ARG and "shared" in moe.moe_last_error()
    st = lib.moe_forward(ctypes.byref(cfg), fake, fake, None, fake, fake, fake, fake, fake, fake,
                         fake, None, None, fake, need - 1, None)
    assert st == moe.MOE_ERR_WORKSPACE
    mis = ctypes.c_void_p((1 << 20) + 4)
    st = lib.moe_forward(ctypes.byref(cfg), mis, fake, None, fake, fake, fake, fake, fake, fake,
                         fake, None, None, fake, need, None)
    assert st == moe.MOE_ERR_UNSUPPORTED
    st = lib.moe_route(ctypes.byref(cfg), fake, fake, None, None, fake, fake, need, None)
    assert st == moe.MOE_ERR_INVALID_ARG
    st = lib.moe_permute(ctypes.byref(cfg), fake, fake, fake, fake, fake, 16, None)
    assert st == moe.MOE_ERR_WORKSPACE
    st = lib.moe_forward_timed(ctypes.byref(cfg), *([fake] * 10), None, None, fake, need, None,
                               None, 3)
    assert st == moe.MOE_ERR_INVALID_ARG
    off, nb = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.moe_workspace_view(ctypes.byref(cfg), 99, ctypes.byref(off),
                                  ctypes.byref(nb)) == moe.MOE_ERR_INVALID_ARG


# ------------------------------------------------------------------ dense FFN

def test_dense_config_layout_and_workspace():
    assert ctypes.sizeof(moe.moe_dense_config) == 24
    assert moe.moe_dense_config.swiglu_limit.offset == 16
    s = [moe.moe_dense_workspace_size(moe.make_dense_config(T)) for T in (0, 64, 8192)]
    assert 0 < s[0] < s[1] < s[2]
    assert s[2] >= 8192 * 11264 * 2  # the bf16 SwiGLU activations


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=0), moe.MOE_ERR_INVALID_ARG),
    (dict(inter=0), moe.MOE_ERR_INVALID_ARG),
    (dict(tokens=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(hidden=4000), moe.MOE_ERR_UNSUPPORTED),
    (dict(inter=11200 + 10), moe.MOE_ERR_UNSUPPORTED),
    (dict(tokens=2**20), moe.MOE_ERR_UNSUPPORTED),
])
def test_dense_invalid_configs(kw, status):
    args = dict(tokens=64)
    args.update(kw)
    cfg = moe.make_dense_config(**args)
    lib = moe.load_library()
    assert lib.moe_dense_workspace_size(ctypes.byref(cfg)) == 0
    st = lib.moe_dense_forward(ctypes.byref(cfg), *([None] * 6), 0, None)
    assert st == status, moe.moe_last_error()


def test_dense_errors_before_launch():
    lib = moe.load_library()
    cfg = moe.make_dense_config(64)
    need = moe.moe_dense_workspace_size(cfg)
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    st = lib.moe_dense_forward(ctypes.byref(cfg), fake, fake, None, fake, fake, fake, need, None)
    assert st == moe.MOE_ERR_INVALID_ARG and "NULL" in moe.moe_last_error()
    st = lib.moe_dense_forward(ctypes.byref(cfg), fake, fake, fake, fake, fake, fake, need - 1,
                               None)
    assert st == moe.MOE_ERR_WORKSPACE
    mis = ctypes.c_void_p((1 << 20) + 8)
    st = lib.moe_dense_forward(ctypes.byref(cfg), fake, fake, fake, fake, mis, fake, need, None)
    assert st == moe.MOE_ERR_UNSUPPORTED
    bad = moe.make_dense_config(64)
    bad.reserved = 1
    st = lib.moe_dense_forward(ctypes.byref(bad), fake, fake, fake, fake, fake, fake, need, None)
    assert st == moe.MOE_ERR_INVALID_ARG


def test_fused_errors_before_launch():
    """moe_forward_fused: the batch limits, NULLs and the workspace size are
    checked before anything is enqueued; the workspace views of its control
    and status words lie inside the workspace."""
    lib = moe.load_library()
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    cfg = full(64)
    need = moe.moe_workspace_size(cfg)
    args = [fake, fake, None, fake, fake, fake, fake, fake, fake, fake, None, None, fake]
    st = lib.moe_forward_fused(ctypes.byref(cfg), *args, need - 1, None)
    assert st == moe.MOE_ERR_WORKSPACE
    null_x = [None] + args[1:]
    st = lib.moe_forward_fused(ctypes.byref(cfg), *null_x, need, None)
    assert st == moe.MOE_ERR_INVALID_ARG
    for T, k in ((moe.FUSED_MAX_TOKENS + 1, 8), (moe.FUSED_MAX_TOKENS, 9)):
        big = moe.make_config(T, 4096, 288, k, 1280, 1280)
        st = lib.moe_forward_fused(ctypes.byref(big), *args, moe.moe_workspace_size(big), None)
        assert st == moe.MOE_ERR_UNSUPPORTED and "single-launch" in moe.moe_last_error()
    total = moe.moe_workspace_size(cfg)
    c_off, c_nb = moe.moe_workspace_view(cfg, moe.MOE_WS_FUSED_CTL)
    s_off, s_nb = moe.moe_workspace_view(cfg, moe.MOE_WS_FUSED_STATUS)
    assert c_off + c_nb <= total and c_nb % 256 == 0 and s_nb == 4
    assert c_off <= s_off < c_off + c_nb


def test_noalloc_errors_before_launch():
    """moe_forward_noalloc: a batch whose workspace exceeds the fixed scratch
    and NULL pointers are refused before anything is enqueued (no device
    call); an empty batch returns at once."""
    lib = moe.load_library()
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    args = [fake, fake, None, fake, fake, fake, fake, fake, fake, fake, None, None]
    big = full(1024)
    assert moe.moe_workspace_size(big) > moe.NOALLOC_SCRATCH_BYTES
    st = lib.moe_forward_noalloc(ctypes.byref(big), *args, None)
    assert st == moe.MOE_ERR_WORKSPACE and "scratch" in moe.moe_last_error()
    st = lib.moe_forward_noalloc(ctypes.byref(full(64)), None, *args[1:], None)
    assert st == moe.MOE_ERR_INVALID_ARG
    mis = ctypes.c_void_p((1 << 20) + 8)
    st = lib.moe_forward_noalloc(ctypes.byref(full(64)), mis, *args[1:], None)
    assert st == moe.MOE_ERR_UNSUPPORTED
    st = lib.moe_forward_noalloc(ctypes.byref(full(0)), None, *args[1:10], None, None, None, None)
    assert st == moe.MOE_OK
    assert moe.moe_workspace_size(full(630)) <= moe.NOALLOC_SCRATCH_BYTES
