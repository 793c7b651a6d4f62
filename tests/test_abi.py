"""C-ABI boundary checks that need no GPU: the library loads, exports every function that
include/moe.h declares, sizes plans and workspaces, and rejects invalid calls on the host
before anything is enqueued (every case below fails validation, so no kernel is launched)."""
import ctypes
import os
import re

import pytest

from mixture_experts_layer_lds_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20            # a non-null, 16-byte aligned address that is never dereferenced


def header_functions():
    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return B.lib()


def test_exports_every_declared_function(lib):
    declared = header_functions()
    assert {"moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_forward",
            "moe_backward"} <= set(declared)
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(B.EXPORTS) == declared
    assert b"gfx950" in lib.moe_version()


def test_status_strings(lib):
    for code, name in B.STATUS.items():
        assert lib.moe_status_string(code).decode().startswith(name)


def dims(**kw):
    base = dict(T=256, d=128, n=256, E=8, K=2, dtype="bf16")
    base.update(kw)
    return B.make_dims(**base)


def test_max_rows():
    assert B.moe_max_rows(dims()) == 512
    assert B.moe_max_rows(dims(round_mode=B.ROUND_DOWN, tile_m=64)) == 512
    assert B.moe_max_rows(dims(round_mode=B.ROUND_NEAREST, tile_m=128)) == 512 + 8 * 127
    assert B.moe_max_rows(dims(T=16, E=8, K=2, round_mode=B.ROUND_UP, tile_m=128)) == 16 * 8


def test_workspace_sizes():
    d = dims(T=32768, d=1536, n=256, E=128, K=8)
    for op in range(6):
        assert B.moe_workspace_bytes(d, op) >= 0
    R = 32768 * 8
    assert B.moe_workspace_bytes(d, B.OP_FFN) >= R * 256 * 2
    assert B.moe_workspace_bytes(d, B.OP_FORWARD) >= R * (256 + 1536) * 2
    assert B.moe_workspace_bytes(d, B.OP_BACKWARD) >= R * (4 * 256 + 256 + 1536) * 2


@pytest.mark.parametrize("kw,status", [
    (dict(K=9), -1), (dict(K=0), -1), (dict(E=0, K=1), -1), (dict(E=2000), -1),
    (dict(E=32, K=17), -2), (dict(d=96), -2), (dict(n=100), -2), (dict(d=32), -1), (dict(T=0), -1),
    (dict(dtype="f32", round_mode=7), -1), (dict(round_mode=1, tile_m=0), -1),
    (dict(round_mode=1, tile_m=4096), -1), (dict(round_mode=4), -1),
])
def test_invalid_dims_rejected(lib, kw, status):
    d = dims(**kw)
    plan = B.PlanStruct(*([FAKE] * 9))
    r = lib.moe_route(ctypes.byref(d), None, None, None, FAKE, ctypes.byref(plan), FAKE, 1 << 40, None)
    assert r == status, lib.moe_last_error()
    assert lib.moe_last_error()
    assert B.lib().moe_max_rows(ctypes.byref(d)) == 0


def test_stochastic_rounding_needs_words():
    """MOE_ROUND_STOCHASTIC is valid once round_rand points at the caller's words (it may add up
    to tile_m - 1 rows per expert, like NEAREST and UP)."""
    d = dims(round_mode=4)
    assert B.lib().moe_max_rows(ctypes.byref(d)) == 0
    d.round_rand = FAKE
    assert B.lib().moe_max_rows(ctypes.byref(d)) == B.lib().moe_max_rows(ctypes.byref(dims(round_mode=2)))


def test_route_workspace_grows_with_token_rounding():
    """Token rounding keeps the routing keys transposed ([E][T] words) in the routing workspace,
    on top of the plain plan's bitmap, per-word prefixes and group offsets."""
    T, E = 4096, 64
    plain = B.moe_workspace_bytes(dims(T=T, E=E), B.OP_ROUTE)
    rounded = B.moe_workspace_bytes(dims(T=T, E=E, round_mode=1), B.OP_ROUTE)
    W = T // 32
    assert plain >= 2 * E * W * 4 + (W + 1) * 4
    assert rounded >= plain + E * T * 4
    assert B.moe_workspace_bytes(dims(T=T, E=E, round_mode=1), B.OP_FORWARD) >= rounded


def test_route_workspace_holds_split_router_partials():
    """A bf16 layer whose router GEMM has fewer than 256 tiles of 256 tokens x 128 experts splits
    its reduction over d: the partial products of the slices after the first ([SK-1][T][E] fp32)
    sit after the routing workspace proper.  32768 tokens x 128 experts is 128 tiles: two slices;
    512 tokens x 8 experts at d = 4096 is 2 tiles: four slices; fp32 layers never split."""
    def base(T, E):
        W = (T + 31) // 32
        r = lambda x: (x + 255) // 256 * 256
        return 2 * r(E * W * 4) + r((W + 1) * 4)

    T, E = 32768, 128
    assert B.moe_workspace_bytes(dims(T=T, E=E, d=1536), B.OP_ROUTE) == base(T, E) + T * E * 4
    assert B.moe_workspace_bytes(dims(T=T, E=E, d=1536, dtype="f32"), B.OP_ROUTE) == base(T, E)
    T, E = 512, 8
    assert B.moe_workspace_bytes(dims(T=T, E=E, d=4096), B.OP_ROUTE) == base(T, E) + 3 * T * E * 4
    T, E = 65536, 128  # 256 tiles: no split
    assert B.moe_workspace_bytes(dims(T=T, E=E, d=1536), B.OP_ROUTE) == base(T, E)


def test_decode_argument_checks(lib):
    """moe_decode: plain top-K only, T <= 1024, its own workspace size, required pointers."""
    call = lambda d, ws=1 << 40, out=FAKE: lib.moe_decode(
        ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, out, FAKE, ws, None)
    assert call(dims(round_mode=1)) == -2
    assert call(dims(T=2000)) == -2
    d = dims(T=8)
    need = B.moe_workspace_bytes(d, B.OP_DECODE)
    assert need >= 8 * 2 * (256 + 128) * 4     # activation and fp32 y rows of the 16 (token, expert) pairs
    assert call(d, ws=need - 1) == -3
    assert call(d, out=None) == -1
    assert lib.moe_last_error()


def test_null_and_misaligned_pointers_rejected(lib):
    d = dims()
    plan = B.PlanStruct(*([FAKE] * 9))
    r = lib.moe_route(ctypes.byref(d), None, None, None, None, ctypes.byref(plan), FAKE, 1 << 40, None)
    assert r == -1 and b"logits" in lib.moe_last_error()
    bad = B.PlanStruct(*([FAKE] * 8 + [FAKE + 4]))
    r = lib.moe_route(ctypes.byref(d), None, None, None, FAKE, ctypes.byref(bad), FAKE, 1 << 40, None)
    assert r == -1 and b"meta" in lib.moe_last_error()
    r = lib.moe_route(ctypes.byref(d), None, None, None, FAKE, None, FAKE, 1 << 40, None)
    assert r == -1 and b"plan" in lib.moe_last_error()
    # X given without W_r
    r = lib.moe_route(ctypes.byref(d), FAKE, None, None, FAKE, ctypes.byref(plan), FAKE, 1 << 40, None)
    assert r == -1 and b"W_r" in lib.moe_last_error()
    r = lib.moe_combine(ctypes.byref(d), ctypes.byref(plan), FAKE + 8, 1, FAKE, None)
    assert r == -1 and b"Y_perm" in lib.moe_last_error()


def test_workspace_too_small_rejected(lib):
    d = dims()
    plan = B.PlanStruct(*([FAKE] * 9))
    need = B.moe_workspace_bytes(d, B.OP_FORWARD)
    r = lib.moe_forward(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, ctypes.byref(plan),
                        None, FAKE, FAKE, need - 1, None)
    assert r == -3 and b"workspace" in lib.moe_last_error()
    need_b = B.moe_workspace_bytes(d, B.OP_BACKWARD)
    r = lib.moe_backward(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, FAKE, ctypes.byref(plan), None,
                         FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, need_b - 1, None)
    assert r == -3
    # dW_r without W_r is an argument error
    r = lib.moe_backward(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, FAKE, ctypes.byref(plan), None,
                         FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need_b, None)
    assert r == -1 and b"dW_r" in lib.moe_last_error()


def test_binding_raises_moe_error():
    with pytest.raises(B.MoEError) as ei:
        B.moe_max_rows(dims(K=99))
    assert ei.value.status == -1


def test_fp8_argument_checks(lib):
    """moe_quantize_fp8: K a multiple of 8, bf16 / fp32 sources, required pointers, nothing to do
    for rows = 0.  moe_grouped_ffn_fp8: bf16 layers only, required pointers, its workspace."""
    q = lambda rows, K, dt=1, src=FAKE: lib.moe_quantize_fp8(rows, K, dt, src, FAKE, FAKE, None)
    assert q(4, 12) == -1 and q(4, 0) == -1 and q(-1, 8) == -1
    assert q(4, 16, dt=7) == -2
    assert q(4, 16, src=None) == -1
    assert q(0, 16, src=None) == 0
    plan = B.PlanStruct(*([FAKE] * 9))
    ffn = lambda d, ws=1 << 40, act=FAKE: lib.moe_grouped_ffn_fp8(
        ctypes.byref(d), ctypes.byref(plan), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, act, FAKE,
        FAKE, FAKE, FAKE, ws, None)
    assert ffn(dims(dtype="f32")) == -2
    assert ffn(dims(), act=None) == -1
    need = B.moe_workspace_bytes(dims(), B.OP_FFN_FP8)
    assert need >= (8 + 1) * 4
    assert ffn(dims(), ws=need - 1) == -3


def test_decode_spin_limit_is_validated_on_the_host(lib):
    """A negative spin limit is rejected; a valid one returns the previous limit (host state only)."""
    prev = B.moe_decode_set_spin_limit(1 << 20)
    assert prev >= 0
    with pytest.raises(B.MoEError):
        B.moe_decode_set_spin_limit(-1)
    assert B.moe_decode_set_spin_limit(prev) == 1 << 20


def test_route_noalloc_rejects_layers_beyond_its_buffer(lib):
    """moe_route_noalloc checks the routing workspace the dims need against its static buffer on
    the host, before it touches the device: too large is MOE_EWORKSPACE, nothing enqueued."""
    assert B.moe_route_noalloc_max_bytes() == 64 << 20
    big = dims(T=1 << 20, E=1024, K=8, round_mode=B.ROUND_NEAREST, tile_m=128)
    assert B.moe_workspace_bytes(big, B.OP_ROUTE) > B.moe_route_noalloc_max_bytes()
    plan = B.PlanStruct(*([FAKE] * 9))
    st = lib.moe_route_noalloc(ctypes.byref(big), None, None, None, FAKE, ctypes.byref(plan), None)
    assert st == -3 and b"static buffer" in lib.moe_last_error()


def test_mx_argument_checks(lib):
    """moe_quantize_mx: K a multiple of 64, bf16 / fp32 sources, a known format, required
    pointers, nothing to do for rows = 0; moe_mx_scale_bytes: the group-major size, 0 for invalid
    sizes.  moe_grouped_ffn_mx: bf16 layers only, a known format, T * d below 2^32 (the
    gathered code offsets are 32-bit), required pointers (act optional), its workspace."""
    assert B.moe_mx_scale_bytes(10, 128) == 40 and B.moe_mx_scale_bytes(10, 192) == 80
    assert B.moe_mx_scale_bytes(0, 128) == 0 and B.moe_mx_scale_bytes(-1, 128) == 0
    q = lambda rows, K, dt=1, fmt=B.FP8_E4M3, src=FAKE, sc=FAKE: lib.moe_quantize_mx(rows, K, dt, fmt, src, FAKE, sc, None)
    assert q(4, 96) == -1 and q(4, 0) == -1 and q(-1, 128) == -1
    assert q(4, 128, dt=7) == -2
    assert q(4, 128, fmt=5) == -1
    assert q(4, 128, src=None) == -1 and q(4, 128, sc=None) == -1
    assert q(0, 128, src=None) == 0
    plan = B.PlanStruct(*([FAKE] * 9))
    ffn = lambda d, fmt=B.FP8_E4M3, ws=1 << 40, act_q=FAKE: lib.moe_grouped_ffn_mx(
        ctypes.byref(d), ctypes.byref(plan), fmt, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, act_q,
        FAKE, FAKE, FAKE, ws, None)
    assert ffn(dims(dtype="f32")) == -2
    assert ffn(dims(), fmt=9) == -1
    assert ffn(dims(T=1 << 22, d=1024)) == -2 and b"2^32" in lib.moe_last_error()
    assert ffn(dims(), act_q=None) == -1
    need = B.moe_workspace_bytes(dims(), B.OP_FFN_MX)
    R = B.moe_max_rows(dims())
    assert need >= B.moe_mx_scale_bytes(R, 128)
    assert ffn(dims(), ws=need - 1) == -3
