"""The C-ABI library loads on the CPU, exports every entry point include/moe.h
declares, and rejects invalid arguments before touching a device.  No compute
call is made here (there is no GPU in this environment)."""

import ctypes
import os
import re

import pytest

import expert_token_routing_router_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced (validation fails first)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ["moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine",
                 "moe_bias_update"]:
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = moe.lib()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(moe.EXPORTS) == declared_functions()


def test_status_strings():
    assert moe.status_string(moe.MOE_OK) == "ok"
    assert "invalid" in moe.status_string(moe.MOE_ERR_INVALID_ARG)
    assert "workspace" in moe.status_string(moe.MOE_ERR_WORKSPACE)
    assert moe.status_string(99) == "unknown status"


def _route(desc, ws_bytes=0, ptrs=True, counts=True):
    lib = moe.lib()
    p = FAKE if ptrs else None
    return lib.moe_route(ctypes.byref(desc), p, p, None, None, p, p, p, FAKE if counts else None,
                         FAKE if ws_bytes else None, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=9), moe.MOE_ERR_INVALID_ARG),               # k > E
    (dict(R=3), moe.MOE_ERR_INVALID_ARG),               # E % R != 0
    (dict(G=3), moe.MOE_ERR_INVALID_ARG),               # E % G != 0
    (dict(G=2, kg=3), moe.MOE_ERR_INVALID_ARG),         # kg > G
    (dict(E=16, G=8, kg=1, k=3), moe.MOE_ERR_INVALID_ARG),  # kg * E/G < k
    (dict(N=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(d=0), moe.MOE_ERR_INVALID_ARG),
    (dict(d=12), moe.MOE_ERR_UNSUPPORTED),              # hidden not a multiple of 8
    (dict(E=512, k=2), moe.MOE_ERR_UNSUPPORTED),        # more than 256 experts
    (dict(E=16, k=9), moe.MOE_ERR_UNSUPPORTED),         # k > 8
    (dict(E=128, G=128, kg=2), moe.MOE_ERR_UNSUPPORTED),      # more than 64 groups
    (dict(cf=float("nan")), moe.MOE_ERR_INVALID_ARG),
])
def test_route_rejects_bad_descriptors(kw, status):
    base = dict(N=64, d=64, E=8, k=2, R=4, cf=0.0, G=1, kg=1)
    base.update(kw)
    desc = moe.route_desc(base["N"], base["d"], base["E"], base["k"], base["R"], base["cf"],
                          base["G"], base["kg"])
    assert _route(desc, ws_bytes=1 << 20) == status


def test_route_bad_score_and_dtype():
    d = moe.route_desc(64, 64, 8, 2)
    d.score_fn = 7
    assert _route(d, 1 << 20) == moe.MOE_ERR_INVALID_ARG
    d = moe.route_desc(64, 64, 8, 2)
    d.dtype = 5
    assert _route(d, 1 << 20) == moe.MOE_ERR_INVALID_ARG


def test_route_null_pointers_and_workspace():
    d = moe.route_desc(64, 64, 8, 2)
    assert _route(d, 1 << 20, ptrs=False) == moe.MOE_ERR_INVALID_ARG
    assert _route(d, 1 << 20, counts=False) == moe.MOE_ERR_INVALID_ARG
    need = moe.moe_route_workspace_size(d)
    assert need > 0
    assert _route(d, 0) == moe.MOE_ERR_WORKSPACE
    assert _route(d, need - 8) == moe.MOE_ERR_WORKSPACE


def test_route_misaligned_hidden_states():
    lib = moe.lib()
    d = moe.route_desc(64, 64, 8, 2)
    odd = ctypes.c_void_p(0x10002)
    st = lib.moe_route(ctypes.byref(d), odd, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                       1 << 20, None)
    assert st == moe.MOE_ERR_INVALID_ARG


def test_dispatch_validation():
    lib = moe.lib()
    d = moe.route_desc(64, 64, 8, 2, R=4, cf=1.25)
    need = moe.moe_dispatch_workspace_size(d)
    assert need >= 8 * 4
    args = [FAKE] * 10
    assert lib.moe_dispatch(ctypes.byref(d), *args, None, 0, None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_dispatch(ctypes.byref(d), *args, FAKE, need - 4, None) == moe.MOE_ERR_WORKSPACE
    args2 = list(args)
    args2[2] = None  # x_perm
    assert lib.moe_dispatch(ctypes.byref(d), *args2, FAKE, need, None) == moe.MOE_ERR_INVALID_ARG
    bad = moe.route_desc(64, 64, 8, 2, R=3)
    assert lib.moe_dispatch(ctypes.byref(bad), *args, FAKE, need, None) == moe.MOE_ERR_INVALID_ARG


def test_dispatch_ex_validation():
    """moe_dispatch_ex checks what moe_dispatch checks, plus the admission."""
    lib = moe.lib()
    d = moe.route_desc(64, 64, 8, 2, R=4, cf=1.25)
    need = moe.moe_dispatch_workspace_size(d)
    args = [FAKE] * 10
    for adm in (-1, 4, 7, 8):
        assert lib.moe_dispatch_ex(ctypes.byref(d), adm, *args, FAKE, need,
                                   None) == moe.MOE_ERR_INVALID_ARG
    # The padded layout needs a capacity.
    nocap = moe.route_desc(64, 64, 8, 2, R=4, cf=0.0)
    need0 = moe.moe_dispatch_workspace_size(nocap)
    for adm in (moe.MOE_LAYOUT_PADDED, moe.MOE_LAYOUT_PADDED | moe.MOE_ADMIT_FIRST_CHOICE):
        assert lib.moe_dispatch_ex(ctypes.byref(nocap), adm, *args, FAKE, need0,
                                   None) == moe.MOE_ERR_INVALID_ARG
        assert lib.moe_dispatch_rows(ctypes.byref(nocap), adm) == -1
    # Rows: N*k compact, max(N*k, E*cap) padded (cap = ceil(1.25 * 128 / 8) = 20).
    assert lib.moe_dispatch_rows(ctypes.byref(d), 0) == 128
    assert lib.moe_dispatch_rows(ctypes.byref(d), moe.MOE_LAYOUT_PADDED) == 160
    assert lib.moe_dispatch_rows(ctypes.byref(d), 4) == -1
    for adm in (moe.MOE_ADMIT_TOKEN_ORDER, moe.MOE_ADMIT_FIRST_CHOICE):
        assert lib.moe_dispatch_ex(ctypes.byref(d), adm, *args, FAKE, need - 4,
                                   None) == moe.MOE_ERR_WORKSPACE
        args2 = list(args)
        args2[2] = None  # x_perm
        assert lib.moe_dispatch_ex(ctypes.byref(d), adm, *args2, FAKE, need,
                                   None) == moe.MOE_ERR_INVALID_ARG


def test_dispatch_q8_validation():
    """moe_dispatch_q8 checks what moe_dispatch_ex checks, plus its payload
    buffers and the largest row a wave quantises in registers."""
    lib = moe.lib()
    d = moe.route_desc(64, 64, 8, 2, R=4, cf=1.25)
    need = moe.moe_dispatch_workspace_size(d)
    rest = [FAKE] * 7  # row_of_slot .. rank_counts

    def call(desc, adm=0, xq=FAKE, sc=FAKE, ws_bytes=need):
        return lib.moe_dispatch_q8(ctypes.byref(desc), adm, FAKE, FAKE, xq, sc, *rest, FAKE,
                                   ws_bytes, None)
    assert call(d, xq=None) == moe.MOE_ERR_INVALID_ARG
    assert call(d, sc=None) == moe.MOE_ERR_INVALID_ARG
    assert call(d, xq=ctypes.c_void_p(0x10008)) == moe.MOE_ERR_INVALID_ARG       # 16-byte alignment
    assert call(d, sc=ctypes.c_void_p(0x10002)) == moe.MOE_ERR_INVALID_ARG       # 4-byte alignment
    assert call(d, adm=5) == moe.MOE_ERR_INVALID_ARG
    assert call(d, ws_bytes=need - 4) == moe.MOE_ERR_WORKSPACE
    assert call(moe.route_desc(64, 8200, 8, 2)) == moe.MOE_ERR_UNSUPPORTED  # > 8192 bf16
    f32 = moe.route_desc(64, 4104, 8, 2)
    f32.dtype = moe.MOE_F32
    assert call(f32) == moe.MOE_ERR_UNSUPPORTED                   # > 4096 fp32


def test_dispatch_halves_validation():
    """moe_dispatch_layout checks the layout arguments and workspace (x is not
    needed); moe_permute / moe_permute_q8 check rows, x and the output."""
    lib = moe.lib()
    d = moe.route_desc(64, 64, 8, 2, R=4, cf=1.25)
    need = moe.moe_dispatch_workspace_size(d)
    outs = [FAKE] * 7  # row_of_slot .. rank_counts
    assert lib.moe_dispatch_layout(ctypes.byref(d), 0, FAKE, *outs, FAKE, need - 4,
                                   None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_dispatch_layout(ctypes.byref(d), 4, FAKE, *outs, FAKE, need,
                                   None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch_layout(ctypes.byref(d), 0, None, *outs, FAKE, need,
                                   None) == moe.MOE_ERR_INVALID_ARG
    bad = moe.route_desc(64, 64, 8, 2, R=3)
    assert lib.moe_dispatch_layout(ctypes.byref(bad), 0, FAKE, *outs, FAKE, need,
                                   None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_permute(ctypes.byref(d), None, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_permute(ctypes.byref(d), FAKE, None, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_permute(ctypes.byref(d), FAKE, FAKE, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_permute(ctypes.byref(d), FAKE, FAKE, ctypes.c_void_p(0x10008),
                           None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_permute_q8(ctypes.byref(d), FAKE, FAKE, None, FAKE,
                              None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_permute_q8(ctypes.byref(d), FAKE, FAKE, FAKE, None,
                              None) == moe.MOE_ERR_INVALID_ARG
    wide = moe.route_desc(64, 8200, 8, 2)
    assert lib.moe_permute_q8(ctypes.byref(wide), FAKE, FAKE, FAKE, FAKE,
                              None) == moe.MOE_ERR_UNSUPPORTED


def test_dequantize_q8_validation():
    lib = moe.lib()
    ok = dict(M=16, d=64, dt=moe.MOE_BF16, q=FAKE, s=FAKE, n=FAKE, out=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.moe_dequantize_q8(a["M"], a["d"], a["dt"], a["q"], a["s"], a["n"], a["out"],
                                     None)
    assert call(M=-1) == moe.MOE_ERR_INVALID_ARG
    assert call(dt=7) == moe.MOE_ERR_INVALID_ARG
    assert call(d=60) == moe.MOE_ERR_UNSUPPORTED
    for key in ("q", "s", "n", "out"):
        assert call(**{key: None}) == moe.MOE_ERR_INVALID_ARG
    assert call(q=ctypes.c_void_p(0x10008)) == moe.MOE_ERR_INVALID_ARG
    assert call(out=ctypes.c_void_p(0x10004)) == moe.MOE_ERR_INVALID_ARG
    assert call(M=0, q=None, s=None, n=None, out=None) == moe.MOE_OK  # nothing to do


def test_expert_ffn_validation():
    lib = moe.lib()
    F = FAKE
    call = lambda E, M, d, h, act, dt, w3=None, ws=F, wsb=1 << 30: lib.moe_expert_ffn(  # noqa: E731
        E, M, d, h, act, dt, F, F, F, w3, F, F, None, ws, wsb, None)
    assert call(0, 100, 64, 64, moe.MOE_RELU, moe.MOE_BF16) == moe.MOE_ERR_INVALID_ARG
    assert call(8, -1, 64, 64, moe.MOE_RELU, moe.MOE_BF16) == moe.MOE_ERR_INVALID_ARG
    assert call(8, 100, 96, 64, moe.MOE_RELU, moe.MOE_BF16) == moe.MOE_ERR_UNSUPPORTED
    assert call(8, 100, 64, 100, moe.MOE_RELU, moe.MOE_BF16) == moe.MOE_ERR_UNSUPPORTED
    assert call(8, 100, 64, 64, 5, moe.MOE_BF16) == moe.MOE_ERR_INVALID_ARG
    assert call(8, 100, 64, 64, moe.MOE_SWIGLU, moe.MOE_BF16) == moe.MOE_ERR_INVALID_ARG  # no w3
    assert call(8, 100, 64, 64, moe.MOE_RELU, moe.MOE_BF16, w3=F) == moe.MOE_ERR_INVALID_ARG
    assert call(8, 100, 64, 64, moe.MOE_RELU, moe.MOE_BF16, ws=None) == moe.MOE_ERR_WORKSPACE
    need = moe.moe_expert_ffn_workspace_size(8, 100, 64, 64, "relu", "bf16")
    assert call(8, 100, 64, 64, moe.MOE_RELU, moe.MOE_BF16, wsb=need - 1) == moe.MOE_ERR_WORKSPACE
    assert call(8, 0, 64, 64, moe.MOE_RELU, moe.MOE_BF16) == moe.MOE_OK  # nothing to do


def test_expert_ffn_fused_validation():
    """The fused combine argument is checked before any launch: its sizes, its
    arrays and the accumulator's alignment; y_rows is optional only with it."""
    lib = moe.lib()
    F = FAKE

    def call(fc, y=None, M=100, stage="all"):
        ref = ctypes.byref(fc) if fc is not None else None
        if stage == "down":
            return lib.moe_expert_ffn_down(8, M, 64, 64, moe.MOE_RELU, moe.MOE_BF16, F, F, y, ref,
                                           F, 1 << 30, None)
        return lib.moe_expert_ffn(8, M, 64, 64, moe.MOE_RELU, moe.MOE_BF16, F, F, F, None, F, y,
                                  ref, F, 1 << 30, None)

    def fc(**kw):
        a = dict(N=10, k=2, w=0x10000, tor=0x10000, sor=0x10000, acc=0x10000)
        a.update(kw)
        return moe.FusedCombine(a["N"], a["k"], a["w"], a["tor"], a["sor"], a["acc"])

    for stage in ("all", "down"):
        assert call(None, stage=stage) == moe.MOE_ERR_INVALID_ARG  # neither y_rows nor fused
        assert call(fc(k=0), stage=stage) == moe.MOE_ERR_INVALID_ARG
        assert call(fc(k=9), stage=stage) == moe.MOE_ERR_INVALID_ARG
        assert call(fc(N=-1), stage=stage) == moe.MOE_ERR_INVALID_ARG
        assert call(fc(w=None), stage=stage) == moe.MOE_ERR_INVALID_ARG
        assert call(fc(tor=None), stage=stage) == moe.MOE_ERR_INVALID_ARG
        assert call(fc(sor=None), stage=stage) == moe.MOE_ERR_INVALID_ARG
        assert call(fc(acc=None), stage=stage) == moe.MOE_ERR_INVALID_ARG
        assert call(fc(acc=0x10008), stage=stage) == moe.MOE_ERR_INVALID_ARG  # misaligned
        # no rows and no tokens: nothing to do
        assert call(fc(N=0, tor=None, sor=None, w=None, acc=None), M=0, stage=stage) == moe.MOE_OK


def test_dispatch_noalloc_validation():
    """The dispatch without a workspace checks its arguments, and that the batch
    fits its static scratch (1 MiB), before touching any device."""
    lib = moe.lib()
    F = FAKE

    def call(desc, adm=0, **null):
        args = [F] * 10
        for i in null.get("at", ()):
            args[i] = None
        return lib.moe_dispatch_noalloc(ctypes.byref(desc), adm, *args, None)

    # 2^21 slots over 256 experts: 2048 tiles x 256 experts x 4 bytes = 2 MiB
    assert call(moe.route_desc(1 << 18, 64, 256, 8, 8)) == moe.MOE_ERR_UNSUPPORTED
    assert call(moe.route_desc(64, 64, 8, 9)) == moe.MOE_ERR_INVALID_ARG       # k > E
    assert call(moe.route_desc(64, 64, 8, 2), adm=8) == moe.MOE_ERR_INVALID_ARG  # bad flags
    assert call(moe.route_desc(64, 64, 8, 2), adm=moe.MOE_LAYOUT_PADDED) == \
        moe.MOE_ERR_INVALID_ARG  # padded layout needs a capacity
    for i in range(10):  # every array is required for a non-empty batch
        assert call(moe.route_desc(64, 64, 8, 2), at=(i,)) == moe.MOE_ERR_INVALID_ARG, i


def test_pack_weights_validation():
    lib = moe.lib()
    pack = lib.moe_expert_ffn_pack_weights
    A, B = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x10000 + (1 << 30))
    assert pack(0, 64, 64, moe.MOE_BF16, A, B, None) == moe.MOE_ERR_INVALID_ARG
    assert pack(2, 64, 64, 7, A, B, None) == moe.MOE_ERR_INVALID_ARG
    assert pack(2, 64, 64, moe.MOE_F32, A, B, None) == moe.MOE_ERR_UNSUPPORTED
    assert pack(2, 96, 64, moe.MOE_BF16, A, B, None) == moe.MOE_ERR_UNSUPPORTED
    assert pack(2, 64, 32, moe.MOE_BF16, A, B, None) == moe.MOE_ERR_UNSUPPORTED
    assert pack(2, 64, 64, moe.MOE_BF16, None, B, None) == moe.MOE_ERR_INVALID_ARG
    assert pack(2, 64, 64, moe.MOE_BF16, A, ctypes.c_void_p(0x10008), None) == \
        moe.MOE_ERR_INVALID_ARG  # misaligned
    assert pack(2, 64, 64, moe.MOE_BF16, A, ctypes.c_void_p(0x10000 + 4096), None) == \
        moe.MOE_ERR_INVALID_ARG  # overlaps the source


def test_combine_and_bias_validation():
    lib = moe.lib()
    d = moe.route_desc(64, 64, 8, 2)
    assert lib.moe_combine(ctypes.byref(d), None, FAKE, FAKE, None, None, None, FAKE, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(ctypes.byref(moe.route_desc(0, 64, 8, 2)), None, None, None, None,
                           None, None, None, None) == moe.MOE_OK
    # Finishing a fused accumulator needs neither y_perm nor the routing arrays,
    # but the accumulator must be 16-byte aligned and y present.
    assert lib.moe_combine(ctypes.byref(d), None, None, None, None, None,
                           ctypes.c_void_p(0x10004), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(ctypes.byref(d), None, None, None, None, None, FAKE, None,
                           None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_bias_update(0, 10, 1, FAKE, 1e-3, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_bias_update(8, 10, 1, None, 1e-3, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_bias_update(8, 10, 1, FAKE, float("inf"), FAKE, None) == \
        moe.MOE_ERR_INVALID_ARG


def test_binding_requires_device_tensors():
    import torch
    desc = moe.route_desc(4, 64, 8, 2)
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moe.moe_route(desc, x, x, None, None, None, None, None, None, None)


def test_bench_refuses_more_than_one_gpu(capsys, monkeypatch):
    """bench.py --gpus 2 prints why and exits with status 2 before touching a GPU."""
    import json
    import sys

    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as ex:
        bench.main()
    assert ex.value.code == 2
    assert "one GPU" in json.loads(capsys.readouterr().out.strip())["error"]


def test_backward_validation():
    lib = moe.lib()
    d = moe.route_desc(64, 64, 8, 2)
    args = [FAKE] * 6
    for i in range(6):
        bad = list(args)
        bad[i] = None
        assert lib.moe_combine_backward(ctypes.byref(d), *bad, None) == moe.MOE_ERR_INVALID_ARG
    mis = list(args)
    mis[0] = ctypes.c_void_p(0x10008)  # dy misaligned
    assert lib.moe_combine_backward(ctypes.byref(d), *mis, None) == moe.MOE_ERR_INVALID_ARG
    for i in range(3):
        bad = [FAKE] * 3
        bad[i] = None
        assert lib.moe_permute_backward(ctypes.byref(d), *bad, None) == moe.MOE_ERR_INVALID_ARG
    bad_desc = moe.route_desc(64, 64, 8, 2, R=3)
    assert lib.moe_permute_backward(ctypes.byref(bad_desc), FAKE, FAKE, FAKE,
                                    None) == moe.MOE_ERR_INVALID_ARG


def test_expert_ffn_backward_validation():
    """Host-side checks of moe_expert_ffn_backward: every rejected call returns
    before any launch (no device is touched)."""
    lib = moe.lib()
    E, M, d, h = 4, 100, 64, 96
    need = lib.moe_expert_ffn_backward_workspace_size(E, M, d, h, moe.MOE_SWIGLU, moe.MOE_BF16)
    assert need > 0
    # fp32, a d or h off the 32 grid, and too many experts are unsupported.
    assert lib.moe_expert_ffn_backward_workspace_size(E, M, d, h, moe.MOE_SWIGLU, moe.MOE_F32) == 0
    assert lib.moe_expert_ffn_backward_workspace_size(E, M, 48, h, moe.MOE_SWIGLU,
                                                      moe.MOE_BF16) == 0
    assert lib.moe_expert_ffn_backward_workspace_size(1025, M, d, h, moe.MOE_GELU,
                                                      moe.MOE_BF16) == 0

    def call(E=E, M=M, d=d, h=h, act=moe.MOE_SWIGLU, dtype=moe.MOE_BF16, x=FAKE, off=FAKE,
             w3=FAKE, dw3=FAKE, dy=FAKE, ws=FAKE, ws_bytes=need, rows=None):
        return lib.moe_expert_ffn_backward(E, M, d, h, act, dtype, x, off, rows, FAKE, w3, FAKE,
                                           dy, FAKE, FAKE, dw3, FAKE, ws, ws_bytes, None)

    assert call(dtype=moe.MOE_F32) == moe.MOE_ERR_UNSUPPORTED
    assert call(d=48) == moe.MOE_ERR_UNSUPPORTED
    assert call(h=80) == moe.MOE_ERR_UNSUPPORTED
    assert call(E=0) == moe.MOE_ERR_INVALID_ARG
    assert call(M=-1) == moe.MOE_ERR_INVALID_ARG
    assert call(act=3) == moe.MOE_ERR_INVALID_ARG
    assert call(dtype=7) == moe.MOE_ERR_INVALID_ARG
    assert call(off=None) == moe.MOE_ERR_INVALID_ARG
    assert call(w3=None) == moe.MOE_ERR_INVALID_ARG          # SwiGLU needs W3 ...
    assert call(dw3=None) == moe.MOE_ERR_INVALID_ARG         # ... and its gradient
    assert call(act=moe.MOE_GELU) == moe.MOE_ERR_INVALID_ARG  # GELU takes neither
    assert call(x=None) == moe.MOE_ERR_INVALID_ARG
    assert call(dy=ctypes.c_void_p(0x10008)) == moe.MOE_ERR_INVALID_ARG  # misaligned
    assert call(rows=ctypes.c_void_p(0x10002)) == moe.MOE_ERR_INVALID_ARG  # misaligned int32
    assert call(ws_bytes=need - 1) == moe.MOE_ERR_WORKSPACE
    assert call(ws=None) == moe.MOE_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p(0x10010)) == moe.MOE_ERR_WORKSPACE  # not 256-aligned


def test_expert_ffn_backward_packed_validation():
    """Host-side checks of moe_expert_ffn_backward_packed (the backward's own
    checks plus the forward GEMM's 64-grid for d and h) and of
    moe_expert_ffn_pack_weights_t: every rejected call returns before any
    launch."""
    lib = moe.lib()
    E, M, d, h = 4, 100, 64, 128
    need = lib.moe_expert_ffn_backward_packed_workspace_size(E, M, d, h, moe.MOE_SWIGLU,
                                                             moe.MOE_BF16)
    assert need > lib.moe_expert_ffn_backward_workspace_size(E, M, d, h, moe.MOE_SWIGLU,
                                                             moe.MOE_BF16)
    for args in ((E, M, 96, h, moe.MOE_SWIGLU, moe.MOE_BF16),     # d on the 32 grid only
                 (E, M, d, 96, moe.MOE_GELU, moe.MOE_BF16),       # h likewise
                 (E, M, d, h, moe.MOE_SWIGLU, moe.MOE_F32),
                 (1025, M, d, h, moe.MOE_RELU, moe.MOE_BF16)):
        assert lib.moe_expert_ffn_backward_packed_workspace_size(*args) == 0, args

    def call(E=E, M=M, d=d, h=h, act=moe.MOE_SWIGLU, dtype=moe.MOE_BF16, x=FAKE, off=FAKE,
             w1=FAKE, w3=FAKE, w2t=FAKE, w13t=FAKE, dw3=FAKE, dy=FAKE, ws=FAKE, ws_bytes=need,
             rows=None):
        return lib.moe_expert_ffn_backward_packed(E, M, d, h, act, dtype, x, off, rows, w1, w3,
                                                  w2t, w13t, dy, FAKE, FAKE, dw3, FAKE, ws,
                                                  ws_bytes, None)

    assert call(d=96) == moe.MOE_ERR_UNSUPPORTED
    assert call(h=96) == moe.MOE_ERR_UNSUPPORTED
    assert call(dtype=moe.MOE_F32) == moe.MOE_ERR_UNSUPPORTED
    assert call(E=0) == moe.MOE_ERR_INVALID_ARG
    assert call(act=3) == moe.MOE_ERR_INVALID_ARG
    assert call(off=None) == moe.MOE_ERR_INVALID_ARG
    for key in ("w1", "w2t", "w13t"):
        assert call(**{key: None}) == moe.MOE_ERR_INVALID_ARG, key
        assert call(**{key: ctypes.c_void_p(0x10008)}) == moe.MOE_ERR_INVALID_ARG, key
    assert call(w3=None) == moe.MOE_ERR_INVALID_ARG          # SwiGLU needs W3 ...
    assert call(dw3=None) == moe.MOE_ERR_INVALID_ARG         # ... and its gradient
    assert call(act=moe.MOE_GELU) == moe.MOE_ERR_INVALID_ARG  # GELU takes neither
    assert call(x=None) == moe.MOE_ERR_INVALID_ARG
    assert call(rows=ctypes.c_void_p(0x10002)) == moe.MOE_ERR_INVALID_ARG
    assert call(ws_bytes=need - 1) == moe.MOE_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p(0x10010)) == moe.MOE_ERR_WORKSPACE

    pack = lib.moe_expert_ffn_pack_weights_t
    A, B, C = (ctypes.c_void_p(0x10000), ctypes.c_void_p(0x10000 + (1 << 30)),
               ctypes.c_void_p(0x10000 + (2 << 30)))
    assert pack(0, 64, 64, 64, moe.MOE_BF16, A, None, B, None) == moe.MOE_ERR_INVALID_ARG
    assert pack(2, 64, 128, 64, moe.MOE_BF16, A, None, B, None) == moe.MOE_ERR_INVALID_ARG
    assert pack(2, 64, 64, 64, moe.MOE_F32, A, None, B, None) == moe.MOE_ERR_UNSUPPORTED
    assert pack(2, 96, 64, 64, moe.MOE_BF16, A, None, B, None) == moe.MOE_ERR_UNSUPPORTED
    assert pack(2, 64, 60, 128, moe.MOE_BF16, A, C, B, None) == moe.MOE_ERR_UNSUPPORTED
    assert pack(2, 64, 64, 128, moe.MOE_BF16, A, None, B, None) == moe.MOE_ERR_INVALID_ARG
    assert pack(2, 64, 64, 64, moe.MOE_BF16, A, C, B, None) == moe.MOE_ERR_INVALID_ARG
    assert pack(2, 64, 64, 128, moe.MOE_BF16, A, C, ctypes.c_void_p(0x10000 + 4096), None) == \
        moe.MOE_ERR_INVALID_ARG  # overlaps wa
