"""The C ABI on the host: the library loads, exports what the header declares, and
rejects bad arguments before touching the device (no GPU needed)."""
import ctypes
import os
import re

import pytest

import tensor_mlp_shard_amd as tpm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp_mlp_shard.h")

OK, INVALID, SHAPE, ALIGN = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tpm.LIB_PATH):
        from tensor_mlp_shard_amd import build
        build.build()
    return tpm.capi()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_\w+|tpm_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["tp_mlp_shard_plan", "tp_mlp_shard_create", "tp_mlp_shard_fwd",
              "tp_partials_reduce", "tp_mlp_shard_destroy", "tpm_status_str"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(6):
        assert tpm.tpm_status_str(s)
    assert tpm.tpm_status_str(99) == "unknown status"


def desc(**kw):
    base = dict(d_model=8192, ffn_shard=3584, max_tokens=8192, activation="silu_gate",
                in_dtype=tpm.BF16, out_dtype=tpm.F32, path="auto")
    base.update(kw)
    return tpm.make_desc(**base)


def plan_rc(d):
    info = tpm.TpmPlanInfo()
    return tpm.capi().tp_mlp_shard_plan(ctypes.byref(d), ctypes.byref(info)), info


def test_plan_decode_shard_sizes(lib):
    p = tpm.tp_mlp_shard_plan(desc())
    assert p["packed_weight_bytes"] == 8192 * 7168 * 2 + 8192 * 3584 * 2
    assert p["ffn_padded"] == 3584
    assert p["stream_max_tokens"] == 64 and p["kernels_per_fwd"] == 2
    assert p["workspace_bytes"] >= 8192 * 3584 * 2


def test_plan_pads_ragged_ffn(lib):
    p = tpm.tp_mlp_shard_plan(desc(d_model=512, ffn_shard=200, activation="tanh"))
    assert p["ffn_padded"] == 256
    p = tpm.tp_mlp_shard_plan(desc(d_model=512, ffn_shard=200, activation="silu_gate"))
    assert p["ffn_padded"] == 256
    p = tpm.tp_mlp_shard_plan(desc(d_model=64, ffn_shard=7, in_dtype=tpm.F32, activation="tanh"))
    assert p["ffn_padded"] == 7 and p["stream_max_tokens"] == 0


@pytest.mark.parametrize("kw,code", [
    (dict(d_model=0), SHAPE), (dict(ffn_shard=0), SHAPE), (dict(max_tokens=-1), SHAPE),
    (dict(d_model=8200), SHAPE),  # bf16 needs d % 64 == 0
    (dict(d_model=8200, in_dtype=tpm.F32), OK),
    (dict(in_dtype=7), INVALID), (dict(out_dtype=-1), INVALID),
    (dict(d_model=1 << 21), SHAPE),
])
def test_plan_validation(lib, kw, code):
    rc, _ = plan_rc(desc(**kw))
    assert rc == code


def test_plan_rejects_bad_enums_and_nulls(lib):
    d = desc()
    d.act = 3
    assert plan_rc(d)[0] == INVALID
    d = desc()
    d.path = 9
    assert plan_rc(d)[0] == INVALID
    info = tpm.TpmPlanInfo()
    assert lib.tp_mlp_shard_plan(None, ctypes.byref(info)) == INVALID
    assert lib.tp_mlp_shard_plan(ctypes.byref(desc()), None) == INVALID


def test_create_rejects_before_any_device_work(lib):
    h = ctypes.c_void_p(1234)
    d = desc()
    assert lib.tp_mlp_shard_create(ctypes.byref(d), None, None, None, ctypes.byref(h)) == INVALID
    assert h.value is None  # out is cleared on error
    assert lib.tp_mlp_shard_create(ctypes.byref(d), ctypes.c_void_p(0x1000),
                                   ctypes.c_void_p(0x1008), None, ctypes.byref(h)) == ALIGN
    bad = desc(d_model=100)
    assert lib.tp_mlp_shard_create(ctypes.byref(bad), ctypes.c_void_p(0x1000),
                                   ctypes.c_void_p(0x2000), None, ctypes.byref(h)) == SHAPE
    assert lib.tp_mlp_shard_create(ctypes.byref(d), ctypes.c_void_p(0x1000),
                                   ctypes.c_void_p(0x2000), None, None) == INVALID


def test_fwd_and_destroy_null_handle(lib):
    assert lib.tp_mlp_shard_fwd(None, ctypes.c_void_p(0x1000), 4, ctypes.c_void_p(0x2000),
                                None) == INVALID
    assert lib.tp_mlp_shard_destroy(None) == OK
    assert lib.tp_mlp_shard_set_timing_events(None, None, 0) == INVALID


def _ptrs(*vals):
    return (ctypes.c_void_p * len(vals))(*vals)


def test_reduce_validation(lib):
    p = _ptrs(0x1000, 0x2000)
    out = ctypes.c_void_p(0x3000)
    assert lib.tp_partials_reduce(None, 2, 16, 0, out, 0, None) == INVALID
    assert lib.tp_partials_reduce(p, 2, 16, 0, None, 0, None) == INVALID
    assert lib.tp_partials_reduce(p, 0, 16, 0, out, 0, None) == SHAPE
    assert lib.tp_partials_reduce(_ptrs(*([0x1000] * 17)), 17, 16, 0, out, 0, None) == SHAPE
    assert lib.tp_partials_reduce(p, 2, -1, 0, out, 0, None) == SHAPE
    assert lib.tp_partials_reduce(p, 2, 16, 5, out, 0, None) == INVALID
    assert lib.tp_partials_reduce(p, 2, 16, 0, out, 5, None) == INVALID
    assert lib.tp_partials_reduce(_ptrs(0x1000, None), 2, 16, 0, out, 0, None) == INVALID
    assert lib.tp_partials_reduce(_ptrs(0x1000, 0x2004), 2, 16, 0, out, 0, None) == ALIGN
    assert lib.tp_partials_reduce(p, 2, 16, 0, ctypes.c_void_p(0x3002), 0, None) == ALIGN
    # in-place needs the same dtype
    assert lib.tp_partials_reduce(p, 2, 16, 0, ctypes.c_void_p(0x1000), 1, None) == INVALID
    # numel = 0 is a no-op that never touches the device
    assert lib.tp_partials_reduce(p, 2, 0, 0, out, 0, None) == OK


def test_python_wrapper_shard_count_mismatch():
    with pytest.raises(ValueError):
        tpm.tensor_parallel_output(None, [1, 2], [1])


def test_reduce_add_rmsnorm_validation(lib):
    f = lib.tp_partials_reduce_add_rmsnorm
    p = _ptrs(0x1000, 0x2000)
    r, ro, g, y = (ctypes.c_void_p(a) for a in (0x3000, 0x4000, 0x5000, 0x6000))

    def call(parts=p, k=2, rows=4, cols=64, ind=0, res=r, resout=ro, resd=0, gam=g, eps=1e-6,
             yy=y, outd=0):
        return f(parts, k, rows, cols, ind, res, resout, resd, gam, ctypes.c_float(eps), yy, outd,
                 None)

    assert call(parts=None) == INVALID
    for kw in ("res", "resout", "gam", "yy"):
        assert call(**{kw: None}) == INVALID, kw
    for kw in ("ind", "resd", "outd"):
        assert call(**{kw: 7}) == INVALID, kw
    assert call(eps=-1.0) == INVALID
    assert call(eps=float("nan")) == INVALID
    assert call(eps=float("inf")) == INVALID
    assert call(k=0) == SHAPE
    assert call(k=17, parts=_ptrs(*([0x1000] * 17))) == SHAPE
    assert call(rows=-1) == SHAPE
    assert call(rows=1 << 31) == SHAPE
    for cols in (0, 4, 12, 32776, 1 << 20):
        assert call(cols=cols) == SHAPE, cols
    assert call(parts=_ptrs(0x1000, None)) == INVALID
    assert call(parts=_ptrs(0x1000, 0x2008)) == ALIGN
    assert call(yy=ctypes.c_void_p(0x6002)) == ALIGN
    assert call(gam=ctypes.c_void_p(0x5004)) == ALIGN
    # rows = 0 is a no-op that never touches the device
    assert call(rows=0) == OK


def test_fp8_validation(lib):
    qf, rf = lib.tp_partials_quantize_fp8, lib.tp_partials_reduce_fp8
    x, q, s = (ctypes.c_void_p(a) for a in (0x1000, 0x2000, 0x3000))
    assert qf(None, 4, 64, 0, q, s, None) == INVALID
    assert qf(x, 4, 64, 0, None, s, None) == INVALID
    assert qf(x, 4, 64, 0, q, None, None) == INVALID
    assert qf(x, 4, 64, 9, q, s, None) == INVALID
    for cols in (0, 8, 24, 32784):
        assert qf(x, 4, cols, 0, q, s, None) == SHAPE, cols
    assert qf(x, -1, 64, 0, q, s, None) == SHAPE
    assert qf(ctypes.c_void_p(0x1004), 4, 64, 0, q, s, None) == ALIGN
    assert qf(x, 0, 64, 0, q, s, None) == OK
    qs, ss, out = _ptrs(0x1000, 0x2000), _ptrs(0x3000, 0x4000), ctypes.c_void_p(0x5000)
    assert rf(None, ss, 2, 4, 64, out, 0, None) == INVALID
    assert rf(qs, None, 2, 4, 64, out, 0, None) == INVALID
    assert rf(qs, ss, 2, 4, 64, None, 0, None) == INVALID
    assert rf(qs, ss, 2, 4, 64, out, 3, None) == INVALID
    assert rf(qs, ss, 0, 4, 64, out, 0, None) == SHAPE
    assert rf(qs, ss, 2, 4, 40, out, 0, None) == SHAPE
    assert rf(qs, _ptrs(0x3000, None), 2, 4, 64, out, 0, None) == INVALID
    assert rf(_ptrs(0x1000, 0x2001), ss, 2, 4, 64, out, 0, None) == ALIGN
    assert rf(qs, ss, 2, 0, 64, out, 0, None) == OK


def test_proj_validation(lib):
    def rc(**kw):
        base = dict(in_features=8192, out_features=1280, max_tokens=64, in_dtype=tpm.BF16,
                    out_dtype=tpm.F32, path=0)
        base.update(kw)
        d = tpm.TpmProjDesc(base["in_features"], base["out_features"], base["max_tokens"],
                            base["in_dtype"], base["out_dtype"], base["path"], 0)
        h = ctypes.c_void_p()
        return lib.tp_proj_create(ctypes.byref(d), ctypes.c_void_p(0x1000), None, ctypes.byref(h)), h
    for kw, code in [({"in_dtype": 5}, INVALID), ({"out_dtype": 5}, INVALID), ({"path": 3}, INVALID),
                     ({"in_features": 0}, SHAPE), ({"out_features": 0}, SHAPE),
                     ({"max_tokens": -1}, SHAPE), ({"in_features": 100}, SHAPE),
                     ({"in_features": 1 << 21}, SHAPE)]:
        r, h = rc(**kw)
        assert r == code, kw
        assert not h.value
    d = tpm.TpmProjDesc(64, 64, 8, tpm.BF16, tpm.F32, 0, 0)
    h = ctypes.c_void_p()
    assert lib.tp_proj_create(ctypes.byref(d), None, None, ctypes.byref(h)) == INVALID
    assert lib.tp_proj_create(ctypes.byref(d), ctypes.c_void_p(0x1001), None, ctypes.byref(h)) == ALIGN
    assert lib.tp_proj_create(None, ctypes.c_void_p(0x1000), None, ctypes.byref(h)) == INVALID
    assert lib.tp_proj_fwd(None, None, 0, None, None) == INVALID
    assert lib.tp_proj_destroy(None) == OK


def test_moe_validation(lib):
    def create(**kw):
        base = dict(d=512, F=256, E=4, T=64, act=1, ind=tpm.BF16, outd=tpm.F32, path=0)
        base.update(kw)
        d = tpm.TpmMoeDesc(base["d"], base["F"], base["E"], base["T"], base["act"], base["ind"],
                           base["outd"], base["path"])
        h = ctypes.c_void_p()
        rc = lib.tp_moe_create(ctypes.byref(d), ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000),
                               None, ctypes.byref(h))
        return rc, h
    for kw, code in [({"act": 5}, INVALID), ({"ind": tpm.F32}, INVALID), ({"outd": 4}, INVALID),
                     ({"d": 100}, SHAPE), ({"d": 0}, SHAPE), ({"F": 0}, SHAPE), ({"E": 0}, SHAPE),
                     ({"E": 1025}, SHAPE), ({"T": -1}, SHAPE), ({"path": 3}, INVALID),
                     ({"path": -1}, INVALID)]:
        rc, h = create(**kw)
        assert rc == code, kw
        assert not h.value
    assert lib.tp_moe_fwd(None, None, None, 0, None, None) == INVALID
    assert lib.tp_moe_destroy(None) == OK


def test_attn_merge_validation(lib):
    v, m, e = _ptrs(0x1000, 0x2000), _ptrs(0x5000, 0x6000), _ptrs(0x7000, 0x8000)
    out = ctypes.c_void_p(0x3000)
    mo, eo = ctypes.c_void_p(0x9000), ctypes.c_void_p(0xa000)
    f = lib.tp_attn_partials_merge
    assert f(None, m, e, 2, 4, 16, 0, out, 0, None, None, None) == INVALID
    assert f(v, None, e, 2, 4, 16, 0, out, 0, None, None, None) == INVALID
    assert f(v, m, e, 2, 4, 16, 0, None, 0, None, None, None) == INVALID
    assert f(v, m, e, 2, 4, 16, 3, out, 0, None, None, None) == INVALID   # dtype
    assert f(v, m, e, 2, 4, 16, 0, out, 0, mo, None, None) == INVALID     # one statistic only
    assert f(v, m, e, 0, 4, 16, 0, out, 0, None, None, None) == SHAPE
    assert f(_ptrs(*([0x1000] * 17)), _ptrs(*([0x5000] * 17)), _ptrs(*([0x7000] * 17)),
             17, 4, 16, 0, out, 0, None, None, None) == SHAPE
    assert f(v, m, e, 2, -1, 16, 0, out, 0, None, None, None) == SHAPE
    assert f(v, m, e, 2, 4, 12, 0, out, 0, None, None, None) == SHAPE   # dim not a multiple of 8
    assert f(v, m, e, 2, 4, 0, 0, out, 0, None, None, None) == SHAPE
    assert f(_ptrs(0x1000, None), m, e, 2, 4, 16, 0, out, 0, None, None, None) == INVALID
    assert f(_ptrs(0x1000, 0x2008), m, e, 2, 4, 16, 0, out, 0, None, None, None) == ALIGN
    assert f(v, _ptrs(0x5000, 0x6002), e, 2, 4, 16, 0, out, 0, None, None, None) == ALIGN
    assert f(v, m, e, 2, 4, 16, 0, ctypes.c_void_p(0x3004), 0, None, None, None) == ALIGN
    # merged statistics may not land on an input's statistics
    assert f(v, m, e, 2, 4, 16, 0, out, 0, ctypes.c_void_p(0x6000), eo, None) == INVALID
    assert f(v, m, e, 2, 4, 16, 0, out, 0, mo, ctypes.c_void_p(0x7000), None) == INVALID
    # in place over rank 0's values needs the same dtype
    assert f(v, m, e, 2, 4, 16, 0, ctypes.c_void_p(0x1000), 1, None, None, None) == INVALID
    # rows = 0 is a no-op that never touches the device
    assert f(v, m, e, 2, 0, 16, 0, out, 0, mo, eo, None) == OK


HIP_ERR = 4  # TPM_ERR_HIP


def _no_device():
    try:
        import torch
        return not torch.cuda.is_available()
    except Exception:
        return True


@pytest.mark.skipif(not _no_device(), reason="the HIP error path is forced by having no device")
def test_create_without_a_device_reports_hip_error(lib):
    """With no GPU, the first HIP call of each create (hipGetDevice) fails: the call
    returns TPM_ERR_HIP, clears *out and leaves nothing allocated; no kernel is
    launched since the failure comes before any allocation."""
    h = ctypes.c_void_p(1234)
    d = desc(d_model=64, ffn_shard=128, max_tokens=8)
    assert lib.tp_mlp_shard_create(ctypes.byref(d), ctypes.c_void_p(0x1000),
                                   ctypes.c_void_p(0x2000), None, ctypes.byref(h)) == HIP_ERR
    assert h.value is None
    pd = tpm.TpmProjDesc(64, 64, 8, tpm.BF16, tpm.F32, 0, 0)
    h = ctypes.c_void_p(1234)
    assert lib.tp_proj_create(ctypes.byref(pd), ctypes.c_void_p(0x1000), None,
                              ctypes.byref(h)) == HIP_ERR
    assert h.value is None
    md = tpm.TpmMoeDesc(512, 256, 4, 64, 1, tpm.BF16, tpm.F32, 0)
    h = ctypes.c_void_p(1234)
    assert lib.tp_moe_create(ctypes.byref(md), ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000),
                             None, ctypes.byref(h)) == HIP_ERR
    assert h.value is None
