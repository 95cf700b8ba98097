"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, agrees with the oracle on the NF4 levels, and rejects bad arguments
synchronously with the documented codes (nothing is launched)."""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import formats as ofmt
from quantized_base_lora_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


@pytest.fixture(scope="module")
def lib():
    return binding.load()


def test_header_lists_the_four_named_calls():
    names = declared_functions()
    for n in ("quant_pack", "qlora_linear_fwd", "qlora_linear_bwd", "layer_stream_prefetch"):
        assert n in names
    assert len(names) >= 16


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(binding.EXPORTS) <= set(declared_functions())


def test_version(lib):
    assert binding.version() == 1


def test_nf4_levels_equal_oracle_bitwise():
    ours = np.array(binding.nf4_levels(), dtype=np.float32)
    assert np.array_equal(ours.view(np.uint32), ofmt.nf4_codebook().view(np.uint32))


@pytest.mark.parametrize("signed", [True, False])
def test_dyn8_levels_equal_oracle_bitwise(signed):
    """The library's 8-bit optimizer-state levels, built by its own routine at
    compile time, equal the oracle's bit for bit."""
    from oracle import adamw8
    ours = np.array(binding.dyn8_levels(signed), dtype=np.float32)
    assert np.array_equal(ours.view(np.uint32), adamw8.dynamic_levels(signed).view(np.uint32))


def test_adamw8_argument_errors(lib):
    P = FAKE.value
    hp = binding.AdamwHparamsC(1e-3, 0.9, 0.999, 1e-8, 0.0, 1.0, 1, 0)
    t = (binding.Adamw8TensorC * 1)(binding.Adamw8TensorC(P, P, P, P, P, P, None, 12))
    assert lib.ql_adamw8_step(t, 1, ctypes.byref(hp), None) == binding.QL_EINVAL     # n % 8
    assert "multiple of 8" in _err(lib)
    t = (binding.Adamw8TensorC * 1)(binding.Adamw8TensorC(P, P, P + 4, P, P, P, None, 16))
    assert lib.ql_adamw8_step(t, 1, ctypes.byref(hp), None) == binding.QL_EINVAL     # codes not 8-byte aligned
    t = (binding.Adamw8TensorC * 1)(binding.Adamw8TensorC(P, None, P, P, P, P, None, 16))
    assert lib.ql_adamw8_step(t, 1, ctypes.byref(hp), None) == binding.QL_EINVAL
    bad = binding.AdamwHparamsC(1e-3, 1.0, 0.999, 1e-8, 0.0, 1.0, 1, 0)
    t = (binding.Adamw8TensorC * 1)(binding.Adamw8TensorC(P, P, P, P, P, P, None, 16))
    assert lib.ql_adamw8_step(t, 1, ctypes.byref(bad), None) == binding.QL_EINVAL
    bad = binding.AdamwHparamsC(1e-3, 0.9, 0.999, 1e-8, 0.0, 1.0, 0, 0)
    assert lib.ql_adamw8_step(t, 1, ctypes.byref(bad), None) == binding.QL_EINVAL
    assert lib.ql_adamw8_step(t, 33, ctypes.byref(hp), None) == binding.QL_EINVAL


def test_workspace_query(lib):
    assert binding.workspace_bytes(binding.OP_PACK, binding.FMT_NF4, 64, 64) >= 8
    a = binding.workspace_bytes(binding.OP_BWD, binding.FMT_NF4, 1024, 2048, 1000, 16)
    b = binding.workspace_bytes(binding.OP_BWD, binding.FMT_NF4, 1024, 2048, 8192, 16)
    assert b > a >= 16 * 1024 * 2 + 1000 * 16 * 4
    assert a % 256 == 0 and b % 256 == 0


FAKE = ctypes.c_void_p(0x10000)       # aligned, never dereferenced: calls fail before any launch


def _qw(fmt=binding.FMT_NF4, n=64, k=128, reserved=0, codes=FAKE.value, scales=FAKE.value):
    return binding.QWeightC(fmt, reserved, n, k, codes, scales)


def _err(lib):
    return lib.ql_last_error().decode()


def test_pack_argument_errors(lib):
    P = FAKE
    assert lib.quant_pack(9, P, 64, 128, P, P, P, 256, None) == binding.QL_EUNSUPPORTED
    assert lib.quant_pack(binding.FMT_NF4, P, 64, 96, P, P, P, 256, None) == binding.QL_EINVAL
    assert "multiple of 64" in _err(lib)
    assert lib.quant_pack(binding.FMT_NVFP4, P, 64, 48, P, P, P, 256, None) == binding.QL_EINVAL
    assert "multiple of 32" in _err(lib)
    assert lib.quant_pack(binding.FMT_Q4_0, P, 48, 64, P, P, P, 256, None) == binding.QL_EINVAL
    assert lib.quant_pack(binding.FMT_Q4_0, None, 64, 64, P, P, P, 256, None) == binding.QL_EINVAL
    assert lib.quant_pack(binding.FMT_Q4_0, ctypes.c_void_p(0x10004), 64, 64, P, P, P, 256, None) == binding.QL_EINVAL
    assert lib.quant_pack(binding.FMT_FP8, P, 64, 64, P, P, P, 8, None) == binding.QL_EWORKSPACE


def test_layer_argument_errors(lib):
    P = FAKE
    qw = _qw()
    fwd = lib.qlora_linear_fwd
    assert fwd(ctypes.byref(qw), P, 16, P, P, 12, 16.0, P, P, None, 0, None) == binding.QL_EUNSUPPORTED
    assert fwd(ctypes.byref(qw), None, 16, P, P, 16, 16.0, P, P, None, 0, None) == binding.QL_EINVAL
    assert fwd(ctypes.byref(qw), P, -1, P, P, 16, 16.0, P, P, None, 0, None) == binding.QL_EINVAL
    assert fwd(ctypes.byref(qw), P, 0, P, P, 16, 16.0, P, P, None, 0, None) == binding.QL_OK
    bad = _qw(reserved=1)
    assert fwd(ctypes.byref(bad), P, 16, P, P, 16, 16.0, P, P, None, 0, None) == binding.QL_EINVAL
    bad = _qw(codes=0x10008)
    assert fwd(ctypes.byref(bad), P, 16, P, P, 16, 16.0, P, P, None, 0, None) == binding.QL_EINVAL
    bwd = lib.qlora_linear_bwd
    assert bwd(ctypes.byref(qw), P, P, P, 1024, P, P, 16, 16.0, P, P, P, 0, P, 0, None) == binding.QL_EWORKSPACE
    assert bwd(ctypes.byref(qw), P, P, None, 1024, P, P, 16, 16.0, P, P, P, 0, P, 1 << 30, None) == binding.QL_EINVAL
    assert lib.qlora_dequant(None, P, P, None) == binding.QL_EINVAL
    assert lib.ql_act_quant_e4m3(P, 4, 24, P, P, P, None) == binding.QL_EINVAL


def test_stream_read_argument_errors(lib):
    """The measurement read refuses null or misaligned pointers and sizes that
    are not a positive multiple of 16, before any launch."""
    P = FAKE
    assert lib.ql_stream_read(None, 1024, P, None) == binding.QL_EINVAL
    assert lib.ql_stream_read(P, 1024, None, None) == binding.QL_EINVAL
    assert lib.ql_stream_read(P, 0, P, None) == binding.QL_EINVAL
    assert lib.ql_stream_read(P, 1000, P, None) == binding.QL_EINVAL
    assert lib.ql_stream_read(ctypes.c_void_p(P.value + 8), 1024, P, None) == binding.QL_EINVAL
    assert lib.ql_stream_read(P, 1024, ctypes.c_void_p(P.value + 2), None) == binding.QL_EINVAL


def test_size_limits_refused(lib):
    """Shapes whose 32-bit buffer offsets would overflow are refused before
    any launch: more than QL_MAX_FEATURES per side, or codes of 2 GiB or more
    (the one-byte formats reach it first)."""
    P = FAKE
    big = 524288
    assert lib.quant_pack(binding.FMT_NF4, P, 64, 2 * big, P, P, P, 256, None) == binding.QL_EUNSUPPORTED
    assert "features" in _err(lib)
    assert lib.quant_pack(binding.FMT_Q4_0, P, 2 * big, 64, P, P, P, 256, None) == binding.QL_EUNSUPPORTED
    # 65536 x 32768 one-byte codes = 2 GiB: refused; the 4-bit form (1 GiB) passes the size check
    assert lib.quant_pack(binding.FMT_Q8_0, P, 65536, 32768, P, P, P, 256, None) == binding.QL_EUNSUPPORTED
    assert "2 GiB" in _err(lib)
    assert lib.quant_pack(binding.FMT_Q4_0, P, 65536, 32768, P, P, P, 8, None) == binding.QL_EWORKSPACE
    qw = _qw(binding.FMT_FP8, 65536, 32768)
    assert lib.qlora_linear_fwd(ctypes.byref(qw), P, 16, P, P, 16, 16.0, P, P, None, 0, None) == binding.QL_EUNSUPPORTED
    qw = _qw(binding.FMT_NF4, 64, 2 * big)
    assert lib.qlora_linear_bwd(ctypes.byref(qw), P, P, P, 16, P, P, 16, 16.0, P, P, P, 0, P, 1 << 30,
                                None) == binding.QL_EUNSUPPORTED
    assert lib.qlora_dequant(ctypes.byref(qw), P, P, None) == binding.QL_EUNSUPPORTED
    # the largest accepted side
    assert lib.quant_pack(binding.FMT_NF4, P, 64, big, P, P, P, 8, None) == binding.QL_EWORKSPACE


def test_noalloc_backward_refuses_oversized_scratch(lib):
    """The allocation-free backward refuses, before touching a GPU, a shape
    whose scratch exceeds its fixed array (the FP8 base at 8192 tokens needs
    its activation split planes: 236 MB)."""
    P = FAKE
    need = binding.workspace_bytes(binding.OP_BWD, binding.FMT_FP8, 12288, 4096, 8192, 32)
    assert need > binding.NOALLOC_SCRATCH_BYTES
    qw = _qw(binding.FMT_FP8, 12288, 4096)
    rc = lib.qlora_linear_bwd_noalloc(ctypes.byref(qw), P, P, P, 8192, P, P, 32, 64.0, P, P, P, 0, None)
    assert rc == binding.QL_EUNSUPPORTED
    assert "scratch" in _err(lib)
    assert lib.qlora_linear_bwd_noalloc(None, P, P, P, 16, P, P, 16, 16.0, P, P, P, 0, None) == binding.QL_EINVAL


def test_pool_argument_errors(lib):
    h = ctypes.c_void_p()
    slots = (ctypes.c_void_p * 2)(0x10000, 0x10100)
    hosts = (ctypes.c_void_p * 3)(0x20000, 0x30000, 0x40000)
    sizes = (ctypes.c_size_t * 3)(100, 100, 5000)
    assert lib.ql_pool_create(ctypes.byref(h), 0, slots, 4096, 3, hosts, sizes) == binding.QL_EINVAL
    assert lib.ql_pool_create(ctypes.byref(h), 2, slots, 4096, 3, hosts, sizes) == binding.QL_EINVAL
    assert "exceeds slot size" in _err(lib)
    odd = (ctypes.c_void_p * 2)(0x10000, 0x10010)
    sizes_ok = (ctypes.c_size_t * 3)(100, 100, 100)
    assert lib.ql_pool_create(ctypes.byref(h), 2, odd, 4096, 3, hosts, sizes_ok) == binding.QL_EINVAL
    assert lib.layer_stream_prefetch(None, 0, None) == binding.QL_EINVAL
    assert lib.ql_pool_destroy(None) == binding.QL_OK


def test_adamw_argument_errors(lib):
    T = binding.AdamwTensorC
    hp = binding.AdamwHparamsC(1e-3, 0.9, 0.999, 1e-8, 0.0, 1.0, 1, 0)
    good = T(0x10000, 0x20000, 0x30000, 0x40000, None, 64)
    arr = (T * 1)(good)
    step = lib.ql_adamw_step
    assert step(arr, 33, ctypes.byref(hp), None) == binding.QL_EINVAL
    assert step(arr, -1, ctypes.byref(hp), None) == binding.QL_EINVAL
    assert step(arr, 1, None, None) == binding.QL_EINVAL
    assert step(None, 1, ctypes.byref(hp), None) == binding.QL_EINVAL
    for field, value in (("step", 0), ("reserved", 1), ("beta1", 1.0), ("beta2", -0.1), ("lr", -1e-3),
                         ("eps", float("nan")), ("weight_decay", float("inf"))):
        bad = binding.AdamwHparamsC(1e-3, 0.9, 0.999, 1e-8, 0.0, 1.0, 1, 0)
        setattr(bad, field, value)
        assert step(arr, 1, ctypes.byref(bad), None) == binding.QL_EINVAL, field
    for kw in ({"n": 6}, {"param": None}, {"grad": 0x20008}, {"param_bf16": 0x50004}):
        t = T(0x10000, 0x20000, 0x30000, 0x40000, None, 64)
        for k, v in kw.items():
            setattr(t, k, v)
        assert step((T * 1)(t), 1, ctypes.byref(hp), None) == binding.QL_EINVAL, kw


def test_plan_argument_errors(lib):
    P = FAKE
    qw = _qw()
    h = ctypes.c_void_p()
    assert lib.ql_plan_create(None) == binding.QL_EINVAL
    assert lib.ql_plan_create(ctypes.byref(h)) == binding.QL_OK
    try:
        add_f, add_b = lib.ql_plan_add_fwd, lib.ql_plan_add_bwd
        # the same checks as the direct calls, and nothing recorded on error
        assert add_f(h, ctypes.byref(qw), P, 16, P, P, 12, 16.0, P, P, None, 0) == binding.QL_EUNSUPPORTED
        assert add_f(h, ctypes.byref(qw), None, 16, P, P, 16, 16.0, P, P, None, 0) == binding.QL_EINVAL
        assert add_b(h, ctypes.byref(qw), P, P, P, 1024, P, P, 16, 16.0, P, P, P, 0, P, 0) == binding.QL_EWORKSPACE
        assert lib.ql_plan_size(h) == 0
        assert add_f(None, ctypes.byref(qw), P, 16, P, P, 16, 16.0, P, P, None, 0) == binding.QL_EINVAL
        assert lib.ql_plan_add_event(h, None) == binding.QL_EINVAL
        # valid calls are recorded (nothing is launched until run)
        assert add_f(h, ctypes.byref(qw), P, 0, P, P, 16, 16.0, P, P, None, 0) == binding.QL_OK
        ws = binding.workspace_bytes(binding.OP_BWD, qw.format, qw.n_out, qw.k_in, 16, 16)
        assert add_b(h, ctypes.byref(qw), P, P, P, 16, P, P, 16, 16.0, P, P, P, 0, P, ws) == binding.QL_OK
        assert lib.ql_plan_add_event(h, ctypes.c_void_p(0x1234)) == binding.QL_OK
        assert lib.ql_plan_size(h) == 3
        assert lib.ql_plan_run(None, None) == binding.QL_EINVAL
    finally:
        assert lib.ql_plan_destroy(h) == binding.QL_OK
    assert lib.ql_plan_size(None) == 0


def test_group_argument_errors(lib):
    """Grouped calls: validated like single calls, one base format, and no
    call may write a buffer another call of the group reads or writes."""
    m, r = 16, 16
    q1 = _qw(codes=0x100000, scales=0x110000)
    q2 = _qw(codes=0x120000, scales=0x130000)
    ws = binding.workspace_bytes(binding.OP_FWD, q1.format, q1.n_out, q1.k_in, m, r)

    def call(qw, base):   # every buffer of a call at its own address range
        return binding.FwdCallC(ctypes.addressof(qw), base, base + 0x10000, base + 0x20000, 16.0, 0,
                                base + 0x30000, base + 0x40000, base + 0x50000, ws)

    a = call(q1, 0x1000000)
    b = call(q2, 0x2000000)
    grp = lib.qlora_linear_fwd_group
    assert grp((binding.FwdCallC * 2)(a, b), 0, m, r, None) == binding.QL_EINVAL
    assert grp((binding.FwdCallC * 2)(a, b), 9, m, r, None) == binding.QL_EINVAL
    assert grp(None, 2, m, r, None) == binding.QL_EINVAL
    assert grp((binding.FwdCallC * 2)(a, b), 2, m, 12, None) == binding.QL_EUNSUPPORTED
    # call 1 writes its y onto call 0's input x
    bad = call(q2, 0x2000000)
    bad.y = a.x
    assert grp((binding.FwdCallC * 2)(a, bad), 2, m, r, None) == binding.QL_EINVAL
    assert "not independent" in _err(lib)
    # two calls sharing one workspace
    bad = call(q2, 0x2000000)
    bad.ws = a.ws
    assert grp((binding.FwdCallC * 2)(a, bad), 2, m, r, None) == binding.QL_EINVAL
    # mixed base formats
    q3 = _qw(fmt=binding.FMT_Q4_0, codes=0x140000, scales=0x150000)
    c = call(q3, 0x3000000)
    assert grp((binding.FwdCallC * 2)(a, c), 2, m, r, None) == binding.QL_EINVAL
    assert "formats" in _err(lib)
    # reading the same input is allowed (q, k and v share x): the plan records it
    shared = call(q2, 0x2000000)
    shared.x = a.x
    h = ctypes.c_void_p()
    assert lib.ql_plan_create(ctypes.byref(h)) == binding.QL_OK
    try:
        assert lib.ql_plan_add_fwd_group(h, (binding.FwdCallC * 2)(a, shared), 2, m, r) == binding.QL_OK
        assert lib.ql_plan_add_fwd_group(h, (binding.FwdCallC * 2)(a, bad), 2, m, r) == binding.QL_EINVAL
        assert lib.ql_plan_size(h) == 1
    finally:
        lib.ql_plan_destroy(h)


def test_stack_argument_errors(lib):
    A = binding.AdapterC
    ok = [A(0x10000, 0x20000, 8, 16.0), A(0x30000, 0x40000, 8, 16.0)]
    alpha = ctypes.c_float()
    st = lib.ql_stack_adapters
    P = FAKE
    assert st((A * 2)(*ok), 1, 64, 128, P, P, ctypes.byref(alpha), None) == binding.QL_EINVAL
    assert st((A * 2)(*ok), 9, 64, 128, P, P, ctypes.byref(alpha), None) == binding.QL_EINVAL
    assert st((A * 2)(*ok), 2, 64, 128, P, None, ctypes.byref(alpha), None) == binding.QL_EINVAL
    assert st((A * 2)(*ok), 2, 64, 128, P, P, None, None) == binding.QL_EINVAL
    assert st((A * 2)(ok[0], A(0x30000, 0x40000, 4, 16.0)), 2, 64, 128, P, P, ctypes.byref(alpha), None) \
        == binding.QL_EUNSUPPORTED
    assert st((A * 2)(ok[0], A(0x30000, 0x40008, 8, 16.0)), 2, 64, 128, P, P, ctypes.byref(alpha), None) \
        == binding.QL_EINVAL
    assert st((A * 2)(ok[0], A(0x30000, 0x40000, 8, -1.0)), 2, 64, 128, P, P, ctypes.byref(alpha), None) \
        == binding.QL_EINVAL
    assert st((A * 2)(ok[0], A(0x30000, 0x40000, 0, 16.0)), 2, 64, 128, P, P, ctypes.byref(alpha), None) \
        == binding.QL_EINVAL
