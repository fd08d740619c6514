"""Host-side checks of libgdn.so that need no GPU: every symbol include/gdn.h declares is
exported, and every validation error path returns its status code before any HIP call."""

import ctypes
import os
import re

import pytest
import torch

import gated_deltanet_linear_amd as gdn
from gated_deltanet_linear_amd import GdnShape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.library_path()):
        pytest.fail("libgdn.so not built: run __graft_entry__.build() first")
    return gdn._load()


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "gdn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_symbols()
    assert {"gdn_prepare", "gdn_chunk_forward", "gdn_recurrent_step"} <= set(names)
    raw = ctypes.CDLL(gdn.library_path())
    for name in names:
        assert hasattr(raw, name), f"libgdn.so does not export {name}"


def test_version_and_status_strings(lib):
    hdr = open(os.path.join(ROOT, "include", "gdn.h")).read()
    declared = int(re.search(r"#define GDN_ABI_VERSION (\d+)", hdr).group(1))
    assert lib.gdn_abi_version() == declared == gdn.ABI_VERSION
    for code in range(6):
        assert lib.gdn_status_string(code).startswith(b"GDN_")


def _shape(**kw):
    base = dict(num_seqs=2, total_tokens=300, num_qk_heads=16, num_v_heads=32, head_dim_k=128,
                head_dim_v=128, qkv_dtype=1, out_dtype=1, in_dtype=1, scale=1.0)
    base.update(kw)
    return GdnShape(**base)


def test_workspace_size_formula(lib):
    s = _shape()
    expect = (2 + 300 // 64) * 32 * 20992
    assert lib.gdn_chunk_forward_workspace_size(ctypes.byref(s)) == expect
    assert lib.gdn_chunk_forward_workspace_size(ctypes.byref(_shape(num_v_heads=33))) == 0
    assert lib.gdn_chunk_forward_workspace_size(None) == 0


FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: calls below fail validation first


def _chunk(lib, s, ws_bytes=1 << 40, q=FAKE, ws=FAKE, cu=FAKE, v=FAKE, o=FAKE, k=FAKE):
    return lib.gdn_chunk_forward(ctypes.byref(s) if s is not None else None, cu, q, k, v,
                                 FAKE, FAKE, None, o, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(num_v_heads=33), INVALID),
    (dict(num_seqs=0), INVALID),
    (dict(total_tokens=-1), INVALID),
    (dict(qkv_dtype=7), INVALID),
    (dict(out_dtype=-1), INVALID),
    (dict(head_dim_k=0), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(head_dim_k=96, head_dim_v=96), UNSUPPORTED),
    (dict(head_dim_k=128, head_dim_v=64), UNSUPPORTED),
    (dict(total_tokens=1 << 30, num_v_heads=64, num_qk_heads=16), UNSUPPORTED),
])
def test_chunk_forward_rejects_bad_shapes(lib, kw, code):
    assert _chunk(lib, _shape(**kw)) == code


def test_chunk_forward_rejects_bad_pointers_and_workspace(lib):
    s = _shape()
    assert _chunk(lib, None) == INVALID
    assert _chunk(lib, s, cu=None) == INVALID
    assert _chunk(lib, s, q=None) == INVALID
    for name in ("q", "k", "v", "o"):  # 16-byte row accesses
        for off in (2, 8):
            assert _chunk(lib, s, **{name: ctypes.c_void_p((1 << 20) + off)}) == INVALID, name
    assert _chunk(lib, s, ws=ctypes.c_void_p((1 << 20) + 64)) == INVALID  # ws not 256-aligned
    need = lib.gdn_chunk_forward_workspace_size(ctypes.byref(s))
    assert _chunk(lib, s, ws_bytes=need - 1) == WS_SMALL
    assert lib.gdn_chunk_intra(ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 40,
                               None) == INVALID
    assert lib.gdn_chunk_scan(ctypes.byref(s), FAKE, FAKE, FAKE, None, None, FAKE, None, FAKE,
                              1 << 40, None) == INVALID
    assert lib.gdn_chunk_scan(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE,
                              need - 1, None) == WS_SMALL
    mis = ctypes.c_void_p((1 << 20) + 8)
    assert lib.gdn_chunk_scan(ctypes.byref(s), FAKE, FAKE, FAKE, mis, None, FAKE, None, FAKE,
                              1 << 40, None) == INVALID  # v
    assert lib.gdn_chunk_scan(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, mis, None, FAKE,
                              1 << 40, None) == INVALID  # o


def test_split_qkv_dtype_only_on_the_prefill_calls(lib):
    """GDN_DTYPE_F32_SPLIT (2) passes the chunked-prefill calls' validation (they get as far as
    the workspace check) and the workspace size, and is refused by the decode step and the
    backward."""
    s = _shape(qkv_dtype=2)
    need = lib.gdn_chunk_forward_workspace_size(ctypes.byref(s))
    assert need == lib.gdn_chunk_forward_workspace_size(ctypes.byref(_shape())) > 0
    assert _chunk(lib, s, ws_bytes=need - 1) == WS_SMALL
    assert lib.gdn_chunk_intra(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1,
                               None) == WS_SMALL
    assert lib.gdn_chunk_scan(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE,
                              need - 1, None) == WS_SMALL
    assert _chunk(lib, _shape(qkv_dtype=3), ws_bytes=need - 1) == INVALID
    s2 = _shape(total_tokens=2, qkv_dtype=2)
    assert lib.gdn_recurrent_step(ctypes.byref(s2), *([FAKE] * 7), None) == INVALID
    assert lib.gdn_chunk_backward_workspace_size(ctypes.byref(s)) == 0
    with pytest.raises(gdn.GdnError):  # the binding takes split_f32 for float32 q/k/v only
        gdn._shape(1, 4, 1, 1, 32, 32, torch.bfloat16, torch.bfloat16, split_f32=True)
    assert gdn._shape(1, 4, 1, 1, 32, 32, torch.float32, torch.float32,
                      split_f32=True).qkv_dtype == 2


def test_recurrent_step_validation(lib):
    s = _shape(total_tokens=2)
    args = [FAKE] * 7
    assert lib.gdn_recurrent_step(ctypes.byref(_shape(total_tokens=3)), *args, None) == INVALID
    for i in range(7):
        a = list(args)
        a[i] = None
        assert lib.gdn_recurrent_step(ctypes.byref(s), *a, None) == INVALID
    a = list(args)
    a[5] = ctypes.c_void_p((1 << 20) + 4)  # state must be 16-byte aligned
    assert lib.gdn_recurrent_step(ctypes.byref(s), *a, None) == INVALID
    assert lib.gdn_recurrent_step(ctypes.byref(_shape(total_tokens=2, state_dtype=7)), *args,
                                  None) == INVALID
    assert lib.gdn_recurrent_step(ctypes.byref(_shape(total_tokens=2, head_dim_k=48,
                                                      head_dim_v=48)), *args, None) == UNSUPPORTED


def test_prepare_validation(lib):
    s = _shape()
    good = [FAKE] * 8  # cu, x, w, bias, a, b, A_log, dt_bias
    outs = [FAKE] * 5

    def call(shape, ins, eps, o):
        return lib.gdn_prepare(ctypes.byref(shape), *ins, eps, *o, None)

    assert call(_shape(in_dtype=5), good, 1e-6, outs) == INVALID
    assert call(s, good, -1.0, outs) == INVALID
    assert call(s, good, float("nan"), outs) == INVALID
    for i in (0, 1, 2, 4, 5, 6, 7):  # every input except the optional bias
        ins = list(good)
        ins[i] = None
        assert call(s, ins, 1e-6, outs) == INVALID
    for i in range(5):
        o = list(outs)
        o[i] = None
        assert call(s, good, 1e-6, o) == INVALID
    for i in (1, 3):  # mixed_qkv and the conv bias must be 16-byte aligned
        ins = list(good)
        ins[i] = ctypes.c_void_p((1 << 20) + 8)
        assert call(s, ins, 1e-6, outs) == INVALID
    for i in (4, 5):  # a, b
        ins = list(good)
        ins[i] = ctypes.c_void_p((1 << 20) + 4)
        assert call(s, ins, 1e-6, outs) == INVALID
    for i in (3, 4):  # g, beta
        o = list(outs)
        o[i] = ctypes.c_void_p((1 << 20) + 4)
        assert call(s, good, 1e-6, o) == INVALID
    assert call(_shape(head_dim_k=16, head_dim_v=16), good, 1e-6, outs) == UNSUPPORTED


def test_decode_prepare_validation(lib):
    # one token per sequence
    s = _shape(num_seqs=4, total_tokens=4)
    ins = [FAKE] * 8  # x, window, w, bias, a, b, A_log, dt_bias
    outs = [FAKE] * 5  # q, k, v, g, beta

    def call(shape, ins, eps, outs):
        return lib.gdn_decode_prepare(ctypes.byref(shape), *ins, eps, *outs, None)

    assert call(_shape(num_seqs=4, total_tokens=5), ins, 1e-6, outs) == INVALID
    assert call(s, ins, -1.0, outs) == INVALID
    for i in (0, 1, 2, 4, 5, 6, 7):  # every input except the optional bias
        bad = list(ins)
        bad[i] = None
        assert call(s, bad, 1e-6, outs) == INVALID
    for i in range(5):
        o = list(outs)
        o[i] = None
        assert call(s, ins, 1e-6, o) == INVALID
    for i in (0, 1, 2, 3):  # x, window, taps, bias must be 16-byte aligned
        bad = list(ins)
        bad[i] = ctypes.c_void_p((1 << 20) + 8)
        assert call(s, bad, 1e-6, outs) == INVALID
    assert call(_shape(num_seqs=4, total_tokens=4, head_dim_k=16, head_dim_v=16), ins, 1e-6,
                outs) == UNSUPPORTED


def test_decode_step_validation(lib):
    s = _shape(num_seqs=4, total_tokens=4)
    ins = [FAKE] * 8  # x, window, w, bias, a, b, A_log, dt_bias

    def call(shape, ins, eps=1e-6, state=FAKE, o=FAKE):
        return lib.gdn_decode_step(ctypes.byref(shape), *ins, eps, state, o, None)

    assert call(_shape(num_seqs=4, total_tokens=5), ins) == INVALID
    assert call(s, ins, eps=-1.0) == INVALID
    for i in (0, 1, 2, 4, 5, 6, 7):  # every input except the optional bias
        bad = list(ins)
        bad[i] = None
        assert call(s, bad) == INVALID
    assert call(s, ins, state=None) == INVALID
    assert call(s, ins, o=None) == INVALID
    for i in (0, 1, 2, 3):  # x, window, taps, bias must be 16-byte aligned
        bad = list(ins)
        bad[i] = ctypes.c_void_p((1 << 20) + 8)
        assert call(s, bad) == INVALID
    assert call(s, ins, state=ctypes.c_void_p((1 << 20) + 4)) == INVALID
    assert call(_shape(num_seqs=4, total_tokens=4, head_dim_k=64, head_dim_v=128), ins) \
        == UNSUPPORTED
    assert call(_shape(num_seqs=4, total_tokens=4, head_dim_k=16, head_dim_v=16), ins) \
        == UNSUPPORTED
    # G = 128 V heads per QK head: q, k and 128 v rows of 128 floats exceed the 64 KiB of LDS
    assert call(_shape(num_seqs=4, total_tokens=4, num_qk_heads=1, num_v_heads=128), ins) \
        == UNSUPPORTED


def test_chunk_backward_validation(lib):
    s = _shape()
    ins = [FAKE] * 10  # cu, q, k, v, g, beta, h0, dout, dht  (+ placeholder)
    outs = [FAKE] * 6  # dq, dk, dv, dg, dbeta, dh0
    need = lib.gdn_chunk_backward_workspace_size(ctypes.byref(s))
    assert need > 0

    def call(shape, ins=ins[:9], outs=outs, ws=FAKE, nbytes=need):
        return lib.gdn_chunk_backward(ctypes.byref(shape), *ins, *outs, ws, nbytes, None)

    assert call(s, nbytes=need - 1) == WS_SMALL
    assert call(s, ws=ctypes.c_void_p((1 << 20) + 64)) == INVALID
    for i in (0, 1, 2, 3, 4, 5, 7):  # all but the optional initial state and dht
        bad = list(ins[:9])
        bad[i] = None
        assert call(s, ins=bad) == INVALID
    for i in range(5):  # all but the optional dh0
        o = list(outs)
        o[i] = None
        assert call(s, outs=o) == INVALID
    mis = ctypes.c_void_p((1 << 20) + 8)
    for i in (1, 2, 3, 7):  # q, k, v, dout: 16-byte row accesses
        bad = list(ins[:9])
        bad[i] = mis
        assert call(s, ins=bad) == INVALID, i
    for i in (0, 1, 2):  # dq, dk, dv
        o = list(outs)
        o[i] = mis
        assert call(s, outs=o) == INVALID, i
    assert call(_shape(state_dtype=3)) == INVALID
    assert call(_shape(head_dim_k=48, head_dim_v=48)) == UNSUPPORTED


def test_gated_rmsnorm_validation(lib):
    s = _shape()

    def call(shape, o=FAKE, z=FAKE, w=None, off=0.0, eps=1e-6, out=FAKE):
        return lib.gdn_gated_rmsnorm(ctypes.byref(shape), o, z, w, off, eps, out, None)

    assert call(s, o=None) == INVALID
    assert call(s, z=None) == INVALID
    assert call(s, out=None) == INVALID
    assert call(s, eps=-1.0) == INVALID
    assert call(s, off=float("nan")) == INVALID
    assert call(s, z=ctypes.c_void_p((1 << 20) + 4)) == INVALID
    assert call(s, w=ctypes.cast(ctypes.c_void_p((1 << 20) + 8), ctypes.POINTER(ctypes.c_float))) \
        == INVALID
    assert call(_shape(in_dtype=9)) == INVALID
    assert call(_shape(head_dim_k=48, head_dim_v=48)) == UNSUPPORTED


def test_python_binding_refuses_cpu_tensors():
    import torch

    x = torch.zeros(4, 1, 32)
    g = torch.zeros(4, 1)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(gdn.GdnError):
        gdn.chunk_forward(x, x, x, g, g, cu)
    with pytest.raises(gdn.GdnError):
        gdn.recurrent_step(x, x, x, g, g, torch.zeros(4, 1, 32, 32))


def test_chunk_forward_noalloc_validation(lib):
    """The no-allocation entry point validates like gdn_chunk_forward and refuses a shape whose
    workspace exceeds its device array before any HIP call."""
    def call(shape, q=FAKE, v=FAKE, o=FAKE, cu=FAKE):
        return lib.gdn_chunk_forward_noalloc(ctypes.byref(shape) if shape is not None else None,
                                             cu, q, FAKE, v, FAKE, FAKE, None, o, None, None)

    assert call(None) == INVALID
    assert call(_shape(num_v_heads=33)) == INVALID
    assert call(_shape(head_dim_k=96, head_dim_v=96)) == UNSUPPORTED
    # 64 MiB holds 3196 records of 20992 bytes: 1 x 4096 tokens at 32 V heads is 65 x 32 = 2080
    limit = 64 << 20
    big = _shape(num_seqs=1, total_tokens=8192)  # 129 slots x 32 heads x 20992 > 64 MiB
    assert lib.gdn_chunk_forward_workspace_size(ctypes.byref(big)) > limit
    assert call(big) == 5  # GDN_ERR_SCRATCH_LIMIT
    assert b"SCRATCH_LIMIT" in lib.gdn_status_string(5)
    ok = _shape(num_seqs=1, total_tokens=4096)
    assert lib.gdn_chunk_forward_workspace_size(ctypes.byref(ok)) <= limit
    assert call(ok, cu=None) == INVALID
    assert call(ok, q=None) == INVALID
    assert call(ok, v=ctypes.c_void_p((1 << 20) + 8)) == INVALID
    assert call(ok, o=ctypes.c_void_p((1 << 20) + 8)) == INVALID


def test_gated_decode_validation(lib):
    """gdn_recurrent_step_gated and gdn_decode_step_gated: the step's checks plus the gate's (z
    given, 16-byte aligned z and weight, eps >= 0, a finite offset, a valid in_dtype)."""
    s = _shape(num_seqs=4, total_tokens=4)
    mis = ctypes.c_void_p((1 << 20) + 8)

    def rstep(shape, z=FAKE, w=None, off=1.0, eps=1e-6, out=FAKE, state=FAKE):
        return lib.gdn_recurrent_step_gated(ctypes.byref(shape), FAKE, FAKE, FAKE, FAKE, FAKE,
                                            state, z, w, off, eps, out, None)

    def dstep(shape, z=FAKE, w=None, off=1.0, eps=1e-6, out=FAKE):
        return lib.gdn_decode_step_gated(ctypes.byref(shape), *([FAKE] * 8), 1e-6, FAKE, z, w,
                                         off, eps, out, None)

    for call in (rstep, dstep):
        assert call(_shape(num_seqs=4, total_tokens=5)) == INVALID
        assert call(s, z=None) == INVALID
        assert call(s, out=None) == INVALID
        assert call(s, z=mis) == INVALID
        assert call(s, w=mis) == INVALID
        assert call(s, eps=-1.0) == INVALID
        assert call(s, eps=float("nan")) == INVALID
        assert call(s, off=float("nan")) == INVALID
        assert call(_shape(num_seqs=4, total_tokens=4, in_dtype=9)) == INVALID
        assert call(_shape(num_seqs=4, total_tokens=4, head_dim_k=48, head_dim_v=48)) \
            == UNSUPPORTED
    assert rstep(s, state=ctypes.c_void_p((1 << 20) + 4)) == INVALID
    # G = 64 V heads per QK head: q, k, 64 v and 64 z rows and the factors exceed 64 KiB of LDS
    assert dstep(_shape(num_seqs=4, total_tokens=4, num_qk_heads=1, num_v_heads=64)) \
        == UNSUPPORTED
