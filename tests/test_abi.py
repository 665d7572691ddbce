"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, the ctypes structs match the C layout, and invalid
arguments are rejected before anything touches a device."""
import ctypes
import os
import re
import subprocess

import pytest

from causal_linear_attention_attn_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linattn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_lists_exactly_the_binding_exports():
    assert _declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (la_\w+)$", out, flags=re.M))
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    fields_p = [f for f, _ in _lib.PrefillArgs._fields_]
    fields_d = [f for f, _ in _lib.DecodeArgs._fields_]
    fields_b = [f for f, _ in _lib.BackwardArgs._fields_]
    fields_x = [f for f, _ in _lib.DeltaBackwardArgs._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "linattn.h"',
             "int main(void){"]
    lines.append('printf("%zu\\n", sizeof(la_prefill_args));')
    for f in fields_p:
        lines.append(f'printf("%zu\\n", offsetof(la_prefill_args, {f}));')
    lines.append('printf("%zu\\n", sizeof(la_decode_args));')
    for f in fields_d:
        lines.append(f'printf("%zu\\n", offsetof(la_decode_args, {f}));')
    lines.append('printf("%zu\\n", sizeof(la_backward_args));')
    for f in fields_b:
        lines.append(f'printf("%zu\\n", offsetof(la_backward_args, {f}));')
    lines.append('printf("%zu\\n", sizeof(la_delta_backward_args));')
    for f in fields_x:
        lines.append(f'printf("%zu\\n", offsetof(la_delta_backward_args, {f}));')
    lines.append("return 0;}")
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-I", os.path.dirname(HEADER),
                    str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True,
                                          text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(_lib.PrefillArgs)]
    want += [getattr(_lib.PrefillArgs, f).offset for f in fields_p]
    want += [ctypes.sizeof(_lib.DecodeArgs)]
    want += [getattr(_lib.DecodeArgs, f).offset for f in fields_d]
    want += [ctypes.sizeof(_lib.BackwardArgs)]
    want += [getattr(_lib.BackwardArgs, f).offset for f in fields_b]
    want += [ctypes.sizeof(_lib.DeltaBackwardArgs)]
    want += [getattr(_lib.DeltaBackwardArgs, f).offset for f in fields_x]
    assert got == want


def test_status_strings(lib):
    for s in range(6):
        assert lib.la_status_str(s) != b"unknown status"
    assert lib.la_status_str(99) == b"unknown status"
    assert lib.la_abi_version() == _lib.ABI_VERSION


def _args(**kw):
    a = _lib.PrefillArgs()
    a.B, a.H, a.N, a.d, a.dv = 1, 1, 4, 8, 8
    a.dtype, a.rule, a.fmap = _lib.LA_BF16, _lib.LA_RULE_LINEAR, _lib.LA_FMAP_ELU1
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    a.q = a.k = a.v = a.o = fake
    a.eps = 1e-6
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("bad", [
    dict(B=-1), dict(N=-2), dict(d=0), dict(dv=129), dict(d=200), dict(dtype=7),
    dict(rule=5), dict(fmap=3), dict(eps=-1.0), dict(eps=float("nan")),
    dict(eps=float("inf")), dict(q=None), dict(o=None),
    dict(g=ctypes.c_void_p(0x2000)),                       # gate on LINEAR
    dict(rule=_lib.LA_RULE_DELTA),                          # DELTA with elu1
    dict(rule=_lib.LA_RULE_DELTA, fmap=_lib.LA_FMAP_IDENTITY),  # DELTA, no g
    dict(rule=_lib.LA_RULE_DELTA, fmap=_lib.LA_FMAP_IDENTITY,
         g=ctypes.c_void_p(0x2000), z_out=ctypes.c_void_p(0x3000)),
    dict(rule=_lib.LA_RULE_DELTA, fmap=_lib.LA_FMAP_IDENTITY,
         g=ctypes.c_void_p(0x2000), gamma=ctypes.c_void_p(0x3000)),
    dict(alpha=ctypes.c_void_p(0x2000), gamma=ctypes.c_void_p(0x3000)),  # both decays
    dict(conv_weight=ctypes.c_void_p(0x2000), conv_width=0),  # conv width 1..4
    dict(conv_weight=ctypes.c_void_p(0x2000), conv_width=5),
    dict(conv_width=2),                                     # width without filters
    dict(conv_in=ctypes.c_void_p(0x2000)),                  # cache without filters
    dict(conv_out=ctypes.c_void_p(0x2000)),
    dict(conv_weight=ctypes.c_void_p(0x2000), conv_width=4,  # caches overlap partly
         conv_in=ctypes.c_void_p(0x4000), conv_out=ctypes.c_void_p(0x4002)),
])
def test_prefill_rejects_invalid_arguments(lib, bad):
    a = _args(**bad)
    assert lib.la_prefill(ctypes.byref(a), None) == _lib.LA_EINVAL


def test_prefill_null_args_and_unsupported_grid(lib):
    assert lib.la_prefill(None, None) == _lib.LA_EINVAL
    a = _args(B=70000, H=40000)  # B*H past the int32 range
    assert lib.la_prefill(ctypes.byref(a), None) == _lib.LA_EUNSUPPORTED
    # the delta rule's sequential pass: 512 threads per (head, 16 value
    # columns) along one grid axis of at most 2^32 - 1 work-items
    a = _args(B=1 << 21, H=1, dv=128, rule=_lib.LA_RULE_DELTA, fmap=_lib.LA_FMAP_IDENTITY,
              g=ctypes.c_void_p(0x2000))
    assert lib.la_prefill(ctypes.byref(a), None) == _lib.LA_EUNSUPPORTED
    fake = ctypes.c_void_p(0x2000)
    # fp32, d = dv = 128: convolution and per-channel decay exceed the LDS together
    a = _args(dtype=_lib.LA_F32, d=128, dv=128, alpha=fake, conv_weight=fake, conv_width=4)
    assert lib.la_prefill(ctypes.byref(a), None) == _lib.LA_EUNSUPPORTED
    assert lib.la_prefill_workspace_size(ctypes.byref(_args(d=0))) == \
        ctypes.c_size_t(-1).value


def test_delta_workspace_must_be_16_byte_aligned(lib):
    fake = ctypes.c_void_p(0x2000)
    a = _args(rule=_lib.LA_RULE_DELTA, fmap=_lib.LA_FMAP_IDENTITY, g=fake)
    need = lib.la_prefill_workspace_size(ctypes.byref(a))
    assert 0 < need < 1 << 30
    a.workspace, a.workspace_bytes = ctypes.c_void_p(0x4004), need
    assert lib.la_prefill(ctypes.byref(a), None) == _lib.LA_EINVAL
    a.workspace, a.workspace_bytes = ctypes.c_void_p(0x4000), need - 1
    assert lib.la_prefill(ctypes.byref(a), None) == _lib.LA_EWORKSPACE


def test_empty_inputs_are_noops(lib):
    for kw in (dict(B=0), dict(H=0)):
        a = _args(**kw)
        a.q = a.k = a.v = a.o = None
        assert lib.la_prefill(ctypes.byref(a), None) == _lib.LA_OK
        assert lib.la_prefill_workspace_size(ctypes.byref(a)) == 0


@pytest.mark.parametrize("bad", [
    dict(B=-1), dict(d=0), dict(dv=300), dict(dtype=2), dict(rule=9),
    dict(eps=-0.5), dict(S=None), dict(z=None),
    dict(rule=_lib.LA_RULE_DELTA),                          # elu1 + delta
    dict(rule=_lib.LA_RULE_DELTA, fmap=_lib.LA_FMAP_IDENTITY),  # z given, no g
    dict(alpha=ctypes.c_void_p(0x2000), gamma=ctypes.c_void_p(0x3000)),  # both decays
    dict(conv_weight=ctypes.c_void_p(0x2000), conv_width=0,
         conv_cache=ctypes.c_void_p(0x3000)),
    dict(conv_weight=ctypes.c_void_p(0x2000), conv_width=5,
         conv_cache=ctypes.c_void_p(0x3000)),
    dict(conv_weight=ctypes.c_void_p(0x2000), conv_width=3),   # no cache
    dict(conv_width=2), dict(conv_cache=ctypes.c_void_p(0x3000)),  # no filters
])
def test_decode_rejects_invalid_arguments(lib, bad):
    a = _lib.DecodeArgs()
    a.B, a.H, a.d, a.dv = 2, 2, 8, 8
    a.dtype, a.rule, a.fmap = _lib.LA_BF16, _lib.LA_RULE_LINEAR, _lib.LA_FMAP_ELU1
    fake = ctypes.c_void_p(0x1000)
    a.q = a.k = a.v = a.o = a.S = a.z = fake
    a.eps = 1e-6
    for k, v in bad.items():
        setattr(a, k, v)
    assert lib.la_decode_step(ctypes.byref(a), None) == _lib.LA_EINVAL


def test_decode_conv_on_delta_needs_its_cache(lib):
    a = _lib.DecodeArgs()
    a.B, a.H, a.d, a.dv = 2, 2, 8, 8
    a.dtype, a.rule, a.fmap = _lib.LA_BF16, _lib.LA_RULE_DELTA, _lib.LA_FMAP_IDENTITY
    fake = ctypes.c_void_p(0x1000)
    a.q = a.k = a.v = a.o = a.S = a.g = fake
    a.conv_weight, a.conv_width = fake, 4  # width 4 without a conv cache
    assert lib.la_decode_step(ctypes.byref(a), None) == _lib.LA_EINVAL


@pytest.mark.parametrize("dtype,esz", [(_lib.LA_BF16, 2), (_lib.LA_F32, 4)])
def test_delta_conv_workspace_holds_the_convolved_inputs(lib, dtype, esz):
    """Behind a convolution the delta rule runs on convolved copies of q, k
    and v at the start of the workspace, each region rounded up to 256
    bytes; the rule's own workspace follows."""
    fake = ctypes.c_void_p(0x2000)
    kw = dict(B=2, H=3, N=37, d=24, dv=40, dtype=dtype, rule=_lib.LA_RULE_DELTA,
              fmap=_lib.LA_FMAP_IDENTITY, g=fake)
    plain = lib.la_prefill_workspace_size(ctypes.byref(_args(**kw)))
    conv = lib.la_prefill_workspace_size(ctypes.byref(_args(conv_weight=fake, conv_width=3,
                                                            **kw)))
    r256 = lambda n: (n + 255) // 256 * 256
    rows = 2 * 3 * 37
    assert conv - plain == 2 * r256(rows * 24 * esz) + r256(rows * 40 * esz)


def _bargs(**kw):
    a = _lib.BackwardArgs()
    a.B, a.H, a.N, a.d, a.dv = 1, 2, 4, 8, 8
    a.dtype, a.fmap = _lib.LA_BF16, _lib.LA_FMAP_ELU1
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    a.q = a.k = a.v = a.o = a.den = a.grad_o = a.grad_q = a.grad_k = a.grad_v = fake
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("bad", [
    dict(B=-1), dict(N=-1), dict(d=0), dict(dv=129), dict(dtype=5), dict(fmap=7),
    dict(q=None), dict(den=None), dict(grad_o=None), dict(grad_v=None),
])
def test_backward_rejects_invalid_arguments(lib, bad):
    a = _bargs(**bad)
    assert lib.la_backward(ctypes.byref(a), None) == _lib.LA_EINVAL


def test_backward_per_channel_decay_arguments(lib):
    """alpha (GLA's decay) excludes gamma, needs grad_alpha, and fp32 takes
    it only up to d = 64; with alpha the workspace holds the per-token and
    per-chunk buffers even at one segment, and must be 16-byte aligned."""
    fake = ctypes.c_void_p(0x1000)
    a = _bargs(alpha=fake, grad_alpha=fake, gamma=fake)
    assert lib.la_backward(ctypes.byref(a), None) == _lib.LA_EINVAL
    a = _bargs(grad_alpha=fake)  # no alpha
    assert lib.la_backward(ctypes.byref(a), None) == _lib.LA_EINVAL
    a = _bargs(alpha=fake)  # no grad_alpha with tokens
    assert lib.la_backward(ctypes.byref(a), None) == _lib.LA_EINVAL
    a = _bargs(dtype=_lib.LA_F32, d=128, dv=16, alpha=fake, grad_alpha=fake)
    assert lib.la_backward(ctypes.byref(a), None) == _lib.LA_EUNSUPPORTED
    assert lib.la_backward_workspace_size(ctypes.byref(a)) == ctypes.c_size_t(-1).value
    a = _bargs(alpha=fake, grad_alpha=fake)
    n = lib.la_backward_workspace_size(ctypes.byref(a))
    r256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    B, H, N, d, dv = 1, 2, 4, 8, 8
    nch = (N + 31) // 32
    assert n == r256(B * H * N * d * 4) + r256(B * H * nch * (d * dv + 2 * d) * 4)
    assert lib.la_backward(ctypes.byref(a), None) == _lib.LA_EWORKSPACE
    a.workspace, a.workspace_bytes = ctypes.c_void_p(0x1004), n
    assert lib.la_backward(ctypes.byref(a), None) == _lib.LA_EINVAL


def test_backward_unsupported_and_sizes(lib):
    assert lib.la_backward(None, None) == _lib.LA_EINVAL
    # fp32 with d and dv above 64 runs over two value halves: it needs a
    # workspace even with one segment (the halves' buffers)
    a = _bargs(dtype=_lib.LA_F32, d=128, dv=100)
    assert 0 < lib.la_backward_workspace_size(ctypes.byref(a)) < ctypes.c_size_t(-1).value
    assert lib.la_backward(ctypes.byref(a), None) == _lib.LA_EWORKSPACE
    a = _bargs(dtype=_lib.LA_F32, d=128, dv=64)  # one pass: no workspace at one segment
    assert lib.la_backward_workspace_size(ctypes.byref(a)) == 0
    a = _bargs(B=70000, H=40000)  # B*H past the int32 range
    assert lib.la_backward(ctypes.byref(a), None) == _lib.LA_EUNSUPPORTED
    a = _bargs(B=0)
    assert lib.la_backward(ctypes.byref(a), None) == _lib.LA_OK
    assert lib.la_backward_workspace_size(ctypes.byref(a)) == 0


def test_backward_workspace_halves_with_forward_workspace(lib):
    """With the forward's workspace given, only the adjoint slots are needed:
    one forward workspace's worth, half of what recomputing the states takes."""
    a = _bargs(B=4, H=16, N=4096, d=64, dv=64)
    own = lib.la_backward_workspace_size(ctypes.byref(a))
    f = _args(B=4, H=16, N=4096, d=64, dv=64)
    fwd = lib.la_prefill_workspace_size(ctypes.byref(f))
    assert fwd > 0 and own == 2 * fwd
    a.fwd_workspace = ctypes.c_void_p(0x10000)
    assert lib.la_backward_workspace_size(ctypes.byref(a)) == fwd


def test_prefill_den_out_only_for_linear(lib):
    a = _args(rule=_lib.LA_RULE_DELTA, fmap=_lib.LA_FMAP_IDENTITY, g=ctypes.c_void_p(0x2000),
              den_out=ctypes.c_void_p(0x3000))
    assert lib.la_prefill(ctypes.byref(a), None) == _lib.LA_EINVAL
    # with GLA's per-channel decay too (the backward takes alpha): a valid size
    a = _args(den_out=ctypes.c_void_p(0x3000), alpha=ctypes.c_void_p(0x2000))
    assert lib.la_prefill_workspace_size(ctypes.byref(a)) != ctypes.c_size_t(-1).value


@pytest.mark.parametrize("dtype,esz", [(_lib.LA_BF16, 2), (_lib.LA_F32, 4)])
def test_training_forward_with_conv_keeps_the_convolved_inputs(lib, dtype, esz):
    """With denominators and a convolution the prefill convolves into copies
    of q, k, v at the start of its workspace, ahead of the plain rule's."""
    fake = ctypes.c_void_p(0x2000)
    kw = dict(B=2, H=3, N=4100, d=64, dv=40, dtype=dtype)
    plain = lib.la_prefill_workspace_size(ctypes.byref(_args(den_out=fake, **kw)))
    conv = lib.la_prefill_workspace_size(ctypes.byref(_args(den_out=fake, conv_weight=fake,
                                                            conv_width=4, **kw)))
    r256 = lambda n: (n + 255) // 256 * 256
    rows = 2 * 3 * 4100
    assert conv - plain == 2 * r256(rows * 64 * esz) + r256(rows * 40 * esz)


@pytest.mark.parametrize("maker", ["_bargs", "_xargs"])
def test_backward_conv_fields_validated(lib, maker):
    fake = ctypes.c_void_p(0x2000)
    mk = globals()[maker]
    entry = lib.la_backward if maker == "_bargs" else lib.la_delta_backward
    size = lib.la_backward_workspace_size if maker == "_bargs" else \
        lib.la_delta_backward_workspace_size
    for bad in (dict(conv_weight=fake, conv_width=4),                     # no dW output
                dict(conv_weight=fake, conv_width=5, grad_conv_weight=fake),
                dict(conv_width=2), dict(conv_in=fake), dict(grad_conv_out=fake),
                dict(grad_conv_weight=fake), dict(grad_conv_in=fake)):
        a = mk(**bad)
        assert entry(ctypes.byref(a), None) == _lib.LA_EINVAL, bad
        assert size(ctypes.byref(a)) == ctypes.c_size_t(-1).value, bad
    a = mk(N=300)
    plain = size(ctypes.byref(a))
    a = mk(N=300, conv_weight=fake, conv_width=3, grad_conv_weight=fake)
    assert size(ctypes.byref(a)) > plain


def test_state_init_rejects_invalid_arguments(lib):
    assert lib.la_state_init(None, None, 1, 1, 8, 8, None) == _lib.LA_EINVAL
    assert lib.la_state_init(ctypes.c_void_p(0x1000), None, 1, 1, 0, 8, None) == \
        _lib.LA_EINVAL
    assert lib.la_state_init(None, None, 0, 4, 8, 8, None) == _lib.LA_OK


def _xargs(**kw):
    a = _lib.DeltaBackwardArgs()
    a.B, a.H, a.N, a.d, a.dv = 1, 2, 4, 8, 8
    a.dtype = _lib.LA_BF16
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    a.q = a.k = a.v = a.g = a.grad_o = a.grad_q = a.grad_k = a.grad_v = a.grad_g = fake
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("bad", [
    dict(B=-1), dict(N=-1), dict(d=0), dict(dv=129), dict(dtype=5),
    dict(q=None), dict(g=None), dict(grad_o=None), dict(grad_g=None),
    dict(alpha=ctypes.c_void_p(0x2000)),        # decay without its gradient
    dict(grad_alpha=ctypes.c_void_p(0x2000)),   # gradient without a decay
])
def test_delta_backward_rejects_invalid_arguments(lib, bad):
    a = _xargs(**bad)
    assert lib.la_delta_backward(ctypes.byref(a), None) == _lib.LA_EINVAL


def test_delta_backward_unsupported_and_workspace(lib):
    assert lib.la_delta_backward(None, None) == _lib.LA_EINVAL
    a = _xargs(dtype=_lib.LA_F32)  # bf16 only
    assert lib.la_delta_backward(ctypes.byref(a), None) == _lib.LA_EUNSUPPORTED
    assert lib.la_delta_backward_workspace_size(ctypes.byref(a)) == ctypes.c_size_t(-1).value
    a = _xargs(B=70000, H=40000)
    assert lib.la_delta_backward(ctypes.byref(a), None) == _lib.LA_EUNSUPPORTED
    a = _xargs()
    need = lib.la_delta_backward_workspace_size(ctypes.byref(a))
    assert 0 < need < 1 << 30
    assert lib.la_delta_backward(ctypes.byref(a), None) == _lib.LA_EWORKSPACE
    a.workspace, a.workspace_bytes = ctypes.c_void_p(0x4004), need
    assert lib.la_delta_backward(ctypes.byref(a), None) == _lib.LA_EINVAL
    a = _xargs(B=0)
    assert lib.la_delta_backward(ctypes.byref(a), None) == _lib.LA_OK
    assert lib.la_delta_backward_workspace_size(ctypes.byref(a)) == 0
