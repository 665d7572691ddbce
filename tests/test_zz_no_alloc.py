"""la_prefill_noalloc (the prefill with its workspace in the library's static
device scratch) against la_prefill through the C ABI: the same kernels on the
same inputs, so the results agree bit for bit.  Two calls in a row, the
second smaller, for each rule; a call needing more than the scratch is
refused before anything runs."""
import pytest
import torch

import causal_linear_attention_attn_amd as la
from causal_linear_attention_attn_amd import _lib, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run_both(x, **kw):
    q, k, v = x["q"], x["k"], x["v"]
    ref = la.prefill(q, k, v, **kw)
    got = la.prefill(q, k, v, noalloc=True, **kw)
    torch.cuda.synchronize()
    return ref, got


def _same(ref, got):
    for a, b in zip(ref, got):
        if a is None:
            assert b is None
        else:
            assert torch.equal(a, b)


@pytest.mark.parametrize("rule", ["linear", "delta"])
def test_noalloc_matches_prefill_two_calls(rule):
    if rule == "linear":  # several segments: the scratch holds the scan slots
        w = inputs.WORKLOADS[4]
        shapes = [dict(H=32, N=32768), dict(H=4, N=5000)]
    else:  # the per-chunk records of the delta rule
        w = inputs.WORKLOADS[6]
        shapes = [dict(B=2, H=16, N=8192), dict(B=1, H=3, N=1000)]
    for i, shp in enumerate(shapes):
        x = inputs.make_prefill(w, DEV, **shp)
        kw = dict(gamma=x["gamma"], eps=w.eps) if rule == "linear" else \
            dict(rule="delta", g=x["g"], alpha=x["alpha"])
        need = la.workspace_size(x["q"], x["k"], x["v"], **kw)
        assert 0 < need <= _lib.NOALLOC_SCRATCH_BYTES, need
        ref, got = _run_both(x, **kw)
        print(f"[noalloc] {rule} call {i}: {shp} workspace {need} B", flush=True)
        _same(ref, got)


def test_noalloc_refuses_more_than_the_scratch():
    w = inputs.WORKLOADS[5]
    x = inputs.make_prefill(w, DEV, B=2, H=32, N=8192)  # about 200 MB of records
    need = la.workspace_size(x["q"], x["k"], x["v"], rule="delta", g=x["g"])
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    o = torch.full((2, 32, 8192, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(la.LinattnError) as e:
        la.prefill(x["q"], x["k"], x["v"], rule="delta", g=x["g"], o=o, noalloc=True)
    assert e.value.status == _lib.LA_ESCRATCH
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())  # nothing ran
    with pytest.raises(ValueError):
        la.prefill(x["q"], x["k"], x["v"], rule="delta", g=x["g"], noalloc=True,
                   workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
