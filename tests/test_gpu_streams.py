"""Every call enqueues on the caller's stream: the same step run on the
default stream, on a side stream made current, and with an explicit
`stream=` argument gives bit-identical outputs and caches (the kernels
are deterministic), and work ordered on the side stream around the calls
sees their results."""
import numpy as np
import pytest
import torch

from gpu_helpers import DeviceInputs, dev
from synthetic import generate, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_273_amd as m

    return m


def _buffers(pkv, d):
    """Fresh copies of the caches and NaN-filled outputs, on the current stream."""
    inp = d.inp
    wl = inp.wl
    S = 64
    ms = pkv.max_splits_for(int(inp.context_lens.max()), S)
    f = dict(dtype=torch.float32, device=dev())
    return dict(k=d.k.clone(), v=d.v.clone(), ws=pkv.make_workspace(d.q[0], d.k),
                out_b=torch.full((wl.B, wl.Hq, wl.D), float("nan"), **f),
                out_s=torch.full((wl.B, wl.Hq, wl.D), float("nan"), **f),
                po=torch.empty((wl.B, wl.Hq, ms, wl.D), **f),
                pl=torch.empty((wl.B, wl.Hq, ms), **f), S=S)


def _launch(pkv, d, x, stream=None):
    """Fused append + balanced attention, then split 64 + reduce."""
    sc = float(d.inp.scale)
    pkv.paged_append_decode_attention_balanced(d.q[0], d.k_new, d.v_new, x["k"], x["v"], d.bt,
                                               d.cl, sc, workspace=x["ws"], out=x["out_b"],
                                               stream=stream)
    pkv.paged_decode_attention(d.q[0], x["k"], x["v"], d.bt, d.cl, sc, split_tokens=x["S"],
                               partial_out=x["po"], partial_lse=x["pl"], stream=stream)
    pkv.split_context_reduce(x["po"], x["pl"], d.cl, x["S"], out=x["out_s"], stream=stream)


def _host(x):
    return [x[n].cpu().numpy().view(np.uint8) for n in ("out_b", "out_s", "k", "v")]


@pytest.mark.parametrize("name", ["tiny_b4_hq8_hkv2_d64_bs16", "llama8b_b32_ctx4096_bs16"])
def test_side_stream_matches_default_stream(pkv, name):
    print(f"streams {name}", flush=True)
    inp = generate(make_workload(name))
    d = DeviceInputs(inp)
    side = torch.cuda.Stream()                     # default priority
    cur = torch.cuda.current_stream()
    ref = _buffers(pkv, d)
    _launch(pkv, d, ref)
    torch.cuda.synchronize()

    side.wait_stream(cur)
    with torch.cuda.stream(side):                  # the binding takes the current stream
        x_cur = _buffers(pkv, d)
        _launch(pkv, d, x_cur)
    x_exp = _buffers(pkv, d)                       # made on the default stream ...
    side.wait_stream(cur)                          # ... so the side stream waits for them
    _launch(pkv, d, x_exp, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    want = _host(ref)
    for x in (x_cur, x_exp):
        for a, b in zip(want, _host(x)):
            assert np.array_equal(a, b)
