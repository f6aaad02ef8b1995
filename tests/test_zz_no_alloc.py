"""paged_decode_attention_balanced_noalloc -- the balanced decode whose
workspace is the library's static per-GPU scratch array (for callers that
cannot allocate) -- against paged_decode_attention_balanced with a
caller-owned workspace: two calls in a row, the second with a smaller batch,
in bf16 and fp8; both entry points run the same kernels, so their outputs
agree bit for bit, and both agree with the oracle within the tolerance."""
import numpy as np
import pytest
import torch

from gpu_helpers import DeviceInputs, assert_close, dev, fp8_group, host_appended
from synthetic import generate, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_273_amd as m

    return m


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_noalloc_matches_workspace_entry(orc, pkv, kv):
    shapes = [dict(B=16, ctx_uniform=(1, 6000), max_blocks=188, seed=273501),
              dict(B=5, ctx_uniform=(1, 900), max_blocks=29, seed=273502)]
    for i, shape in enumerate(shapes):
        print(f"no-alloc call {i} ({kv}): B={shape['B']}", flush=True)
        inp = generate(make_workload("llama70b_b64_ragged1k_16k_bs32", **shape))
        wl = inp.wl
        if kv == "fp8":
            kc, vc, ks, vs = fp8_group(orc, inp)
            kp, vp = host_appended(orc, inp, kv_dtype="fp8", k_pool=kc, v_pool=vc, ks=ks,
                                   vs=vs)
            d = DeviceInputs(inp, k_pool=kp, v_pool=vp, k_scale=ks, v_scale=vs)
        else:
            ks = vs = None
            kp, vp = host_appended(orc, inp)
            d = DeviceInputs(inp, k_pool=kp, v_pool=vp)
        sc = float(inp.scale)
        ws = pkv.make_workspace(d.q[0], d.k)
        lse_ws = torch.empty((wl.B, wl.Hq), dtype=torch.float32, device=dev())
        out_ws = pkv.paged_decode_attention_balanced(d.q[0], d.k, d.v, d.bt, d.cl, sc,
                                                     workspace=ws, lse_out=lse_ws,
                                                     k_scale=d.ks, v_scale=d.vs)
        out = torch.full((wl.B, wl.Hq, wl.D), float("nan"), device=dev())
        lse = torch.full((wl.B, wl.Hq), float("nan"), device=dev())
        pkv.paged_decode_attention_balanced_noalloc(d.q[0], d.k, d.v, d.bt, d.cl, sc, out=out,
                                                    lse_out=lse, k_scale=d.ks, v_scale=d.vs)
        torch.cuda.synchronize()
        assert torch.equal(out, out_ws) and torch.equal(lse, lse_ws), f"call {i}"
        ref, rlse = orc.paged_attention(inp.query[0], kp, vp, inp.block_tables,
                                        inp.context_lens, inp.scale, block_size=wl.block_size,
                                        Hkv=wl.Hkv, kv_dtype=kv, k_scale=ks, v_scale=vs)
        assert_close(out, ref, f"no-alloc call {i}")
        assert_close(lse, rlse, f"no-alloc call {i} lse")


def test_noalloc_rejects_a_workspace_beyond_its_array(pkv):
    """int8 caches with 16 query heads per kv head need more than the
    static array holds on a full device: a clear error, nothing launched."""
    need = pkv.paged_decode_workspace_size(32, 2, 128, 16, pkv.PKV_INT8)
    q = torch.zeros((1, 32, 128), dtype=torch.int16, device=dev())
    k = torch.zeros((4, 16, 2, 128), dtype=torch.uint8, device=dev())
    sc = torch.ones((4, 2, 2), dtype=torch.float32, device=dev())
    bt = torch.zeros((1, 1), dtype=torch.int32, device=dev())
    cl = torch.ones((1,), dtype=torch.int32, device=dev())
    out = torch.empty((1, 32, 128), dtype=torch.float32, device=dev())
    if need <= 18 << 20:
        pytest.skip(f"this device needs only {need} bytes for that shape")
    with pytest.raises(pkv.PagedKVError, match="unsupported"):
        pkv.paged_decode_attention_balanced_noalloc(q, k, k.clone(), bt, cl, 0.1, out=out,
                                                    k_scale=sc, v_scale=sc.clone(),
                                                    kv_dtype="int8")
