"""GPU parity of the fused decode step: paged_append_decode_attention and
paged_append_decode_attention_balanced (append + attention in one launch).

The step they compute is [B] "What the KV Cache Stores and Why": store the
new token's K and V, then attend the new query over every cached token,
the new one included.  Against the oracle (append, then attention):
  * the caches after the call equal the oracle's appended pools byte for
    byte (every format: bf16, fp8 per block / per head / per tensor, int8
    symmetric and asymmetric);
  * outputs and lse within the attention tolerance, on every schedule
    (single pass, fixed splits + split_context_reduce, balanced) and on the
    edge context lengths of every supported shape.
The synthetic pools hold NaN at each sequence's slot T - 1 until it is
appended, so a read of that slot before its write shows up as NaN.
At the full workload sizes the fused call is compared with the separate
append + attention calls, which the full-size tests compare with the
oracle: outputs bit for bit, caches byte for byte.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_close, dev, fp8_group, tables_to_dev, to_dev
from synthetic import generate, make_workload

pytestmark = pytest.mark.gpu
TINY = "tiny_b4_hq8_hkv2_d64_bs16"
KINDS = ["bf16", "fp8", "fp8_head", "fp8_tensor", "int8", "int8_sym"]
EDGE_CTX = (1, 2, 15, 16, 17, 31, 32, 33, 47, 63, 64, 65, 100, 255, 300)


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_273_amd as m

    return m


def _dtype(kind):
    return "int8" if kind.startswith("int8") else kind


def _caches(orc, inp, kind):
    """Host cache arrays (codes) and scales of group 0 in format `kind`."""
    wl = inp.wl
    if kind == "bf16":
        return inp.k_pool[0], inp.v_pool[0], None, None
    if kind == "fp8":
        return fp8_group(orc, inp)
    sc = []
    for src in (inp.k_pool[0], inp.v_pool[0]):
        if kind.startswith("int8"):
            sc.append(orc.int8_block_params(src, inp.block_tables, inp.context_lens,
                                            wl.block_size, symmetric=(kind == "int8_sym")))
        else:
            sc.append(orc.fp8_wide_scales(src, inp.block_tables, inp.context_lens,
                                          wl.block_size, per_tensor=(kind == "fp8_tensor")))
    return (orc.quantize_pool(inp.k_pool[0], sc[0], _dtype(kind)),
            orc.quantize_pool(inp.v_pool[0], sc[1], _dtype(kind)), sc[0], sc[1])


def _oracle_step(orc, inp, kc, vc, ks, vs, kind):
    kp, vp = kc.copy(), vc.copy()
    orc.append(inp.k_new[0], inp.v_new[0], kp, vp, inp.block_tables, inp.context_lens,
               inp.wl.block_size, kv_dtype=_dtype(kind), k_scale=ks, v_scale=vs)
    out, lse = orc.paged_attention(inp.query[0], kp, vp, inp.block_tables, inp.context_lens,
                                   inp.scale, block_size=inp.wl.block_size, Hkv=inp.wl.Hkv,
                                   kv_dtype=_dtype(kind), k_scale=ks, v_scale=vs)
    return kp, vp, out, lse


class Dev:
    def __init__(self, inp, kc, vc, ks, vs, kind):
        self.k, self.v = to_dev(kc), to_dev(vc)
        self.ks = None if ks is None else to_dev(ks)
        self.vs = None if vs is None else to_dev(vs)
        self.bt, self.cl = tables_to_dev(inp.block_tables, inp.context_lens,
                                         inp.wl.block_size, kc.shape[0])
        self.q = to_dev(inp.query[0])
        self.k_new, self.v_new = to_dev(inp.k_new[0]), to_dev(inp.v_new[0])
        self.kw = dict(k_scale=self.ks, v_scale=self.vs, kv_dtype=_dtype(kind))


def _fused(pkv, inp, d, mode, split=48):
    """One fused step; returns out, lse (split: through split_context_reduce)."""
    wl = inp.wl
    lse = torch.empty((wl.B, wl.Hq), dtype=torch.float32, device=dev())
    sc = float(inp.scale)
    if mode == "single":
        out = pkv.paged_append_decode_attention(d.q, d.k_new, d.v_new, d.k, d.v, d.bt, d.cl,
                                                sc, lse_out=lse, **d.kw)
    elif mode == "split":
        ms = pkv.max_splits_for(int(inp.context_lens.max()), split)
        po = torch.full((wl.B, wl.Hq, ms, wl.D), float("nan"), device=dev())
        pl = torch.full((wl.B, wl.Hq, ms), float("nan"), device=dev())
        pkv.paged_append_decode_attention(d.q, d.k_new, d.v_new, d.k, d.v, d.bt, d.cl, sc,
                                          split_tokens=split, partial_out=po, partial_lse=pl,
                                          **d.kw)
        out = pkv.split_context_reduce(po, pl, d.cl, split, lse_out=lse)
    else:
        ws = pkv.make_workspace(d.q, d.k, kv_dtype=d.kw["kv_dtype"])
        ws.fill_(0xFF)
        out = pkv.paged_append_decode_attention_balanced(d.q, d.k_new, d.v_new, d.k, d.v, d.bt,
                                                         d.cl, sc, workspace=ws, lse_out=lse,
                                                         **d.kw)
    torch.cuda.synchronize()
    return out, lse


def _check(orc, pkv, inp, kind, mode, split, what):
    kc, vc, ks, vs = _caches(orc, inp, kind)
    d = Dev(inp, kc, vc, ks, vs, kind)
    out, lse = _fused(pkv, inp, d, mode, split)
    kp, vp, ref, rlse = _oracle_step(orc, inp, kc, vc, ks, vs, kind)
    assert np.array_equal(d.k.cpu().numpy().view(kp.dtype), kp), f"{what}: K cache"
    assert np.array_equal(d.v.cpu().numpy().view(vp.dtype), vp), f"{what}: V cache"
    assert_close(out, ref, what)
    assert_close(lse, rlse, what + " lse")


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("mode,split", [("single", 0), ("split", 16), ("split", 48),
                                        ("split", 512), ("balanced", 0)])
def test_tiny(orc, pkv, kind, mode, split):
    inp = generate(make_workload(TINY))
    what = f"fused tiny {kind} {mode} {split}"
    print(what, flush=True)
    _check(orc, pkv, inp, kind, mode, split, what)


@pytest.mark.parametrize("kind", ["bf16", "fp8", "int8"])
@pytest.mark.parametrize("G", [1, 8, 16])
@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("D", [64, 128])
def test_shapes(orc, pkv, D, bs, G, kind):
    Hkv = 2
    wl = make_workload(TINY, B=len(EDGE_CTX), Hq=G * Hkv, Hkv=Hkv, D=D, block_size=bs,
                       ctx_fixed=EDGE_CTX, max_blocks=(300 + bs - 1) // bs + 1,
                       pool="holes10", seed=2000 + D + bs + G)
    inp = generate(wl)
    for mode, split in (("single", 0), ("split", 2 * bs), ("balanced", 0)):
        what = f"fused D={D} bs={bs} G={G} {kind} {mode}"
        print(what, flush=True)
        _check(orc, pkv, inp, kind, mode, split, what)


def _separate(pkv, inp, d, mode, split, ws):
    wl = inp.wl
    sc = float(inp.scale)
    pkv.paged_kv_append(d.k_new, d.v_new, d.k, d.v, d.bt, d.cl, **d.kw)
    if mode == "split":
        ms = pkv.max_splits_for(int(inp.context_lens.max()), split)
        po = torch.empty((wl.B, wl.Hq, ms, wl.D), dtype=torch.float32, device=dev())
        pl = torch.empty((wl.B, wl.Hq, ms), dtype=torch.float32, device=dev())
        pkv.paged_decode_attention(d.q, d.k, d.v, d.bt, d.cl, sc, split_tokens=split,
                                   partial_out=po, partial_lse=pl, **d.kw)
        return pkv.split_context_reduce(po, pl, d.cl, split)
    return pkv.paged_decode_attention_balanced(d.q, d.k, d.v, d.bt, d.cl, sc, workspace=ws,
                                               **d.kw)


def _fused_full(pkv, inp, d, mode, split, ws):
    wl = inp.wl
    sc = float(inp.scale)
    if mode == "split":
        ms = pkv.max_splits_for(int(inp.context_lens.max()), split)
        po = torch.empty((wl.B, wl.Hq, ms, wl.D), dtype=torch.float32, device=dev())
        pl = torch.empty((wl.B, wl.Hq, ms), dtype=torch.float32, device=dev())
        pkv.paged_append_decode_attention(d.q, d.k_new, d.v_new, d.k, d.v, d.bt, d.cl, sc,
                                          split_tokens=split, partial_out=po,
                                          partial_lse=pl, **d.kw)
        return pkv.split_context_reduce(po, pl, d.cl, split)
    return pkv.paged_append_decode_attention_balanced(d.q, d.k_new, d.v_new, d.k, d.v, d.bt,
                                                      d.cl, sc, workspace=ws, **d.kw)


@pytest.mark.parametrize("name,mode,split", [
    ("llama70b_b4_ctx32k_split512_prefix2k", "split", 512),
    ("llama70b_b64_ragged1k_16k_bs32", "balanced", 0),
    ("llama8b_b32_ctx4096_bs16", "balanced", 0),
])
def test_full_size_equals_separate_calls(pkv, name, mode, split):
    """Same kernels, same bytes: the fused step must reproduce the separate
    append + attention bit for bit, caches included."""
    inp = generate(make_workload(name))
    print(f"fused full size {name} {mode}", flush=True)
    a = Dev(inp, inp.k_pool[0], inp.v_pool[0], None, None, "bf16")
    ws = pkv.make_workspace(a.q, a.k) if mode == "balanced" else None
    ref = _separate(pkv, inp, a, mode, split, ws)
    torch.cuda.synchronize()
    kref, vref = a.k, a.v
    b = Dev(inp, inp.k_pool[0], inp.v_pool[0], None, None, "bf16")
    out = _fused_full(pkv, inp, b, mode, split, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert torch.equal(out, ref)
    assert torch.equal(b.k, kref) and torch.equal(b.v, vref)


def test_fused_rejects_missing_rows(pkv):
    inp = generate(make_workload(TINY))
    d = Dev(inp, inp.k_pool[0], inp.v_pool[0], None, None, "bf16")
    with pytest.raises(Exception):
        pkv.paged_append_decode_attention(d.q, d.k_new, None, d.k, d.v, d.bt, d.cl, 0.125)


@pytest.mark.parametrize("mode,split", [("single", 0), ("split", 32), ("split", 512),
                                        ("balanced", 0)])
def test_empty_and_one_token_sequences(orc, pkv, mode, split):
    """T = 0 sequences are neither written nor attended (out 0, lse -inf);
    T = 1 sequences attend only the row the call itself writes (= V)."""
    ctx = (0, 5000, 0, 1, 33, 7000, 0, 64, 1)
    wl = make_workload("llama70b_b64_ragged1k_16k_bs32", B=len(ctx), ctx_fixed=ctx,
                       max_blocks=220, Hq=16, Hkv=2, seed=5100)
    inp = generate(wl)
    what = f"fused empty {mode} {split}"
    print(what, flush=True)
    d = Dev(inp, inp.k_pool[0], inp.v_pool[0], None, None, "bf16")
    out, lse = _fused(pkv, inp, d, mode, split)
    kp, vp, ref, rlse = _oracle_step(orc, inp, inp.k_pool[0], inp.v_pool[0], None, None, "bf16")
    assert np.array_equal(d.k.cpu().numpy().view(kp.dtype), kp), what
    assert np.array_equal(d.v.cpu().numpy().view(vp.dtype), vp), what
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for b in (0, 2, 6):
        assert np.all(o[b] == 0) and np.all(np.isneginf(l[b])), b
    keep = [1, 3, 4, 5, 7, 8]
    assert_close(o[keep], ref[keep], what)
    assert_close(l[keep], rlse[keep], what + " lse")
    # one token: out is exactly that token's V row (softmax weight 1)
    from synthetic import f32_from_bf16_bits
    for b in (3, 8):
        v = f32_from_bf16_bits(inp.v_new[0][b]).astype(np.float32)     # [Hkv, D]
        assert np.array_equal(o[b], np.repeat(v, wl.G, axis=0)), b


def test_fused_deterministic(pkv):
    """Two fused calls on the same inputs give the same bits (the second call
    rewrites the same rows)."""
    inp = generate(make_workload("llama70b_b64_ragged1k_16k_bs32", B=16,
                                 ctx_uniform=(100, 3000), max_blocks=100, Hq=16, Hkv=2))
    d = Dev(inp, inp.k_pool[0], inp.v_pool[0], None, None, "bf16")
    outs = [_fused(pkv, inp, d, mode, 64)[0].clone() for mode in ("balanced", "balanced")]
    assert torch.equal(outs[0], outs[1])
    outs = [_fused(pkv, inp, d, "split", 64)[0].clone() for _ in range(2)]
    assert torch.equal(outs[0], outs[1])
