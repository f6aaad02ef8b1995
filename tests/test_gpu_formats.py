"""GPU parity of the other 1-byte cache formats against the oracle:
E4M3 with one scale per kv head or per tensor ([B] "FP8 KV cache": per-head
or per-tensor scaling), and INT8 codes with a per-(block, kv head) scale and
zero point, symmetric and asymmetric ([B] "INT8 KV cache").

Writes (append, multi-token write, all 65,536 bf16 inputs) are compared bit
for bit; attention (single pass, fixed splits + reduce, balanced, multi-
query) element by element; block moves carry the int8 (scale, zero point)
pairs with their blocks.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_close, dev, tables_to_dev, to_dev
from synthetic import generate, generate_multiquery, make_workload

pytestmark = pytest.mark.gpu
TINY = "tiny_b4_hq8_hkv2_d64_bs16"
KINDS = ["fp8_head", "fp8_tensor", "int8", "int8_sym"]
EDGE_CTX = (1, 2, 15, 16, 17, 31, 32, 33, 47, 63, 64, 65, 100, 255, 300)


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_273_amd as m

    return m


def _dtype(kind):
    return "int8" if kind.startswith("int8") else kind


def _params(orc, kind, src, tables, ctx, bs):
    if kind.startswith("int8"):
        return orc.int8_block_params(src, tables, ctx, bs, symmetric=(kind == "int8_sym"))
    return orc.fp8_wide_scales(src, tables, ctx, bs, per_tensor=(kind == "fp8_tensor"))


def _caches(orc, inp, kind, group=0):
    wl = inp.wl
    ks = _params(orc, kind, inp.k_pool[group], inp.block_tables, inp.context_lens,
                 wl.block_size)
    vs = _params(orc, kind, inp.v_pool[group], inp.block_tables, inp.context_lens,
                 wl.block_size)
    return (orc.quantize_pool(inp.k_pool[group], ks, _dtype(kind)),
            orc.quantize_pool(inp.v_pool[group], vs, _dtype(kind)), ks, vs)


class Dev:
    def __init__(self, inp, kc, vc, ks, vs, kind):
        self.k, self.v = to_dev(kc), to_dev(vc)
        self.ks, self.vs = to_dev(ks), to_dev(vs)
        self.bt, self.cl = tables_to_dev(inp.block_tables, inp.context_lens,
                                         inp.wl.block_size, kc.shape[0])
        self.q = to_dev(inp.query[0])
        self.k_new, self.v_new = to_dev(inp.k_new[0]), to_dev(inp.v_new[0])
        self.dt = _dtype(kind)


def _oracle_step(orc, inp, kc, vc, ks, vs, kind):
    kp, vp = kc.copy(), vc.copy()
    orc.append(inp.k_new[0], inp.v_new[0], kp, vp, inp.block_tables, inp.context_lens,
               inp.wl.block_size, kv_dtype=_dtype(kind), k_scale=ks, v_scale=vs)
    out, lse = orc.paged_attention(inp.query[0], kp, vp, inp.block_tables, inp.context_lens,
                                   inp.scale, block_size=inp.wl.block_size, Hkv=inp.wl.Hkv,
                                   kv_dtype=_dtype(kind), k_scale=ks, v_scale=vs)
    return kp, vp, out, lse


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("mode", ["single", "split", "balanced"])
def test_tiny_step(orc, pkv, kind, mode):
    inp = generate(make_workload(TINY))
    print(f"format {kind} {mode}", flush=True)
    kc, vc, ks, vs = _caches(orc, inp, kind)
    d = Dev(inp, kc, vc, ks, vs, kind)
    kw = dict(k_scale=d.ks, v_scale=d.vs, kv_dtype=d.dt)
    pkv.paged_kv_append(d.k_new, d.v_new, d.k, d.v, d.bt, d.cl, **kw)
    kp, vp, ref, rlse = _oracle_step(orc, inp, kc, vc, ks, vs, kind)
    torch.cuda.synchronize()
    assert np.array_equal(d.k.cpu().numpy(), kp) and np.array_equal(d.v.cpu().numpy(), vp)
    wl = inp.wl
    lse = torch.empty((wl.B, wl.Hq), dtype=torch.float32, device=dev())
    sc = float(inp.scale)
    if mode == "single":
        out = pkv.paged_decode_attention(d.q, d.k, d.v, d.bt, d.cl, sc, lse_out=lse, **kw)
    elif mode == "split":
        ms = pkv.max_splits_for(int(inp.context_lens.max()), 48)
        po = torch.full((wl.B, wl.Hq, ms, wl.D), float("nan"), device=dev())
        pl = torch.full((wl.B, wl.Hq, ms), float("nan"), device=dev())
        pkv.paged_decode_attention(d.q, d.k, d.v, d.bt, d.cl, sc, split_tokens=48,
                                   partial_out=po, partial_lse=pl, **kw)
        out = pkv.split_context_reduce(po, pl, d.cl, 48, lse_out=lse)
    else:
        ws = pkv.make_workspace(d.q, d.k, kv_dtype=d.dt)
        ws.fill_(0xFF)
        out = pkv.paged_decode_attention_balanced(d.q, d.k, d.v, d.bt, d.cl, sc, workspace=ws,
                                                  lse_out=lse, **kw)
    torch.cuda.synchronize()
    assert_close(out, ref, f"{kind} {mode}")
    assert_close(lse, rlse, f"{kind} {mode} lse")


@pytest.mark.parametrize("kind", ["fp8_head", "int8"])
@pytest.mark.parametrize("G", [1, 8, 16])
@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("D", [64, 128])
def test_shapes_balanced(orc, pkv, D, bs, G, kind):
    Hkv = 2
    wl = make_workload(TINY, B=len(EDGE_CTX), Hq=G * Hkv, Hkv=Hkv, D=D, block_size=bs,
                       ctx_fixed=EDGE_CTX, max_blocks=(300 + bs - 1) // bs + 1,
                       pool="holes10", seed=3000 + D + bs + G)
    inp = generate(wl)
    print(f"format shape {kind} D={D} bs={bs} G={G}", flush=True)
    kc, vc, ks, vs = _caches(orc, inp, kind)
    d = Dev(inp, kc, vc, ks, vs, kind)
    kw = dict(k_scale=d.ks, v_scale=d.vs, kv_dtype=d.dt)
    pkv.paged_kv_append(d.k_new, d.v_new, d.k, d.v, d.bt, d.cl, **kw)
    _, _, ref, rlse = _oracle_step(orc, inp, kc, vc, ks, vs, kind)
    ws = pkv.make_workspace(d.q, d.k, kv_dtype=d.dt)
    lse = torch.empty((wl.B, wl.Hq), dtype=torch.float32, device=dev())
    out = pkv.paged_decode_attention_balanced(d.q, d.k, d.v, d.bt, d.cl, float(inp.scale),
                                              workspace=ws, lse_out=lse, **kw)
    torch.cuda.synchronize()
    assert_close(out, ref, f"{kind} shapes")
    assert_close(lse, rlse, f"{kind} shapes lse")


@pytest.mark.parametrize("kind", KINDS)
def test_multiquery(orc, pkv, kind):
    wl = make_workload("tiny_mq_b4_hq8_hkv2_d64_bs16")
    mq = generate_multiquery(wl)
    base = mq.base
    kc, vc, ks, vs = _caches(orc, base, kind)
    dt = _dtype(kind)
    k, v, kd, vd = to_dev(kc), to_dev(vc), to_dev(ks), to_dev(vs)
    qs = to_dev(mq.query_start)
    bt, cl = tables_to_dev(base.block_tables, base.context_lens, wl.block_size, kc.shape[0])
    max_q = int(mq.query_lens.max())
    pkv.paged_kv_write(to_dev(mq.k_rows[0]), to_dev(mq.v_rows[0]), qs, k, v, bt, cl, max_q,
                       k_scale=kd, v_scale=vd, kv_dtype=dt)
    kp, vp = kc.copy(), vc.copy()
    orc.write_tokens(mq.k_rows[0], mq.v_rows[0], mq.query_start, kp, vp, base.block_tables,
                     base.context_lens, wl.block_size, kv_dtype=dt, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    assert np.array_equal(k.cpu().numpy(), kp) and np.array_equal(v.cpu().numpy(), vp)
    q = to_dev(mq.query[0])
    ws = pkv.make_multiquery_workspace(q, k, max_q, kv_dtype=dt)
    out = pkv.paged_multiquery_attention(q, qs, k, v, bt, cl, float(base.scale), max_q,
                                         workspace=ws, k_scale=kd, v_scale=vd, kv_dtype=dt)
    torch.cuda.synchronize()
    ref, _ = orc.multiquery_attention(mq.query[0], mq.query_start, kp, vp, base.block_tables,
                                      base.context_lens, base.scale, block_size=wl.block_size,
                                      Hkv=wl.Hkv, kv_dtype=dt, k_scale=ks, v_scale=vs)
    assert_close(out, ref, f"{kind} multiquery")


@pytest.mark.parametrize("params", [(1.0, 128.0), (0.0078125, 0.0), (1.0 / 3.0, 255.0),
                                    (7.3, 17.0), (2.0 ** -12, 128.0), (3e4, 100.0)])
def test_int8_encode_exhaustive(orc, pkv, params):
    """All 65,536 bf16 bit patterns through the int8 append: codes equal
    the oracle's (same binary32 division and round-half-even)."""
    B, Hkv, D, bs = 64, 8, 128, 16
    sc, zp = params
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(B, Hkv, D)
    tables = np.arange(B, dtype=np.int32).reshape(B, 1)
    ctx = np.full(B, 1, dtype=np.int32)
    prm = np.empty((B, Hkv, 2), dtype=np.float32)
    prm[..., 0], prm[..., 1] = sc, zp
    vprm = prm.copy()
    vprm[..., 0] = np.float32(1.0) / np.float32(sc)
    kc = np.zeros((B, bs, Hkv, D), dtype=np.uint8)
    vc = np.zeros_like(kc)
    vbits = bits[::-1].copy()
    dk, dv = to_dev(kc), to_dev(vc)
    dbt, dcl = tables_to_dev(tables, ctx, bs, B)
    pkv.paged_kv_append(to_dev(bits), to_dev(vbits), dk, dv, dbt, dcl,
                        k_scale=to_dev(prm), v_scale=to_dev(vprm), kv_dtype="int8")
    torch.cuda.synchronize()
    orc.append(bits, vbits, kc, vc, tables, ctx, bs, kv_dtype="int8", k_scale=prm,
               v_scale=vprm)
    gk, gv = dk.cpu().numpy(), dv.cpu().numpy()
    if not np.array_equal(gk, kc):
        i = tuple(np.argwhere(gk != kc)[0])
        raise AssertionError(f"{params}: K code at {i}: gpu {gk[i]} oracle {kc[i]} "
                             f"(input {bits[i[0], i[2], i[3]]:#06x})")
    assert np.array_equal(gv, vc)


@pytest.mark.parametrize("kind", ["int8", "fp8_head"])
def test_block_moves_carry_their_scales(orc, pkv, kind):
    inp = generate(make_workload(TINY))
    kc, vc, ks, vs = _caches(orc, inp, kind)
    dt = _dtype(kind)
    k, v, kd, vd = to_dev(kc), to_dev(vc), to_dev(ks), to_dev(vs)
    ids = np.array([3, 9, 27], dtype=np.int32)
    ko = torch.empty((3,) + k.shape[1:], dtype=k.dtype, device=dev())
    vo = torch.empty_like(ko)
    per_block = kind == "int8"
    kso = torch.empty((3,) + kd.shape[1:], device=dev()) if per_block else None
    vso = torch.empty_like(kso) if per_block else None
    pkv.paged_kv_gather_blocks(k, v, to_dev(ids), ko, vo, k_scale=kd, v_scale=vd,
                               k_scale_out=kso, v_scale_out=vso, kv_dtype=dt)
    torch.cuda.synchronize()
    assert ko.cpu().numpy().tobytes() == orc.gather_blocks(kc, ids).tobytes()
    if per_block:
        assert np.array_equal(kso.cpu().numpy(), orc.gather_blocks(ks, ids))
        assert np.array_equal(vso.cpu().numpy(), orc.gather_blocks(vs, ids))


def test_int8_full_size_sampled(orc, pkv):
    """The 36-layer workload's shape with an int8 cache (one group, 4 layers
    sharing it), balanced launch configuration; sampled rows."""
    from gpu_helpers import sample_rows

    wl = make_workload("fp8_36layers_groups4_b32_ctx2k_8k", kv_dtype="fp8")
    inp = generate(wl, groups=[0])
    kc, vc, ks, vs = _caches(orc, inp, "int8")
    k, v, kd, vd = to_dev(kc), to_dev(vc), to_dev(ks), to_dev(vs)
    bt, cl = tables_to_dev(inp.block_tables, inp.context_lens, wl.block_size, kc.shape[0])
    kw = dict(k_scale=kd, v_scale=vd, kv_dtype="int8")
    pkv.paged_kv_append(to_dev(inp.k_new[0]), to_dev(inp.v_new[0]), k, v, bt, cl, **kw)
    kp, vp = kc.copy(), vc.copy()
    orc.append(inp.k_new[0], inp.v_new[0], kp, vp, inp.block_tables, inp.context_lens,
               wl.block_size, kv_dtype="int8", k_scale=ks, v_scale=vs)
    for layer in (0, 3):
        q = to_dev(inp.query[layer])
        ws = pkv.make_workspace(q, k, kv_dtype="int8")
        out = pkv.paged_decode_attention_balanced(q, k, v, bt, cl, float(inp.scale),
                                                  workspace=ws, **kw).cpu().numpy()
        for (b, hq) in sample_rows(wl.B, wl.Hq, 16, seed=layer):
            ref, _ = orc.paged_attention(np.ascontiguousarray(inp.query[layer][b:b + 1]), kp, vp,
                                         np.ascontiguousarray(inp.block_tables[b:b + 1]),
                                         np.ascontiguousarray(inp.context_lens[b:b + 1]),
                                         inp.scale, block_size=wl.block_size, Hkv=wl.Hkv,
                                         kv_dtype="int8", k_scale=ks, v_scale=vs)
            assert_close(out[b, hq], ref[0, hq], f"layer {layer} row {b} head {hq}")
