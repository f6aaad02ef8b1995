"""GPU parity of paged_kv_write + paged_multiquery_attention against the CPU
oracle: several new tokens per sequence, each attending causally over its
sequence up to its own position (chunked prefill, [B] "Continuous
Batching"; draft-token verification, [A] "How does speculative decoding
interact with KV-cache compression").

Writes are compared bit for bit; attention element by element at oracle
sizes (every kernel shape, ragged q_b including 0 and q_b = T_b, column
groups beyond one wave), by sampled rows at the 70B verification size,
and by invariants: equal keys with V[t] = t give p / 2 in every row,
physical placement does not matter, repeated calls are bit-identical.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_close, bits16, dev, sample_rows, tables_to_dev, to_dev
from synthetic import bf16_bits_from_f32, generate_multiquery, make_workload

pytestmark = pytest.mark.gpu
TINY = "tiny_mq_b4_hq8_hkv2_d64_bs16"
EDGE_CTX = (1, 2, 15, 16, 17, 31, 32, 33, 47, 63, 64, 65, 100, 255, 300)
Q_CYCLE = (1, 2, 3, 0, 5, 8, 13, 16, 17, 31, 33, 64, 4, 40, 300)


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_273_amd as m

    return m


class MQDevice:
    """Device copies of a multi-query step (one cache group)."""

    def __init__(self, mq, k_pool=None, v_pool=None, k_scale=None, v_scale=None):
        base = mq.base
        self.mq = mq
        self.k = to_dev(base.k_pool[0] if k_pool is None else k_pool)
        self.v = to_dev(base.v_pool[0] if v_pool is None else v_pool)
        self.k_rows = to_dev(mq.k_rows[0])
        self.v_rows = to_dev(mq.v_rows[0])
        self.q = to_dev(mq.query[0])
        self.qs = to_dev(mq.query_start)
        self.bt, self.cl = tables_to_dev(base.block_tables, base.context_lens,
                                         base.wl.block_size, self.k.shape[0])
        self.ks = None if k_scale is None else to_dev(k_scale)
        self.vs = None if v_scale is None else to_dev(v_scale)
        self.max_q = max(1, int(mq.query_lens.max()))


def run_mq(pkv, d, scale=None, write=True):
    mq = d.mq
    sc = float(mq.base.scale) if scale is None else float(scale)
    if write:
        pkv.paged_kv_write(d.k_rows, d.v_rows, d.qs, d.k, d.v, d.bt, d.cl, d.max_q,
                           k_scale=d.ks, v_scale=d.vs)
    ws = pkv.make_multiquery_workspace(d.q, d.k, d.max_q)
    ws.fill_(0xFF)          # NaN garbage: the workspace contents on entry must not matter
    lse = torch.empty((mq.rows, mq.wl.Hq), dtype=torch.float32, device=dev())
    out = pkv.paged_multiquery_attention(d.q, d.qs, d.k, d.v, d.bt, d.cl, sc, d.max_q,
                                         workspace=ws, lse_out=lse, k_scale=d.ks, v_scale=d.vs)
    torch.cuda.synchronize()
    return out, lse


def host_written(orc, mq, k_pool=None, v_pool=None, **kw):
    base = mq.base
    kp = (base.k_pool[0] if k_pool is None else k_pool).copy()
    vp = (base.v_pool[0] if v_pool is None else v_pool).copy()
    orc.write_tokens(mq.k_rows[0], mq.v_rows[0], mq.query_start, kp, vp, base.block_tables,
                     base.context_lens, mq.wl.block_size, **kw)
    return kp, vp


def oracle_mq(orc, mq, kp, vp, scale=None, **kw):
    base = mq.base
    return orc.multiquery_attention(mq.query[0], mq.query_start, kp, vp, base.block_tables,
                                    base.context_lens, base.scale if scale is None else scale,
                                    block_size=mq.wl.block_size, Hkv=mq.wl.Hkv, **kw)


def fp8_pools(orc, mq):
    base, wl = mq.base, mq.wl
    ks = orc.fp8_block_scales(base.k_pool[0], base.block_tables, base.context_lens,
                              wl.block_size)
    vs = orc.fp8_block_scales(base.v_pool[0], base.block_tables, base.context_lens,
                              wl.block_size)
    return (orc.fp8_quantize_pool(base.k_pool[0], ks), orc.fp8_quantize_pool(base.v_pool[0], vs),
            ks, vs)


@pytest.mark.parametrize("scale", [None, 1.0])
@pytest.mark.parametrize("seed", [0, 1])
def test_tiny(orc, pkv, scale, seed):
    mq = generate_multiquery(make_workload(TINY), seed=273010 + seed)
    print(f"mq tiny scale={scale} seed={seed}", flush=True)
    d = MQDevice(mq)
    out, lse = run_mq(pkv, d, scale=scale)
    kp, vp = host_written(orc, mq)
    assert np.array_equal(bits16(d.k), kp) and np.array_equal(bits16(d.v), vp)
    ref, rlse = oracle_mq(orc, mq, kp, vp, scale=scale)
    assert_close(out, ref, "mq out")
    assert_close(lse, rlse, "mq lse")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_write_is_bit_exact(orc, pkv, kv):
    wl = make_workload(TINY, B=len(EDGE_CTX), ctx_fixed=EDGE_CTX, max_blocks=20,
                       pool="holes10", seed=2100)
    mq = generate_multiquery(wl, query_lens=np.array(Q_CYCLE))
    print(f"mq write kv={kv}", flush=True)
    if kv == "fp8":
        kc, vc, ks, vs = fp8_pools(orc, mq)
        d = MQDevice(mq, k_pool=kc, v_pool=vc, k_scale=ks, v_scale=vs)
        kp, vp = host_written(orc, mq, kc, vc, kv_dtype="fp8", k_scale=ks, v_scale=vs)
        pkv.paged_kv_write(d.k_rows, d.v_rows, d.qs, d.k, d.v, d.bt, d.cl, d.max_q,
                           k_scale=d.ks, v_scale=d.vs)
        torch.cuda.synchronize()
        assert np.array_equal(d.k.cpu().numpy(), kp) and np.array_equal(d.v.cpu().numpy(), vp)
    else:
        d = MQDevice(mq)
        kp, vp = host_written(orc, mq)
        pkv.paged_kv_write(d.k_rows, d.v_rows, d.qs, d.k, d.v, d.bt, d.cl, d.max_q)
        torch.cuda.synchronize()
        assert np.array_equal(bits16(d.k), kp) and np.array_equal(bits16(d.v), vp)


@pytest.mark.parametrize("runs", ["short", "long"])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("G", [1, 4, 8, 16])
@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("D", [64, 128])
def test_shapes(orc, pkv, D, bs, G, kv, runs):
    """Every kernel shape; q_b from 0 to T_b, so the causal edge falls at
    every offset of a tile.  "long" runs (up to 300 new tokens) take the
    prefill kernel (256 columns per work-group, K/V staged in LDS); "short"
    runs (q_b * G <= 128) the decode-shaped path with one to four column
    groups per unit."""
    Hkv = 2
    wl = make_workload(TINY, B=len(EDGE_CTX), Hq=G * Hkv, Hkv=Hkv, D=D, block_size=bs,
                       ctx_fixed=EDGE_CTX, max_blocks=(300 + bs - 1) // bs + 1,
                       pool="holes10", kv_dtype=kv, seed=2200 + D + bs + G)
    qlens = np.array(Q_CYCLE) if runs == "long" else np.minimum(np.array(Q_CYCLE), 128 // G)
    mq = generate_multiquery(wl, query_lens=qlens)
    print(f"mq shape D={D} bs={bs} G={G} kv={kv} runs={runs}", flush=True)
    if kv == "fp8":
        kc, vc, ks, vs = fp8_pools(orc, mq)
        d = MQDevice(mq, k_pool=kc, v_pool=vc, k_scale=ks, v_scale=vs)
        kw = dict(kv_dtype="fp8", k_scale=ks, v_scale=vs)
        kp, vp = host_written(orc, mq, kc, vc, **kw)
    else:
        d = MQDevice(mq)
        kw = {}
        kp, vp = host_written(orc, mq)
    out, lse = run_mq(pkv, d)
    ref, rlse = oracle_mq(orc, mq, kp, vp, **kw)
    assert_close(out, ref, "mq shapes")
    assert_close(lse, rlse, "mq shapes lse")


@pytest.mark.parametrize("max_q", [4, 40])
def test_equal_keys_pin_every_position(pkv, max_q):
    """All keys equal, V[t] = t (exact in bf16 up to 256): row i of sequence
    b is the mean of 0..p = p / 2, p = T_b - q_b + i."""
    ctx = (3, 17, 100, 256, 40, 1)
    wl = make_workload(TINY, B=len(ctx), ctx_fixed=ctx, max_blocks=17, Hq=16, Hkv=2, D=128,
                       seed=2300)
    q = np.minimum(np.array([3, 9, max_q, max_q, 40, 1]), np.array(ctx))
    mq = generate_multiquery(wl, query_lens=q)
    base = mq.base
    kp, vp = base.k_pool[0].copy(), base.v_pool[0].copy()
    key = bf16_bits_from_f32(np.random.default_rng(5).standard_normal((wl.Hkv, wl.D)))
    for b in range(wl.B):
        for t in range(int(ctx[b])):
            p = base.block_tables[b, t // wl.block_size]
            kp[p, t % wl.block_size] = key
            vp[p, t % wl.block_size] = bf16_bits_from_f32(np.full((wl.Hkv, wl.D), t, np.float32))
    d = MQDevice(mq, k_pool=kp, v_pool=vp)
    out, _ = run_mq(pkv, d, scale=1.0, write=False)
    want = np.zeros((mq.rows, wl.Hq, wl.D))
    for b in range(wl.B):
        for i in range(int(q[b])):
            want[mq.query_start[b] + i] = (ctx[b] - q[b] + i) / 2.0
    assert_close(out, want, "equal keys")


def test_deterministic_and_placement_free(orc, pkv):
    wl = make_workload("llama70b_b64_ragged1k_16k_bs32_verify4", B=6, ctx_uniform=(1, 3000),
                       max_blocks=94, q_uniform=(1, 9))
    mq = generate_multiquery(wl)
    kp, vp = host_written(orc, mq)
    d = MQDevice(mq, k_pool=kp, v_pool=vp)
    a, la = run_mq(pkv, d, write=False)
    b, lb = run_mq(pkv, d, write=False)
    assert torch.equal(a, b) and torch.equal(la, lb)
    rng = np.random.default_rng(11)
    nb = kp.shape[0]
    perm = rng.permutation(nb)              # new physical index of old block j
    kq, vq = np.empty_like(kp), np.empty_like(vp)
    kq[perm], vq[perm] = kp, vp
    tq = mq.base.block_tables.copy()
    tq[tq >= 0] = perm[tq[tq >= 0]]
    d2 = MQDevice(mq, k_pool=kq, v_pool=vq)
    d2.bt = tables_to_dev(tq, mq.base.context_lens, mq.base.wl.block_size, nb)[0]
    c, lc = run_mq(pkv, d2, write=False)
    assert torch.equal(a, c) and torch.equal(la, lc)
    ref, _ = oracle_mq(orc, mq, kp, vp)
    assert_close(a, ref, "mq")


def test_one_new_token_matches_decode(orc, pkv):
    """q_b = 1 is the decode step: same result as the balanced decode."""
    wl = make_workload("llama70b_b64_ragged1k_16k_bs32_verify4", B=8, ctx_uniform=(1, 2000),
                       max_blocks=64)
    mq = generate_multiquery(wl, query_lens=np.ones(8, dtype=np.int32))
    kp, vp = host_written(orc, mq)
    d = MQDevice(mq, k_pool=kp, v_pool=vp)
    out, lse = run_mq(pkv, d, write=False)
    ws = pkv.make_workspace(d.q, d.k)
    ref = pkv.paged_decode_attention_balanced(d.q, d.k, d.v, d.bt, d.cl, float(mq.base.scale),
                                              workspace=ws)
    torch.cuda.synchronize()
    assert_close(out, ref.cpu().numpy(), "q=1 vs decode")


def test_rows_outside_sequences_untouched(orc, pkv):
    mq = generate_multiquery(make_workload(TINY))
    d = MQDevice(mq)
    pkv.paged_kv_write(d.k_rows, d.v_rows, d.qs, d.k, d.v, d.bt, d.cl, d.max_q)
    extra = 5
    q = torch.zeros((mq.rows + extra, mq.wl.Hq, mq.wl.D), dtype=torch.int16, device=dev())
    q[:mq.rows] = d.q
    out = torch.full((mq.rows + extra, mq.wl.Hq, mq.wl.D), 7.0, device=dev())
    ws = pkv.make_multiquery_workspace(q, d.k, d.max_q)
    pkv.paged_multiquery_attention(q, d.qs, d.k, d.v, d.bt, d.cl, float(mq.base.scale), d.max_q,
                                   workspace=ws, out=out)
    torch.cuda.synchronize()
    assert torch.all(out[mq.rows:] == 7.0)
    kp, vp = host_written(orc, mq)
    ref, _ = oracle_mq(orc, mq, kp, vp)
    assert_close(out[:mq.rows], ref, "mq")


def test_workspace_too_small(pkv):
    mq = generate_multiquery(make_workload(TINY))
    d = MQDevice(mq)
    ws = torch.empty(64, dtype=torch.uint8, device=dev())
    with pytest.raises(pkv.PagedKVError):
        pkv.paged_multiquery_attention(d.q, d.qs, d.k, d.v, d.bt, d.cl, 0.125, d.max_q,
                                       workspace=ws)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_verify4_fullsize_sampled(orc, pkv, kv):
    """The 70B ragged batch with 4 new tokens per sequence, in the launch
    configuration the benchmark times; sampled rows against the oracle
    (row i of sequence b is the decode attention over its first p + 1
    tokens, p = T_b - 4 + i)."""
    wl = make_workload("llama70b_b64_ragged1k_16k_bs32_verify4", kv_dtype=kv)
    mq = generate_multiquery(wl)
    base = mq.base
    print(f"mq verify4 fullsize kv={kv}", flush=True)
    if kv == "fp8":
        kc, vc, ks, vs = fp8_pools(orc, mq)
        kw = dict(kv_dtype="fp8", k_scale=ks, v_scale=vs)
        d = MQDevice(mq, k_pool=kc, v_pool=vc, k_scale=ks, v_scale=vs)
    else:
        kc, vc, ks, vs = base.k_pool[0], base.v_pool[0], None, None
        kw = {}
        d = MQDevice(mq)
    out, lse = run_mq(pkv, d)
    kp, vp = host_written(orc, mq, kc, vc, **kw)
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for (row, hq) in sample_rows(mq.rows, wl.Hq, 24, seed=5):
        b = int(np.searchsorted(mq.query_start, row, side="right") - 1)
        p = int(base.context_lens[b]) - int(mq.query_lens[b]) + (row - int(mq.query_start[b]))
        ref, rl = orc.paged_attention(np.ascontiguousarray(mq.query[0][row:row + 1]), kp, vp,
                                      np.ascontiguousarray(base.block_tables[b:b + 1]),
                                      np.array([p + 1], dtype=np.int32), base.scale,
                                      block_size=wl.block_size, Hkv=wl.Hkv, **kw)
        assert_close(o[row, hq], ref[0, hq], f"row {row} head {hq}")
        assert_close(l[row, hq], rl[0, hq], f"lse row {row} head {hq}")


@pytest.mark.parametrize("B", [60, 300])
def test_many_sequences(orc, pkv, B):
    """Four new tokens per sequence over short ragged contexts, batches of 60
    and 300 (more units than launched work-groups); every row against the
    oracle."""
    wl = make_workload("llama70b_b64_ragged1k_16k_bs32_verify4", B=B, ctx_uniform=(4, 500),
                       max_blocks=16, seed=2500 + B)
    mq = generate_multiquery(wl)
    print(f"mq merge grids B={B}", flush=True)
    d = MQDevice(mq)
    out, lse = run_mq(pkv, d)
    kp, vp = host_written(orc, mq)
    ref, rlse = oracle_mq(orc, mq, kp, vp)
    assert_close(out, ref, f"mq B={B}")
    assert_close(lse, rlse, f"mq B={B} lse")


@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_prefill_chunk_sampled(orc, pkv, kv):
    """A 700-token chunk at the end of 3000-token prompts (8B shape): the
    prefill kernel, sampled rows against the oracle (row i is the decode
    attention over the first T - 700 + i + 1 tokens)."""
    wl = make_workload("llama8b_b4_ctx8k_chunk512", B=2, ctx_fixed=(3000, 2100),
                       max_blocks=200, q_uniform=(700, 700), seed=2400)
    mq = generate_multiquery(wl)
    base = mq.base
    print(f"prefill chunk kv={kv}", flush=True)
    if kv == "int8":
        ks = orc.int8_block_params(base.k_pool[0], base.block_tables, base.context_lens,
                                   wl.block_size)
        vs = orc.int8_block_params(base.v_pool[0], base.block_tables, base.context_lens,
                                   wl.block_size)
        kc, vc = orc.quantize_pool(base.k_pool[0], ks, "int8"), orc.quantize_pool(base.v_pool[0], vs,
                                                                                    "int8")
        kw = dict(kv_dtype="int8", k_scale=ks, v_scale=vs)
        dkw = dict(kv_dtype="int8", k_scale=to_dev(ks), v_scale=to_dev(vs))
    else:
        kc, vc = base.k_pool[0], base.v_pool[0]
        kw, dkw = {}, {}
    d = MQDevice(mq, k_pool=kc, v_pool=vc)
    pkv.paged_kv_write(d.k_rows, d.v_rows, d.qs, d.k, d.v, d.bt, d.cl, d.max_q, **dkw)
    ws = pkv.make_multiquery_workspace(d.q, d.k, d.max_q, kv_dtype=dkw.get("kv_dtype"))
    lse = torch.empty((mq.rows, wl.Hq), dtype=torch.float32, device=dev())
    out = pkv.paged_multiquery_attention(d.q, d.qs, d.k, d.v, d.bt, d.cl, float(base.scale),
                                         d.max_q, workspace=ws, lse_out=lse, **dkw)
    torch.cuda.synchronize()
    kp, vp = host_written(orc, mq, kc, vc, **kw)
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for (row, hq) in sample_rows(mq.rows, wl.Hq, 32, seed=7):
        b = int(np.searchsorted(mq.query_start, row, side="right") - 1)
        p = int(base.context_lens[b]) - int(mq.query_lens[b]) + (row - int(mq.query_start[b]))
        ref, rl = orc.paged_attention(np.ascontiguousarray(mq.query[0][row:row + 1]), kp, vp,
                                      np.ascontiguousarray(base.block_tables[b:b + 1]),
                                      np.array([p + 1], dtype=np.int32), base.scale,
                                      block_size=wl.block_size, Hkv=wl.Hkv, **kw)
        assert_close(o[row, hq], ref[0, hq], f"row {row} head {hq}")
        assert_close(l[row, hq], rl[0, hq], f"lse row {row} head {hq}")


def test_workspace_reused_by_later_calls(orc, pkv):
    """Multi-query calls with different queries share one workspace: each
    merges its own pieces."""
    mq = generate_multiquery(make_workload("llama70b_b64_ragged1k_16k_bs32_verify4", B=8,
                                           ctx_uniform=(100, 6000), max_blocks=188))
    d = MQDevice(mq)
    kp, vp = host_written(orc, mq)
    pkv.paged_kv_write(d.k_rows, d.v_rows, d.qs, d.k, d.v, d.bt, d.cl, d.max_q)
    ws = pkv.make_multiquery_workspace(d.q, d.k, d.max_q)
    base = mq.base
    q_a = mq.query[0]
    q_b = (q_a ^ np.uint16(0x8000)).astype(np.uint16)
    for i, q in enumerate((q_a, q_b, q_a)):
        out = pkv.paged_multiquery_attention(to_dev(q), d.qs, d.k, d.v, d.bt, d.cl,
                                             float(base.scale), d.max_q, workspace=ws)
        torch.cuda.synchronize()
        ref, _ = orc.multiquery_attention(q, mq.query_start, kp, vp, base.block_tables,
                                          base.context_lens, base.scale,
                                          block_size=mq.wl.block_size, Hkv=mq.wl.Hkv)
        assert_close(out[:mq.rows], ref, f"call {i}")
