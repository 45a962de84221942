"""The pooled (kpool) indexer chain on the GPU against the oracle: pool compression of packed
k | gate | valid rows, pool scores, pool -> token expansion with the always-selected tail, and
attention over the expanded tokens (vllm-rdna "Glm5Next (GLM-5.3-Flash) on gfx1030" PR).

Rules: 16-bit pool keys equal the oracle's rounding except where the float64 value sits
within 1e-6 of a rounding midpoint, measured against the pool's largest |k| (the kernel sums
in fp32, whose error scales with the terms, and may round either way there; fewer than 1e-3
of the values may differ), fp32 pool keys within 1e-5; pool scores within the dtype tolerance with
the -inf pattern identical; the expansion fed the oracle's pool selection is bit-exact; end
to end, pool indices follow the tie-band rule and attention is within tolerance of the
oracle evaluated on the GPU's own tokens.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (RTOL, assert_rowwise, binding, check_guards, check_index_rule, dev, guarded, guarded_workspace,
                      host)

pytestmark = pytest.mark.gpu
import torch  # noqa: E402

KP = workloads.KPOOL_DECODE_32K
TORCH = {workloads.F32: torch.float32, workloads.BF16: torch.bfloat16, workloads.F16: torch.float16}


def _bits(t: torch.Tensor) -> np.ndarray:
    return host(t.view(torch.int16)).view(np.uint16)


def _term_scale(packed, D, kpool, row_dtype, pools=slice(None)):
    """Per pool, the largest |k| among its tokens: the scale of the fp32 rounding error of a
    weighted sum whose terms may cancel."""
    k, _, _ = oracle.packed_fields(packed, D, row_dtype)
    B, n_kv, _ = k.shape
    n_pool = n_kv // kpool
    m = np.abs(k[:, :n_pool * kpool]).reshape(B, n_pool, kpool * D).max(axis=2)
    return np.broadcast_to(m[:, pools, None], (B, m[:, pools].shape[1], D))


def _check_pool_keys(got: torch.Tensor, x64: np.ndarray, dtype: int, what: str, term: np.ndarray) -> None:
    if dtype == workloads.F32:
        assert_rowwise(host(got), x64, 1e-5, what)
        return
    want = oracle.encode(x64, dtype)
    g = _bits(got)
    bad = g != want
    if bad.any():
        gv = oracle.decode(g[bad], dtype)
        wv = oracle.decode(want[bad], dtype)
        x = x64[bad]
        near_mid = np.abs(gv - x) <= np.abs(wv - x) + 1e-6 * term[bad]
        assert near_mid.all(), f"{what}: {int((~near_mid).sum())} pool-key values off by more than a midpoint flip"
        assert bad.mean() < 1e-3, f"{what}: {bad.mean():.2e} of the values round differently"


def _compress(inp, wl, out_dtype=None, p0=0, p1=None, fill=None):
    L = binding()
    packed = dev(inp["packed"], wl.idx_dtype)
    odt = wl.idx_dtype if out_dtype is None else out_dtype
    shape = (wl.B, wl.n_kv // wl.kpool, wl.D)
    pooled = guarded(shape, TORCH[odt], fill=fill)
    L.dsa_kpool_compress(packed, dev(inp["ape"]), pooled, wl.D, wl.kpool, p0, p1)
    check_guards(f"{wl.name} pool compression")
    return packed, pooled


@pytest.mark.parametrize("row_dtype,out_dtype", [(workloads.F16, workloads.F16), (workloads.BF16, workloads.BF16),
                                                 (workloads.F32, workloads.F32), (workloads.F16, workloads.F32),
                                                 (workloads.F32, workloads.BF16)])
def test_compress(row_dtype, out_dtype):
    wl = KP.scaled(B=3, n_kv=1030, idx_dtype=row_dtype)   # 257 pools and a partial one
    inp = workloads.gen_kpool(wl, 1, hole_frac=0.2)
    _, pooled = _compress(inp, wl, out_dtype)
    torch.cuda.synchronize()
    x64 = oracle.kpool_compress_f64(inp["packed"], inp["ape"], wl.D, wl.kpool, row_dtype)
    _check_pool_keys(pooled, x64, out_dtype, f"pool keys {row_dtype}->{out_dtype}",
                     _term_scale(inp["packed"], wl.D, wl.kpool, row_dtype))


def test_compress_range_and_pool_sizes():
    L = binding()
    # odd and even pool counts and row strides, every pool size
    for n_kv, kpool in ((203, 1), (203, 2), (203, 3), (203, 8), (204, 2), (204, 4), (204, 8), (204, 3)):
        wl = KP.scaled(B=2, n_kv=n_kv, D=64, kpool=kpool)
        inp = workloads.gen_kpool(wl, 2, hole_frac=0.3)
        n_pool = wl.n_kv // kpool
        p0, p1 = n_pool // 3, n_pool - 1
        _, pooled = _compress(inp, wl, p0=p0, p1=p1, fill=7.0)
        torch.cuda.synchronize()
        x64 = oracle.kpool_compress_f64(inp["packed"], inp["ape"], wl.D, kpool, wl.idx_dtype)
        _check_pool_keys(pooled[:, p0:p1].contiguous(), x64[:, p0:p1], wl.idx_dtype, f"n_kv {n_kv} kpool {kpool} range",
                         _term_scale(inp["packed"], wl.D, kpool, wl.idx_dtype, slice(p0, p1)))
        rest = torch.cat([pooled[:, :p0], pooled[:, p1:]], dim=1)
        assert bool((rest == 7.0).all()), f"n_kv {n_kv} kpool {kpool}: pools outside the range were written"
    # wide rows (D 1024 and 4096)
    for D in (1024, 4096):
        wl = KP.scaled(B=1, n_kv=24, D=D)
        inp = workloads.gen_kpool(wl, 10, hole_frac=0.2)
        _, pooled = _compress(inp, wl)
        torch.cuda.synchronize()
        _check_pool_keys(pooled, oracle.kpool_compress_f64(inp["packed"], inp["ape"], D, 4, wl.idx_dtype),
                         wl.idx_dtype, f"D {D}", _term_scale(inp["packed"], D, 4, wl.idx_dtype))
    # a packed row wider than 2 D + 1 (padded stride)
    wl = KP.scaled(B=2, n_kv=64, D=16)
    inp = workloads.gen_kpool(wl, 3, hole_frac=0.2)
    wide = np.zeros((2, 64, 40), np.uint16)
    wide[:, :, :33] = inp["packed"]
    packed = dev(wide, wl.idx_dtype)
    pooled = torch.empty((2, 16, 16), dtype=torch.float16, device="cuda")
    L.dsa_kpool_compress(packed, dev(inp["ape"]), pooled, 16, 4)
    torch.cuda.synchronize()
    _check_pool_keys(pooled, oracle.kpool_compress_f64(inp["packed"], inp["ape"], 16, 4, wl.idx_dtype),
                     wl.idx_dtype, "padded stride", _term_scale(inp["packed"], 16, 4, wl.idx_dtype))


@pytest.mark.parametrize("n_q,H,dtype,explicit", [(1, 32, workloads.F16, False), (2, 32, workloads.F16, True),
                                                  (16, 32, workloads.F16, True), (12, 20, workloads.BF16, True),
                                                  (3, 4, workloads.F32, True)])
def test_pool_scores(n_q, H, dtype, explicit):
    L = binding()
    wl = KP.scaled(B=3, n_q=n_q, H=H, n_kv=1200, idx_dtype=dtype)
    inp = workloads.gen_kpool(wl, 4, hole_frac=0.1, kv_len=[1200, 1195, 7])
    q_pos = None
    if explicit:
        rng = np.random.default_rng(5)
        q_pos = np.stack([rng.integers(-2, int(n), size=n_q) for n in inp["kv_len"]]).astype(np.int32)
        q_pos[0, 0] = 2   # no complete pool yet
    pooled_o = oracle.kpool_compress(inp["packed"], inp["ape"], wl.D, wl.kpool, dtype, dtype)
    n_pool = wl.n_kv // wl.kpool
    scores = torch.empty((wl.B, n_q, n_pool), dtype=torch.float32, device="cuda")
    L.dsa_kpool_index_score(dev(inp["q"], dtype), dev(pooled_o, dtype), dev(inp["w"]), scores, wl.kpool,
                            kv_len=dev(inp["kv_len"]), q_pos=None if q_pos is None else dev(q_pos), scale=0.75)
    torch.cuda.synchronize()
    want = oracle.kpool_scores(inp["q"], pooled_o, inp["w"], inp["kv_len"], q_pos, 0.75, wl.kpool, dtype, dtype)
    assert_rowwise(host(scores), want, RTOL[dtype], f"pool scores n_q={n_q} H={H}")


def test_expand_bit_exact():
    L = binding()
    for n_q, explicit, top_k in ((1, False, 2048), (3, True, 64), (2, True, 4)):
        wl = KP.scaled(B=4, n_q=n_q, n_kv=1100, top_k=top_k)
        inp = workloads.gen_kpool(wl, 6, hole_frac=0.15)
        q_pos = None
        if explicit:
            rng = np.random.default_rng(7)
            q_pos = np.stack([rng.integers(0, int(n), size=n_q) for n in inp["kv_len"]]).astype(np.int32)
            q_pos[1, 0] = 1
        pooled_o = oracle.kpool_compress(inp["packed"], inp["ape"], wl.D, wl.kpool, wl.idx_dtype, wl.idx_dtype)
        S = oracle.kpool_scores(inp["q"], pooled_o, inp["w"], inp["kv_len"], q_pos, 1.0, wl.kpool,
                                wl.idx_dtype, wl.idx_dtype)
        kp = top_k // wl.kpool
        pidx = oracle.topk(S.reshape(-1, S.shape[-1]), kp).reshape(wl.B, n_q, kp)
        _, _, valid = oracle.packed_fields(inp["packed"], wl.D, wl.idx_dtype)
        want = oracle.kpool_select(S, valid, inp["kv_len"], q_pos, top_k, wl.kpool)
        tok = torch.full(want.shape, 12345, dtype=torch.int32, device="cuda")
        L.dsa_kpool_expand(dev(pidx), dev(inp["packed"], wl.idx_dtype), wl.D, tok, wl.kpool,
                           kv_len=dev(inp["kv_len"]), q_pos=None if q_pos is None else dev(q_pos))
        torch.cuda.synchronize()
        assert np.array_equal(host(tok), want), f"expansion n_q={n_q} top_k={top_k}"


def run_kpool_chain(wl, inp, fused=False):
    """compress every complete pool -> pool scores -> top-k over pools -> tokens -> attention
    (fused: the attention call makes the tokens itself; the expansion still runs for the
    token checks)."""
    L = binding()
    packed, pooled = _compress(inp, wl)
    rows, n_pool, kp = wl.B * wl.n_q, wl.n_kv // wl.kpool, wl.top_k // wl.kpool
    kv_len = dev(inp["kv_len"])
    scores = guarded((wl.B, wl.n_q, n_pool), torch.float32)
    L.dsa_kpool_index_score(dev(inp["q"], wl.idx_dtype), pooled, dev(inp["w"]), scores, wl.kpool, kv_len=kv_len,
                            scale=wl.scale)
    pidx = guarded((wl.B, wl.n_q, kp), torch.int32)
    L.dsa_topk(scores, pidx, kp, workspace=guarded_workspace(L.dsa_topk_workspace_size(rows, n_pool, kp)))
    width = wl.kpool * kp + wl.kpool - 1
    tok = guarded((wl.B, wl.n_q, width), torch.int32)
    L.dsa_kpool_expand(pidx, packed, wl.D, tok, wl.kpool, kv_len=kv_len)
    out = guarded((wl.B, wl.n_q, wl.Hm, wl.d_latent), torch.float32)
    lse = guarded((wl.B, wl.n_q, wl.Hm), torch.float32)
    ws_m = guarded_workspace(L.dsa_sparse_mla_workspace_size(wl.B, wl.n_q, wl.Hm, width, wl.d_latent, 0))
    if fused:
        L.dsa_kpool_sparse_mla_attn(dev(inp["qa"], wl.mla_dtype), dev(inp["latent"], wl.mla_dtype), pidx, packed,
                                    wl.D, wl.kpool, out, wl.d_latent, wl.sm_scale, lse=lse, kv_len=kv_len,
                                    workspace=ws_m)
    else:
        L.dsa_sparse_mla_attn(dev(inp["qa"], wl.mla_dtype), dev(inp["latent"], wl.mla_dtype), tok, out,
                              wl.d_latent, wl.sm_scale, lse=lse, kv_len=kv_len, workspace=ws_m)
    check_guards(f"{wl.name} pooled chain")
    return host(scores), host(pidx), host(tok), host(out), host(lse)


def _check_chain(wl, inp, res, seqs):
    scores, pidx, tok, out, lse = res
    kp = wl.top_k // wl.kpool
    for b in seqs:
        sl = slice(b, b + 1)
        packed_b = inp["packed"][sl]
        pooled_o = oracle.kpool_compress(packed_b, inp["ape"], wl.D, wl.kpool, wl.idx_dtype, wl.idx_dtype)
        S = oracle.kpool_scores(inp["q"][sl], pooled_o, inp["w"][sl], inp["kv_len"][sl], None, wl.scale,
                                wl.kpool, wl.idx_dtype, wl.idx_dtype)
        assert_rowwise(scores[sl], S, RTOL[wl.idx_dtype], f"{wl.name} pool scores b={b}")
        o_p = oracle.topk(S.reshape(-1, S.shape[-1]), kp).reshape(1, wl.n_q, kp)
        check_index_rule(pidx[sl], o_p, S, f"{wl.name} pools b={b}")
        _, _, valid = oracle.packed_fields(packed_b, wl.D, wl.idx_dtype)
        # the GPU's tokens are the expansion of the GPU's own pools
        S_gpu_sel = np.full_like(S, -np.inf)
        for i in range(wl.n_q):
            for p in pidx[b, i]:
                if p >= 0:
                    S_gpu_sel[0, i, p] = 1.0
        assert np.array_equal(tok[sl], oracle.kpool_select(S_gpu_sel, valid, inp["kv_len"][sl], None, wl.top_k,
                                                           wl.kpool)), f"{wl.name} tokens b={b}"
        o_out, o_lse = oracle.sparse_mla(inp["qa"][sl], inp["latent"][sl], tok[sl], wl.sm_scale, wl.d_latent,
                                         wl.mla_dtype, inp["kv_len"][sl])
        assert_rowwise(out[sl], o_out, RTOL[wl.mla_dtype], f"{wl.name} out b={b}")
        assert_rowwise(lse[sl], o_lse, RTOL[wl.mla_dtype], f"{wl.name} lse b={b}")


@pytest.mark.parametrize("fused", [False, True])
def test_chain_small(fused):
    wl = KP.scaled(B=4, n_kv=3000, top_k=256)
    inp = workloads.gen_kpool(wl, 8, hole_frac=0.05)
    _check_chain(wl, inp, run_kpool_chain(wl, inp, fused), range(wl.B))


def test_chain_full_sequences():
    """32768-token caches, top_k 2048 (512 pools, 2051 attended tokens), the decode batch of the
    bench's pooled leg cut to 4 sequences (tails of 0..3 tokens); every sequence compared."""
    wl = KP.scaled(B=4)
    inp = workloads.gen_kpool(wl, 9)
    res = run_kpool_chain(wl, inp)
    assert res[2].shape[-1] == 2051
    _check_chain(wl, inp, res, range(wl.B))


def test_chain_bench_launch_configuration():
    """The bench's pooled leg launch configuration: 32 sequences of 32768 tokens (8 MLA parts
    per query, 64-head workgroups, the fused expansion + attention call); sequences 0, 13 and
    31 (tails of 0, 1 and 3 tokens) drawn from their own streams and compared with the oracle,
    the others valid zero rows."""
    wl = KP
    sel = (0, 13, 31)
    inp = workloads.gen_kpool(wl, 11, seqs=sel)
    res = run_kpool_chain(wl, inp, fused=True)
    _check_chain(wl, inp, res, sel)


def _random_pools(wl, seed, pad_rows=()):
    """Ascending distinct pool indices per query row (any set is a valid input of the
    expansion); rows in pad_rows end with -1 padding."""
    rng = np.random.default_rng(seed)
    n_pool, kp = wl.n_kv // wl.kpool, wl.top_k // wl.kpool
    out = np.empty((wl.B * wl.n_q, kp), np.int32)
    for r in range(wl.B * wl.n_q):
        n = kp // 2 if r in pad_rows else kp
        row = np.sort(rng.choice(n_pool, size=n, replace=False)).astype(np.int32)
        out[r] = np.concatenate([row, np.full(kp - n, -1, np.int32)])
    return out.reshape(wl.B, wl.n_q, kp)


@pytest.mark.parametrize("case", ["nope", "rope_qpos", "hm32", "f32_rows", "bf16_rows", "heads_together",
                                  "rope_together", "nsplit3"])
def test_fused_equals_expand_then_attention(case):
    """dsa_kpool_sparse_mla_attn gives the bits of dsa_kpool_expand + dsa_sparse_mla_attn with
    the same parts: holes, padded pool rows, tails of 0..3 tokens, explicit positions (one
    before the first complete pool, one past the cache), 16-bit and fp32 valid entries."""
    L = binding()
    kw = dict(B=4, n_kv=1100, top_k=256)
    if case in ("rope_qpos", "rope_together"):
        kw.update(n_q=3, d_rope=64)
    if case == "hm32":
        kw.update(Hm=32)
    if case == "f32_rows":
        kw.update(idx_dtype=workloads.F32)
    if case == "bf16_rows":
        kw.update(idx_dtype=workloads.BF16)
    wl = KP.scaled(**kw)
    inp = workloads.gen_kpool(wl, 21, hole_frac=0.15)
    pidx = dev(_random_pools(wl, 22, pad_rows=(1, 2)))
    q_pos = None
    if case in ("rope_qpos", "rope_together"):
        rng = np.random.default_rng(23)
        qp = np.stack([rng.integers(0, int(n), size=wl.n_q) for n in inp["kv_len"]]).astype(np.int32)
        qp[1, 0], qp[2, 1] = 1, int(inp["kv_len"][2]) + 5
        q_pos = dev(qp)
    packed, kv_len = dev(inp["packed"], wl.idx_dtype), dev(inp["kv_len"])
    qa, lat = dev(inp["qa"], wl.mla_dtype), dev(inp["latent"], wl.mla_dtype)
    width = wl.kpool * (wl.top_k // wl.kpool) + wl.kpool - 1
    ns = 3 if case == "nsplit3" else 0
    if case in ("heads_together", "rope_together"):  # small cases split the 64 heads by themselves
        L.dsa_set_tuning("mla_head_split", 1)
    try:
        tok = torch.empty((wl.B, wl.n_q, width), dtype=torch.int32, device="cuda")
        L.dsa_kpool_expand(pidx, packed, wl.D, tok, wl.kpool, kv_len=kv_len, q_pos=q_pos)
        shape = (wl.B, wl.n_q, wl.Hm, wl.d_latent)
        out_a, out_b = (torch.full(shape, 7.0, device="cuda") for _ in range(2))
        lse_a, lse_b = (torch.full(shape[:3], 7.0, device="cuda") for _ in range(2))
        L.dsa_sparse_mla_attn(qa, lat, tok, out_a, wl.d_latent, wl.sm_scale, lse=lse_a, kv_len=kv_len, n_split=ns)
        L.dsa_kpool_sparse_mla_attn(qa, lat, pidx, packed, wl.D, wl.kpool, out_b, wl.d_latent, wl.sm_scale,
                                    lse=lse_b, kv_len=kv_len, q_pos=q_pos, n_split=ns)
        torch.cuda.synchronize()
    finally:
        L.dsa_set_tuning("mla_head_split", 0)
    assert np.array_equal(host(out_a).view(np.uint32), host(out_b).view(np.uint32)), case
    assert np.array_equal(host(lse_a).view(np.uint32), host(lse_b).view(np.uint32)), case


def test_graph_replays_match_eager():
    """The pooled chain (compression, pool scores, top-k over pools, expansion, NoPE MLA with a
    head split and a merge, and the attention call that expands the pools itself) captured in
    a HIP graph gives the eager bits on every replay, with eager work and synchronisations
    between the replays."""
    L = binding()
    wl = KP.scaled(B=3, n_kv=4100, top_k=512)
    inp = workloads.gen_kpool(wl, 12, hole_frac=0.05)
    n_pool, kp = wl.n_kv // wl.kpool, wl.top_k // wl.kpool
    packed, ape = dev(inp["packed"], wl.idx_dtype), dev(inp["ape"])
    q, w, kv_len = dev(inp["q"], wl.idx_dtype), dev(inp["w"]), dev(inp["kv_len"])
    qa, lat = dev(inp["qa"], wl.mla_dtype), dev(inp["latent"], wl.mla_dtype)
    width = wl.kpool * kp + wl.kpool - 1
    pooled = torch.empty((wl.B, n_pool, wl.D), dtype=torch.float16, device="cuda")
    scores = torch.empty((wl.B, 1, n_pool), dtype=torch.float32, device="cuda")
    pidx = torch.empty((wl.B, 1, kp), dtype=torch.int32, device="cuda")
    tok = torch.empty((wl.B, 1, width), dtype=torch.int32, device="cuda")
    out = torch.empty((wl.B, 1, wl.Hm, wl.d_latent), dtype=torch.float32, device="cuda")
    out_f = torch.empty_like(out)
    ws_t = torch.empty(max(1, L.dsa_topk_workspace_size(wl.B, n_pool, kp)), dtype=torch.uint8, device="cuda")
    ns = L.dsa_sparse_mla_num_splits(wl.B, 1, width)
    ws_m = torch.empty(max(1, L.dsa_sparse_mla_workspace_size(wl.B, 1, wl.Hm, width, wl.d_latent, ns)),
                       dtype=torch.uint8, device="cuda")

    def step():
        L.dsa_kpool_compress(packed, ape, pooled, wl.D, wl.kpool)
        L.dsa_kpool_index_score(q, pooled, w, scores, wl.kpool, kv_len=kv_len, scale=wl.scale)
        L.dsa_topk(scores, pidx, kp, workspace=ws_t)
        L.dsa_kpool_expand(pidx, packed, wl.D, tok, wl.kpool, kv_len=kv_len)
        L.dsa_sparse_mla_attn(qa, lat, tok, out, wl.d_latent, wl.sm_scale, kv_len=kv_len, n_split=ns,
                              workspace=ws_m)
        L.dsa_kpool_sparse_mla_attn(qa, lat, pidx, packed, wl.D, wl.kpool, out_f, wl.d_latent, wl.sm_scale,
                                    kv_len=kv_len, n_split=ns, workspace=ws_m)

    step()
    torch.cuda.synchronize()
    outs = (pooled, scores, pidx, tok, out, out_f)
    ref = [host(t.view(torch.int16) if t.dtype == torch.float16 else t).copy() for t in outs]
    assert np.array_equal(ref[5].view(np.uint32), ref[4].view(np.uint32)), "fused attention differs"
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in outs:
            t.fill_(0)  # eager work between replays; the replay must rewrite everything
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("pooled", "scores", "pidx", "tok", "out", "out_fused"), outs, ref):
            got = host(t.view(torch.int16) if t.dtype == torch.float16 else t)
            assert np.array_equal(got.view(np.uint32) if got.dtype == np.float32 else got,
                                  r.view(np.uint32) if r.dtype == np.float32 else r), f"replay {rep}: {name}"
