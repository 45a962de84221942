"""The oracle against its pins, and planted mistakes that the pins must catch (CPU only)."""
import math

import numpy as np
import pytest

import oracle
import workloads
from oracle_pins import (F64, pins_hadamard, pins_kpool_compress, pins_kpool_select, pins_mla, pins_prep,
                         pins_rope, pins_scores, pins_sink, pins_topk)


def test_score_pins():
    pins_scores(oracle.index_score_f64)


def test_topk_pins():
    pins_topk(oracle.topk)


def test_mla_pins():
    pins_mla(oracle.sparse_mla_f64, oracle.dense_mla_f64, oracle.sparse_mla_split_merge_f64)


# ---------------------------------------------------------------------------
# planted mistakes: each copy of an oracle step below differs from the oracle
# in one plausible way; the pins must reject every one of them.
# ---------------------------------------------------------------------------
def _score_mutant(kind):
    def fn(q, k, w, kv_len=None, q_pos=None, scale=1.0, q_dtype=F64, k_dtype=F64):
        qd = oracle.decode(q, q_dtype)
        kd = oracle.decode(k, k_dtype)
        wd = np.asarray(w, np.float64)
        B, n_q, H, D = qd.shape
        n_kv = kd.shape[1]
        kv_len_ = np.full((B,), n_kv) if kv_len is None else np.asarray(kv_len)
        q_pos_ = (kv_len_[:, None] - n_q + np.arange(n_q)[None]) if q_pos is None else np.asarray(q_pos)
        logits = np.einsum("bihd,btd->biht", qd, kd)
        if kind == "transpose_k":
            logits = np.einsum("bihd,btd->biht", qd, kd[:, :, ::-1])
        if kind == "relu_after_sum":
            s = np.maximum(np.einsum("bih,biht->bit", wd, logits), 0)
        elif kind == "relu_of_weighted":
            s = np.einsum("biht->bit", np.maximum(wd[..., None] * logits, 0))
        elif kind == "no_relu":
            s = np.einsum("bih,biht->bit", wd, logits)
        else:
            s = np.einsum("bih,biht->bit", wd, np.maximum(logits, 0))
        if kind != "no_scale":
            s = s * scale
        t = np.arange(n_kv)
        off = 1 if kind == "mask_off_by_one" else 0
        m = (t[None, None] > q_pos_[:, :, None] - off) | (t[None, None] >= kv_len_[:, None, None])
        if kind != "no_mask":
            s[m] = -np.inf
        if kind == "drop_head":
            s = s - scale * np.maximum(logits[:, :, -1], 0) * wd[:, :, -1:]
            s[m] = -np.inf
        return s
    return fn


@pytest.mark.parametrize("kind", ["transpose_k", "relu_after_sum", "relu_of_weighted", "no_relu",
                                  "no_scale", "mask_off_by_one", "no_mask", "drop_head"])
def test_score_pins_catch(kind):
    with pytest.raises(AssertionError):
        pins_scores(_score_mutant(kind))


def test_score_mutant_harness_is_faithful():
    pins_scores(_score_mutant("none"))


def _topk_mutant(kind):
    def fn(scores, top_k):
        s = np.asarray(scores, np.float32)
        out = np.full((s.shape[0], top_k), -1, np.int32)
        for r in range(s.shape[0]):
            row = s[r]
            if kind == "nan_valid":
                valid = np.nonzero(row != -np.inf)[0]
            elif kind == "neginf_valid":
                valid = np.nonzero(~np.isnan(row))[0]
            else:
                valid = np.nonzero(~np.isnan(row) & (row != -np.inf))[0]
            if kind == "ties_high_index":
                order = valid[::-1][np.argsort(-row[valid][::-1], kind="stable")]
            elif kind == "signed_zero":
                key = row[valid].copy()
                key[(key == 0) & np.signbit(key)] = -1e-30
                order = valid[np.argsort(-key, kind="stable")]
            else:
                order = valid[np.argsort(-row[valid], kind="stable")]
            K = min(top_k, valid.size)
            if kind == "k_off_by_one":
                K = max(0, K - 1)
            sel = order[:K] if kind == "rank_order" else np.sort(order[:K])
            out[r, :K] = sel
        return out
    return fn


@pytest.mark.parametrize("kind", ["nan_valid", "neginf_valid", "ties_high_index", "signed_zero",
                                  "k_off_by_one", "rank_order"])
def test_topk_pins_catch(kind):
    with pytest.raises(AssertionError):
        pins_topk(_topk_mutant(kind))


def test_topk_mutant_harness_is_faithful():
    pins_topk(_topk_mutant("none"))


def _mla_mutant(kind):
    def fn(qa, latent, idx, sm_scale, d_latent, dtype=F64, kv_len=None):
        idx = np.asarray(idx)
        B, n_q, Hm, Dc = np.shape(qa)
        n_kv = np.shape(latent)[1]
        kv_len_ = np.full((B,), n_kv) if kv_len is None else np.asarray(kv_len)
        out = np.zeros((B, n_q, Hm, d_latent))
        lse = np.zeros((B, n_q, Hm))
        for b in range(B):
            for i in range(n_q):
                sel = idx[b, i]
                if kind != "keep_padding":
                    sel = sel[(sel >= 0) & (sel < kv_len_[b])]
                rows = oracle.decode(latent[b, sel], dtype)
                qb = oracle.decode(qa[b, i], dtype)
                if rows.shape[0] == 0:
                    out[b, i] = 0
                    lse[b, i] = -np.inf
                    continue
                if kind == "no_rope":
                    z = sm_scale * (qb[:, :d_latent] @ rows[:, :d_latent].T)
                elif kind == "no_sm_scale":
                    z = qb @ rows.T
                else:
                    z = sm_scale * (qb @ rows.T)
                M = z.max(axis=1, keepdims=True)
                e = np.exp(z - M)
                l = e.sum(axis=1, keepdims=True)
                v = rows[:, Dc - d_latent:] if kind == "value_from_tail" else rows[:, :d_latent]
                out[b, i] = (e @ v) / (1.0 if kind == "no_normalise" else l)
                lse[b, i] = (0 if kind == "lse_no_max" else M[:, 0]) + np.log(l[:, 0])
        return out, lse
    return fn


@pytest.mark.parametrize("kind", ["keep_padding", "no_rope", "no_sm_scale", "value_from_tail",
                                  "no_normalise", "lse_no_max"])
def test_mla_pins_catch(kind):
    with pytest.raises(AssertionError):
        pins_mla(_mla_mutant(kind))


def test_mla_mutant_harness_is_faithful():
    pins_mla(_mla_mutant("none"))


# ---------------------------------------------------------------------------
# whole chain on the tiny fp32 workload and the generator's contract
# ---------------------------------------------------------------------------
def test_tiny_chain_and_invariants():
    wl = workloads.TINY_FP32
    inp = workloads.gen_all(wl, seed=0)
    r = oracle.dsa_step(inp, wl)
    assert r["scores"].shape == (1, 1, 256) and np.all(np.isfinite(r["scores"]))
    assert np.all(r["idx"] >= 0) and np.all(np.diff(r["idx"][0, 0]) > 0)
    # top_k >= n_kv selects every row -> dense causal attention (decode: rows 0..n_kv-1)
    full = oracle.topk(r["scores"].reshape(1, -1), wl.n_kv + 5).reshape(1, 1, -1)
    assert np.array_equal(full[0, 0, :wl.n_kv], np.arange(wl.n_kv))
    o_s, l_s = oracle.sparse_mla_f64(inp["qa"], inp["latent"], full, wl.sm_scale, wl.d_latent, wl.mla_dtype)
    o_d, l_d = oracle.dense_mla_f64(inp["qa"][:, :, :2], inp["latent"], wl.sm_scale, wl.d_latent, wl.mla_dtype)
    assert np.allclose(o_s[:, :, :2], o_d, rtol=0, atol=1e-12)


def test_generator_is_per_tensor_and_seeded():
    wl = workloads.GLM_DECODE_8K.scaled(n_kv=300, B=3)
    a = workloads.gen_all(wl, seed=7)
    b = workloads.gen_seq(wl, 7, 2)
    for name in ("q", "k", "w", "qa", "latent"):
        assert np.array_equal(a[name][2], b[name]), name
    c = workloads.gen_all(wl, seed=8)
    assert not np.array_equal(a["k"], c["k"])
    # bf16 rounding is round-to-nearest-even from float32
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e38], np.float32)
    bits = workloads.f32_to_bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.015625 and back[3] == -2.5
    # the rotation keeps the indexer statistics: std of q entries ~ 1/sqrt(128)
    q = oracle.decode(a["q"], workloads.BF16)
    assert abs(q.std() * math.sqrt(128) - 1.0) < 0.1


# ---------------------------------------------------------------------------
# indexer-input preparation
# ---------------------------------------------------------------------------
def test_prep_pins():
    pins_rope(oracle.rope_neox_f64)
    pins_hadamard(oracle.hadamard_f64)
    pins_prep(oracle.indexer_prep_f64, oracle.rope_neox_f64, oracle.cache_append)


def _rope_mutant(kind):
    def fn(x, pos, base, n_rope=64):
        x = np.asarray(x, np.float64)
        h = n_rope // 2
        i = np.arange(h, dtype=np.float64)
        expo = -1.0 * i / n_rope if kind == "half_freq" else -2.0 * i / n_rope
        p = np.asarray(pos, np.float64) + (1.0 if kind == "pos_plus_one" else 0.0)
        th = p[..., None] * np.power(base, expo)
        c, s = np.cos(th), np.sin(th)
        y = x.copy()
        if kind == "interleaved":  # GPT-J pairing (2i, 2i + 1)
            a, b = x[..., 0:n_rope:2], x[..., 1:n_rope:2]
            y[..., 0:n_rope:2] = a * c - b * s
            y[..., 1:n_rope:2] = b * c + a * s
            return y
        lo = 64 if kind == "rope_on_nope" else 0
        a, b = x[..., lo:lo + h], x[..., lo + h:lo + n_rope]
        sg = -1.0 if kind == "sign" else 1.0
        y[..., lo:lo + h] = a * c - sg * b * s
        y[..., lo + h:lo + n_rope] = b * c + sg * a * s
        return y
    return fn


@pytest.mark.parametrize("kind", ["half_freq", "pos_plus_one", "interleaved", "rope_on_nope", "sign"])
def test_rope_pins_catch(kind):
    with pytest.raises(AssertionError):
        pins_rope(_rope_mutant(kind))


def test_rope_mutant_harness_is_faithful():
    pins_rope(_rope_mutant("none"))


def _had_mutant(kind):
    def fn(x):
        x = np.asarray(x, np.float64)
        n = x.shape[-1]
        H = np.ones((1, 1))
        while H.shape[0] < n:
            H = np.block([[H, H], [H, -H]]) if kind != "kron_order" else np.block([[H, -H], [H, H]])
        if kind == "sequency":  # rows sorted by number of sign changes (Walsh order)
            H = H[np.argsort(np.sum(H[:, 1:] != H[:, :-1], axis=1), kind="stable")]
        scale = 1.0 if kind == "no_scale" else 1.0 / math.sqrt(n)
        return x @ (H * scale)
    return fn


@pytest.mark.parametrize("kind", ["kron_order", "sequency", "no_scale"])
def test_hadamard_pins_catch(kind):
    with pytest.raises(AssertionError):
        pins_hadamard(_had_mutant(kind))


def test_hadamard_mutant_harness_is_faithful():
    pins_hadamard(_had_mutant("none"))


def _prep_mutant(kind):
    def fn(q_in, k_in, pos, base, hadamard=True):
        pos = np.asarray(pos)
        def one(x, p):
            if kind == "hadamard_first" and hadamard:
                return oracle.rope_neox_f64(oracle.hadamard_f64(x), p, base)
            y = oracle.rope_neox_f64(x, p, base)
            if hadamard:
                y = oracle.hadamard_f64(y) * (math.sqrt(128.0) if kind == "unscaled" else 1.0)
            return y
        q = None if q_in is None else one(q_in, pos[:, :, None] + (1 if kind == "q_pos_shift" else 0))
        k = None if k_in is None else one(k_in, pos)
        return q, k
    return fn


@pytest.mark.parametrize("kind", ["hadamard_first", "unscaled", "q_pos_shift"])
def test_prep_pins_catch(kind):
    with pytest.raises(AssertionError):
        pins_prep(_prep_mutant(kind), oracle.rope_neox_f64, oracle.cache_append)


def test_prep_mutant_harness_is_faithful():
    pins_prep(_prep_mutant("none"), oracle.rope_neox_f64, oracle.cache_append)


def test_cache_append_catches_off_by_one():
    def bad(cache, rows, pos):
        return oracle.cache_append(cache, rows, np.asarray(pos) + 1)
    with pytest.raises(AssertionError):
        pins_prep(oracle.indexer_prep_f64, oracle.rope_neox_f64, bad)


# ---------------------------------------------------------------------------
# attention sink
# ---------------------------------------------------------------------------
def test_sink_pins():
    pins_sink(oracle.index_score_sink, oracle.index_score, oracle.topk)


def _sink_mutant(kind):
    def fn(q, k, w, kv_len, q_pos, scale, qd, kd, sink_start, n_sink, boost):
        S = oracle.index_score(q, k, w, kv_len, q_pos, scale, qd, kd)
        if n_sink <= 0:
            return S
        B, n_q, n_kv = S.shape
        start = np.zeros(B, np.int64) if (sink_start is None or kind == "global") else np.asarray(sink_start)
        t = np.arange(n_kv)
        for b in range(B):
            hi = start[b] + n_sink + (1 if kind == "one_more" else 0)
            in_sink = (t >= start[b]) & (t < hi)
            if kind == "boost_masked":
                S[b][:, in_sink] = np.float32(boost)
            else:
                S[b][:, in_sink] = S[b][:, in_sink] + np.float32(boost)
        return S
    return fn


@pytest.mark.parametrize("kind", ["global", "one_more", "boost_masked"])
def test_sink_pins_catch(kind):
    with pytest.raises(AssertionError):
        pins_sink(_sink_mutant(kind), oracle.index_score, oracle.topk)


def test_sink_mutant_harness_is_faithful():
    pins_sink(_sink_mutant("none"), oracle.index_score, oracle.topk)


# ---------------------------------------------------------------------------
# pooled indexer
# ---------------------------------------------------------------------------
def test_kpool_compress_pins():
    pins_kpool_compress(oracle.kpool_compress_f64)


def _compress_mutant(kind):
    def fn(packed, ape, D, kpool, row_dtype):
        k, gate, valid = oracle.packed_fields(packed, D, row_dtype)
        ape = np.asarray(ape, np.float64)
        B, n_kv = valid.shape
        n_pool = n_kv // kpool
        off = 1 if kind == "pool_offset" else 0
        out = np.zeros((B, n_pool, D))
        for b in range(B):
            for p in range(n_pool):
                toks = [min(kpool * p + j + off, n_kv - 1) for j in range(kpool)]
                if kind != "include_invalid":
                    toks = [t for t in toks if valid[b, t]]
                if not toks:
                    continue
                if kind == "no_ape":
                    a = np.stack([gate[b, t] for t in toks])
                elif kind == "ape_by_pool":
                    a = np.stack([gate[b, t] + ape[p % kpool] for t in toks])
                else:
                    a = np.stack([gate[b, t] + ape[t - kpool * p - off] for t in toks])
                ax = 1 if kind == "softmax_over_dims" else 0
                e = np.exp(a - a.max(axis=ax, keepdims=True))
                wts = e if kind == "unnormalised" else e / e.sum(axis=ax, keepdims=True)
                out[b, p] = (wts * np.stack([k[b, t] for t in toks])).sum(axis=0)
        return out
    return fn


@pytest.mark.parametrize("kind", ["pool_offset", "include_invalid", "no_ape", "ape_by_pool",
                                  "softmax_over_dims", "unnormalised"])
def test_kpool_compress_pins_catch(kind):
    with pytest.raises(AssertionError):
        pins_kpool_compress(_compress_mutant(kind))


def test_kpool_compress_mutant_harness_is_faithful():
    pins_kpool_compress(_compress_mutant("none"))


def test_kpool_select_pins():
    pins_kpool_select(oracle.kpool_select, oracle.kpool_scores, oracle.dense_mla_f64, oracle.sparse_mla_f64)


def _kscores_mutant(kind):
    def fn(q, pooled, w, kv_len, q_pos, scale, kpool, qd, kd):
        n_q = np.asarray(q).shape[1]
        pl, pp = oracle.kpool_positions(kv_len, q_pos, n_q, kpool)
        if kind == "visible_floor":
            pp = np.asarray(q_pos) // kpool
        if kind == "len_ceil":
            pl = (np.asarray(kv_len) + kpool - 1) // kpool
        return oracle.index_score(q, pooled, w, pl, pp, scale, qd, kd)
    return fn


def _select_mutant(kind):
    def fn(S, valid, kv_len, q_pos, top_k, kpool):
        if kind == "pools_as_tokens":
            return oracle.kpool_select(S, valid, kv_len, q_pos, top_k * kpool, kpool)
        out = oracle.kpool_select(S, valid, kv_len, q_pos, top_k, kpool)
        kp = top_k // kpool
        B, n_q, _ = out.shape
        for b in range(B):
            for i in range(n_q):
                pos = int(np.asarray(q_pos)[b, i])
                if kind == "no_tail":
                    out[b, i, kpool * kp:] = -1
                if kind == "tail_no_lower_bound":  # the tail rule without t >= 0
                    t0 = kpool * ((pos + 1) // kpool)
                    for j in range(kpool - 1):
                        t = t0 + j
                        if t <= pos and t < int(np.asarray(kv_len)[b]) and valid[b, t]:
                            out[b, i, kpool * kp + j] = t
                if kind == "tail_floor":
                    t0 = kpool * (pos // kpool)
                    for j in range(kpool - 1):
                        t = t0 + j
                        out[b, i, kpool * kp + j] = t if (t <= pos and valid[b, t]) else -1
                if kind == "keep_invalid":
                    row = out[b, i]
                    sel = row[:kpool * kp]
                    pools = sorted({int(t) // kpool for t in sel if t >= 0})
                    full = [t for p in pools for t in range(kpool * p, kpool * p + kpool)]
                    row[:len(full)] = full
        return out
    return fn


@pytest.mark.parametrize("kind", ["visible_floor", "len_ceil"])
def test_kpool_score_pins_catch(kind):
    with pytest.raises(AssertionError):
        pins_kpool_select(oracle.kpool_select, _kscores_mutant(kind), oracle.dense_mla_f64, oracle.sparse_mla_f64)


@pytest.mark.parametrize("kind", ["pools_as_tokens", "no_tail", "tail_floor", "keep_invalid",
                                  "tail_no_lower_bound"])
def test_kpool_select_pins_catch(kind):
    with pytest.raises(AssertionError):
        pins_kpool_select(_select_mutant(kind), oracle.kpool_scores, oracle.dense_mla_f64, oracle.sparse_mla_f64)


def test_kpool_mutant_harness_is_faithful():
    pins_kpool_select(_select_mutant("none"), _kscores_mutant("none"), oracle.dense_mla_f64, oracle.sparse_mla_f64)


def test_kpool_generator_sequence_subset():
    """Sequences drawn alone equal the same sequences of the full draw; the others are zero rows
    that keep their valid entries (the GPU tests use this to run the full batch shape)."""
    wl = workloads.KPOOL_DECODE_32K.scaled(B=5, n_kv=64, top_k=16)
    a = workloads.gen_kpool(wl, 3, hole_frac=0.1, seqs=(1, 4))
    b = workloads.gen_kpool(wl, 3, hole_frac=0.1)
    for name in ("packed", "q", "w", "qa", "latent"):
        assert a[name].dtype == b[name].dtype
        assert np.array_equal(a[name][[1, 4]], b[name][[1, 4]]), name
        others = a[name][[0, 2, 3]]
        if name == "packed":
            assert not others[..., :-1].any()
            valid = oracle.decode(others[..., -1], wl.idx_dtype)
            assert np.array_equal(valid, (np.arange(64)[None] < a["kv_len"][[0, 2, 3], None]).astype(float))
        else:
            assert not others.any(), name
    for name in ("ape", "kv_len", "q_pos"):
        assert np.array_equal(a[name], b[name])


# ---------------------------------------------------------------------------
# storage rounding (the expected values of the indexer-prep and pool-compression parity tests)
# ---------------------------------------------------------------------------
from oracle_pins import pins_encode  # noqa: E402


def test_encode_pins():
    pins_encode(oracle.encode)


def _encode_mutant(kind):
    def away(x32, dtype):
        """the next 16-bit code away from zero of the code that truncation gives"""
        return _toward_zero(x32, dtype) + np.uint16(1)

    def _toward_zero(x32, dtype):
        if dtype == oracle.BF16:
            return (x32.view(np.uint32) >> 16).astype(np.uint16)
        r = x32.astype(np.float16)
        over = np.abs(r.astype(np.float64)) > np.abs(x32.astype(np.float64))
        r[over] = np.nextafter(r[over], np.float16(0))
        return r.view(np.uint16)

    def fn(x64, dtype):
        x64 = np.asarray(x64, np.float64)
        if dtype == oracle.F32 or kind == "none":
            return oracle.encode(x64, dtype)
        x32 = x64.astype(np.float32)
        if kind == "truncate":
            out = _toward_zero(x32, dtype)
        elif kind == "half_up":  # ties away from zero
            lo = _toward_zero(x32, dtype)
            hi = away(x32, dtype)
            dlo = np.abs(np.abs(x32.astype(np.float64)) - np.abs(oracle.decode(lo, dtype)))
            dhi = np.abs(np.abs(oracle.decode(hi, dtype)) - np.abs(x32.astype(np.float64)))
            out = np.where(dhi <= dlo, hi, lo)
        elif kind == "skip_f32":  # rounds the float64 value straight to 16 bits
            lo = _toward_zero(x32, dtype)
            sign = lo & np.uint16(0x8000)
            mag = (lo & np.uint16(0x7FFF)).astype(np.int64)
            # float32 may have lost the float64 value's low bits: take the neighbouring
            # magnitudes of that code and compare them with the float64 value itself
            cands = np.stack([np.maximum(mag - 1, 0), mag, mag + 1]).astype(np.uint16)
            d = np.abs(oracle.decode(cands, dtype) - np.abs(x64)[None])
            best = d.min(axis=0, keepdims=True)
            even = (d == best) & ((cands & 1) == 0)
            pick = np.where(even.any(axis=0), even.argmax(axis=0), (d == best).argmax(axis=0))
            out = np.take_along_axis(cands, pick[None], 0)[0] | sign
            big = np.abs(x64) >= float(np.finfo(np.float16).max if dtype == oracle.F16 else 3.38e38)
            out[big] = oracle.encode(x64[big], dtype)  # overflow as the oracle: only the rounding step differs
        nan = np.isnan(x64)
        out = out.copy()
        out[nan] = 0x7FC0 if dtype == oracle.BF16 else 0x7E00
        return out
    return fn


@pytest.mark.parametrize("kind", ["truncate", "half_up", "skip_f32"])
def test_encode_pins_catch(kind):
    with np.errstate(over="ignore", invalid="ignore"):
        with pytest.raises(AssertionError):
            pins_encode(_encode_mutant(kind))


def test_encode_mutant_harness_is_faithful():
    pins_encode(_encode_mutant("none"))
