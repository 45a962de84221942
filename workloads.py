"""Seeded synthetic inputs for the DSA decode/prefill hot path.

This module only draws random numbers and rounds them to storage dtypes. It
holds none of the method's arithmetic (no scoring, selection or attention), so
both the CPU oracle and the HIP path can take their inputs from here.

Every tensor has its own counter-derived stream: numpy's PCG64 seeded with
``SeedSequence([seed, workload_id, sequence, tensor_tag])``. A sequence's
caches therefore do not depend on how many other sequences are generated or in
which order, and one sequence of a big batch can be regenerated alone.

Recipe (shapes follow the GLM-5.2 DSA shape: 32 indexer heads x 128, top-k
2048, 64 MLA heads over a 512 + 64 latent row; see the ds4 "hy3: Metal decode
path" PR, GLM loader shape section, and the ik_llama_opt "DSA lightning
indexer" sub-commit):

* indexer query and keys: N(0, 1) / sqrt(128), drawn in float64. For the
  bf16/f16 workloads both are rotated by the orthonormal Sylvester Hadamard
  matrix H_128 / sqrt(128) in float64 before rounding, as the cached indexer
  keys are stored rotated (ik_llama_opt "decode-correct via persistent
  indexer-K cache" sub-commit). An orthonormal rotation of an i.i.d. Gaussian
  vector is again i.i.d. Gaussian, so the rotation changes values, not their
  distribution.
* per-head indexer weights: U(0, 1), divided by sqrt(32) for the 32-head
  workloads; kept in fp32.
* absorbed MLA query: N(0, 1). Latent cache rows (576 wide): N(0, 1) for the
  tiny fp32 workload, N(0, 0.5) (standard deviation 0.5) otherwise.
* rounding: float64 -> float32 (round to nearest even) -> bf16 or f16 (round
  to nearest even). bf16/f16 tensors are returned as uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np
import scipy.linalg

# dtype codes shared with the C ABI (plain integers; they carry no arithmetic)
F32, BF16, F16 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", BF16: "bf16", F16: "f16"}

# tensor tags for the per-tensor streams
_TAG_Q, _TAG_K, _TAG_W, _TAG_QA, _TAG_LAT = 1, 2, 3, 4, 5
_TAG_PQ, _TAG_PK, _TAG_PLAT = 6, 7, 8
_TAG_KPK, _TAG_GATE, _TAG_APE, _TAG_HOLE = 9, 10, 11, 12


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # stream id of this workload
    B: int                   # sequences
    n_q: int                 # queries per sequence
    H: int                   # indexer heads
    D: int                   # indexer head dim
    n_kv: int                # cached rows per sequence
    top_k: int
    Hm: int                  # MLA heads
    d_latent: int
    d_rope: int
    idx_dtype: int           # indexer q / k dtype
    mla_dtype: int           # absorbed query / latent dtype
    rotate: bool             # Hadamard-rotate indexer q and k
    w_scale: float           # per-head weights ~ U(0,1) * w_scale
    latent_std: float
    scale: float = 1.0       # indexer score scale (applied after the head sum)
    sm_scale: float = 1.0 / 16.0   # 1/sqrt(192 + 64)
    q_pos_start: Optional[int] = None  # causal prefill: query i sits at q_pos_start + i
    kpool: int = 0           # pooled indexer: tokens per pool (0: the per-token indexer)

    @property
    def Dc(self) -> int:
        return self.d_latent + self.d_rope

    @property
    def rows(self) -> int:
        return self.B * self.n_q

    def q_pos(self) -> np.ndarray:
        """Cache position of each query, [B][n_q] int32 (decode: the last n_q rows)."""
        start = self.n_kv - self.n_q if self.q_pos_start is None else self.q_pos_start
        p = start + np.arange(self.n_q, dtype=np.int64)
        return np.broadcast_to(p, (self.B, self.n_q)).astype(np.int32).copy()

    def kv_len(self) -> np.ndarray:
        return np.full((self.B,), self.n_kv, dtype=np.int32)

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the DSA hot path, named by what they are.
TINY_FP32 = Workload("tiny_fp32_decode_256", 0, B=1, n_q=1, H=4, D=128, n_kv=256, top_k=64,
                     Hm=8, d_latent=512, d_rope=64, idx_dtype=F32, mla_dtype=F32,
                     rotate=False, w_scale=1.0, latent_std=1.0)
GLM_DECODE_8K = Workload("glm_decode_b1_8k", 1, B=1, n_q=1, H=32, D=128, n_kv=8192, top_k=2048,
                         Hm=64, d_latent=512, d_rope=64, idx_dtype=BF16, mla_dtype=BF16,
                         rotate=True, w_scale=1.0 / math.sqrt(32.0), latent_std=0.5)
BATCHED_DECODE_32K = Workload("batched_decode_b32_32k", 2, B=32, n_q=1, H=32, D=128, n_kv=32768,
                              top_k=2048, Hm=64, d_latent=512, d_rope=64, idx_dtype=BF16,
                              mla_dtype=BF16, rotate=True, w_scale=1.0 / math.sqrt(32.0),
                              latent_std=0.5)
CHUNKED_PREFILL_16K = Workload("chunked_prefill_4096_after_12288", 3, B=1, n_q=4096, H=32, D=128,
                               n_kv=16384, top_k=2048, Hm=64, d_latent=512, d_rope=64,
                               idx_dtype=BF16, mla_dtype=BF16, rotate=True,
                               w_scale=1.0 / math.sqrt(32.0), latent_std=0.5, q_pos_start=12288)
LONG_DECODE_128K = Workload("long_decode_b8_128k", 4, B=8, n_q=1, H=32, D=128, n_kv=131072,
                            top_k=2048, Hm=64, d_latent=512, d_rope=64, idx_dtype=F16,
                            mla_dtype=BF16, rotate=True, w_scale=1.0 / math.sqrt(32.0),
                            latent_std=0.5)

WORKLOADS = {w.name: w for w in (TINY_FP32, GLM_DECODE_8K, BATCHED_DECODE_32K,
                                 CHUNKED_PREFILL_16K, LONG_DECODE_128K)}


def _rng(seed: int, wid: int, seq: int, tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, wid, seq, tag])))


def hadamard128() -> np.ndarray:
    """Orthonormal Sylvester Hadamard matrix of order 128 (float64)."""
    return scipy.linalg.hadamard(128).astype(np.float64) / math.sqrt(128.0)


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest even); NaN kept quiet. Returns uint16."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(x32)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def round_to(x64: np.ndarray, dtype: int) -> np.ndarray:
    """float64 -> storage representation: float32 array, or uint16 bits for bf16/f16."""
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == F32:
        return x32
    if dtype == BF16:
        return f32_to_bf16_bits(x32)
    if dtype == F16:
        return x32.astype(np.float16).view(np.uint16)
    raise ValueError(f"unknown dtype code {dtype}")


def _draw_normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return rng.standard_normal(shape) * std


def gen_seq(wl: Workload, seed: int, b: int, parts=("q", "k", "w", "qa", "latent")) -> Dict[str, np.ndarray]:
    """Inputs of one sequence b (every tensor has its own stream)."""
    out: Dict[str, np.ndarray] = {}
    rot = hadamard128() if (wl.rotate and wl.D == 128) else None
    s = 1.0 / math.sqrt(wl.D)
    if "q" in parts:
        q = _draw_normal(_rng(seed, wl.wid, b, _TAG_Q), (wl.n_q, wl.H, wl.D), s)
        if rot is not None:
            q = q @ rot
        out["q"] = round_to(q, wl.idx_dtype)
    if "k" in parts:
        k = _draw_normal(_rng(seed, wl.wid, b, _TAG_K), (wl.n_kv, wl.D), s)
        if rot is not None:
            k = k @ rot
        out["k"] = round_to(k, wl.idx_dtype)
    if "w" in parts:
        w = _rng(seed, wl.wid, b, _TAG_W).random((wl.n_q, wl.H)) * wl.w_scale
        out["w"] = w.astype(np.float32)
    if "qa" in parts:
        qa = _draw_normal(_rng(seed, wl.wid, b, _TAG_QA), (wl.n_q, wl.Hm, wl.Dc), 1.0)
        out["qa"] = round_to(qa, wl.mla_dtype)
    if "latent" in parts:
        lat = _draw_normal(_rng(seed, wl.wid, b, _TAG_LAT), (wl.n_kv, wl.Dc), wl.latent_std)
        out["latent"] = round_to(lat, wl.mla_dtype)
    return out


def gen_all(wl: Workload, seed: int, parts=("q", "k", "w", "qa", "latent")) -> Dict[str, np.ndarray]:
    """Inputs of every sequence stacked on a leading batch axis.

    q [B][n_q][H][D], k [B][n_kv][D], w [B][n_q][H] f32, qa [B][n_q][Hm][Dc],
    latent [B][n_kv][Dc], plus kv_len [B] and q_pos [B][n_q] int32.
    """
    per = [gen_seq(wl, seed, b, parts) for b in range(wl.B)]
    out = {name: np.stack([p[name] for p in per]) for name in per[0]}
    out["kv_len"] = wl.kv_len()
    out["q_pos"] = wl.q_pos()
    return out


def gen_prep(wl: Workload, seed: int) -> Dict[str, np.ndarray]:
    """Inputs of the indexer-input preparation for the workload's new tokens (its queries):
    fp32 indexer query and key rows before rope and rotation, drawn like the cached ones
    (N(0, 1) / sqrt(128)); the new 576-wide latent rows in the MLA dtype; the positions
    (the queries' cache positions). q_in [B][n_q][H][128], k_in [B][n_q][128],
    latent_in [B][n_q][Dc], pos [B][n_q] int32."""
    s = 1.0 / math.sqrt(wl.D)
    q = np.stack([_draw_normal(_rng(seed, wl.wid, b, _TAG_PQ), (wl.n_q, wl.H, wl.D), s) for b in range(wl.B)])
    k = np.stack([_draw_normal(_rng(seed, wl.wid, b, _TAG_PK), (wl.n_q, wl.D), s) for b in range(wl.B)])
    lat = np.stack([_draw_normal(_rng(seed, wl.wid, b, _TAG_PLAT), (wl.n_q, wl.Dc), wl.latent_std)
                    for b in range(wl.B)])
    return {"q_in": q.astype(np.float32), "k_in": k.astype(np.float32),
            "latent_in": round_to(lat, wl.mla_dtype), "pos": wl.q_pos()}


# Pooled-indexer decode at the GLM-5.3-Flash DSA shape (vllm-rdna "Glm5Next" PR, architecture
# section: 32 indexer heads x 128, top-k 2048, pools of 4 tokens; MLA without RoPE, 64 heads
# over the 512-wide latent), batched like the 32K decode workload.
KPOOL_DECODE_32K = Workload("kpool_decode_b32_32k", 5, B=32, n_q=1, H=32, D=128, n_kv=32768,
                            top_k=2048, Hm=64, d_latent=512, d_rope=0, idx_dtype=F16,
                            mla_dtype=BF16, rotate=False, w_scale=1.0 / math.sqrt(32.0),
                            latent_std=0.5, kpool=4)


def gen_kpool(wl: Workload, seed: int, hole_frac: float = 0.0, kv_len=None, seqs=None) -> Dict[str, np.ndarray]:
    """Inputs of the pooled-indexer chain. Packed indexer rows [B][n_kv][2 D + 1] in the
    indexer dtype: k ~ N(0, 1) / sqrt(D), gate ~ N(0, 1), valid = 1 for written tokens
    (t < kv_len[b]) and 0 beyond, and 0 for a hole_frac fraction of written tokens when asked;
    ape [kpool][D] fp32 ~ N(0, 1); indexer q [B][n_q][H][D] ~ N(0, 1) / sqrt(D); w ~ U(0, 1)
    * w_scale; absorbed query [B][n_q][Hm][d_latent] ~ N(0, 1); latent [B][n_kv][d_latent] ~
    N(0, latent_std). kv_len defaults to n_kv - (b % kpool), so the sequences end with tails of
    0 .. kpool - 1 tokens; q_pos = kv_len - n_q + i. With seqs given, only those sequences are
    drawn (each from its own streams, so they equal the full draw); the others hold zero keys,
    gates, queries, weights and latent rows with the same valid entries."""
    D, kp = wl.D, wl.kpool
    if kv_len is None:
        kv_len = np.array([wl.n_kv - (b % kp) for b in range(wl.B)], np.int32)
    kv_len = np.asarray(kv_len, np.int32)
    s = 1.0 / math.sqrt(D)
    packed, q, w, qa, lat = [], [], [], [], []
    def zeros(shape, dtype):  # the storage form of 0.0: 0.0f, or all-zero 16-bit patterns
        return np.zeros(shape, np.float32 if dtype == F32 else np.uint16)

    for b in range(wl.B):
        if seqs is not None and b not in seqs:
            pk = zeros((wl.n_kv, 2 * D + 1), wl.idx_dtype)
            pk[:, 2 * D] = round_to((np.arange(wl.n_kv) < kv_len[b]).astype(np.float64), wl.idx_dtype)
            packed.append(pk)
            q.append(zeros((wl.n_q, wl.H, D), wl.idx_dtype))
            w.append(np.zeros((wl.n_q, wl.H), np.float32))
            qa.append(zeros((wl.n_q, wl.Hm, wl.Dc), wl.mla_dtype))
            lat.append(zeros((wl.n_kv, wl.Dc), wl.mla_dtype))
            continue
        k = _draw_normal(_rng(seed, wl.wid, b, _TAG_KPK), (wl.n_kv, D), s)
        gate = _draw_normal(_rng(seed, wl.wid, b, _TAG_GATE), (wl.n_kv, D), 1.0)
        valid = (np.arange(wl.n_kv) < kv_len[b]).astype(np.float64)
        if hole_frac > 0:
            valid[_rng(seed, wl.wid, b, _TAG_HOLE).random(wl.n_kv) < hole_frac] = 0.0
        packed.append(round_to(np.concatenate([k, gate, valid[:, None]], axis=1), wl.idx_dtype))
        q.append(round_to(_draw_normal(_rng(seed, wl.wid, b, _TAG_Q), (wl.n_q, wl.H, D), s), wl.idx_dtype))
        w.append((_rng(seed, wl.wid, b, _TAG_W).random((wl.n_q, wl.H)) * wl.w_scale).astype(np.float32))
        qa.append(round_to(_draw_normal(_rng(seed, wl.wid, b, _TAG_QA), (wl.n_q, wl.Hm, wl.Dc), 1.0), wl.mla_dtype))
        lat.append(round_to(_draw_normal(_rng(seed, wl.wid, b, _TAG_LAT), (wl.n_kv, wl.Dc), wl.latent_std),
                            wl.mla_dtype))
    ape = _draw_normal(_rng(seed, wl.wid, 0, _TAG_APE), (kp, D), 1.0).astype(np.float32)
    q_pos = (kv_len[:, None].astype(np.int64) - wl.n_q + np.arange(wl.n_q)[None]).astype(np.int32)
    return {"packed": np.stack(packed), "ape": ape, "q": np.stack(q), "w": np.stack(w),
            "qa": np.stack(qa), "latent": np.stack(lat), "kv_len": kv_len, "q_pos": q_pos}


def random_scores(rows: int, n: int, seed: int, tie_frac: float = 0.0, neg_inf_frac: float = 0.0,
                  nan_frac: float = 0.0, quantize: Optional[float] = None) -> np.ndarray:
    """fp32 score rows for selection tests: N(0,1), optionally coarsened so that
    ties are frequent, with a fraction of -inf and NaN entries and signed zeros."""
    rng = _rng(seed, 99, rows, n)
    s = rng.standard_normal((rows, n))
    if quantize:
        s = np.round(s / quantize) * quantize
    s = s.astype(np.float32)
    if tie_frac > 0:
        m = rng.random((rows, n)) < tie_frac
        s[m] = np.float32(0.5)
    z = rng.random((rows, n)) < 0.01
    s[z] = np.where(rng.random(int(z.sum())) < 0.5, np.float32(0.0), np.float32(-0.0))
    if neg_inf_frac > 0:
        s[rng.random((rows, n)) < neg_inf_frac] = -np.inf
    if nan_frac > 0:
        s[rng.random((rows, n)) < nan_frac] = np.nan
    return s
