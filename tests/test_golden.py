"""Values the pages print, stored under tests/golden/ with their citations, checked against
the library's host logic and the oracle (CPU only)."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
GOLDEN = os.path.join(ROOT, "tests", "golden")

import oracle  # noqa: E402
import workloads  # noqa: E402


def _read(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split(":")
            out[k.strip()] = int(v)
    return out


def test_indexshare_counts():
    g = _read("indexshare_glm52_layers.txt")
    from sparse_attention_10_amd import dsa
    full = [il for il in range(g["layers"]) if dsa.lib.dsa_layer_computes_topk(il) == 1]
    assert len(full) == g["full_layers"]
    assert g["layers"] - len(full) == g["shared_layers"]
    # every shared layer takes the selection of the most recent full layer before it
    for il in range(g["layers"]):
        src = dsa.lib.dsa_topk_source_layer(il)
        assert src in full and src <= il and not any(src < f <= il for f in full)


def test_kpool_shapes():
    g = _read("kpool_glm5next_shapes.txt")
    wl = workloads.KPOOL_DECODE_32K
    assert (wl.H, wl.D, wl.top_k, wl.kpool, wl.d_latent, wl.d_rope) == (
        g["indexer_heads"], g["indexer_dim"], g["top_k_tokens"], g["kpool"], g["latent_dim"], 0)
    assert 2 * wl.D + 1 == g["packed_row_values"]
    assert g["kpool"] - 1 == g["max_tail"]
    # the oracle's selection of top_k / kpool pools plus the tail has the printed width
    n_pool = 16
    S = np.zeros((1, 1, n_pool))
    valid = np.ones((1, n_pool * g["kpool"]))
    sel = oracle.kpool_select(S, valid, np.array([n_pool * g["kpool"]], np.int32), None,
                              g["top_k_tokens"], g["kpool"])
    assert sel.shape[-1] == g["attended_width"]
