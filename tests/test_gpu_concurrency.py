"""Calls from several host threads at once, each on its own stream with its own outputs and
workspaces: the library keeps no per-call state outside its arguments (the tuning switches are
process-wide and only read), so every thread's results equal, bit for bit, those of the same
calls made one after the other on one stream."""
import threading

import pytest

import workloads
from gpu_util import binding, to_device_inputs

pytestmark = pytest.mark.gpu
import torch  # noqa: E402


class _Step:
    """One fused score -> top-k call and one attention call over a workload's inputs, with
    outputs and workspaces of its own."""

    def __init__(self, L, wl, seed):
        self.L, self.wl = L, wl
        self.d = to_device_inputs(wl, workloads.gen_all(wl, seed))
        B, n_q = wl.B, wl.n_q
        self.idx = torch.empty((B, n_q, wl.top_k), dtype=torch.int32, device="cuda")
        self.scores = torch.empty((B, n_q, wl.n_kv), dtype=torch.float32, device="cuda")
        self.out = torch.empty((B, n_q, wl.Hm, wl.d_latent), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((B, n_q, wl.Hm), dtype=torch.float32, device="cuda")
        self.ws_f = torch.empty(max(1, L.dsa_index_score_topk_workspace_size(B, n_q, wl.H, wl.D, wl.n_kv, wl.top_k,
                                                                            wl.idx_dtype)),
                                dtype=torch.uint8, device="cuda")
        self.ws_m = torch.empty(max(1, L.dsa_sparse_mla_workspace_size(B, n_q, wl.Hm, wl.top_k, wl.d_latent, 0)),
                                dtype=torch.uint8, device="cuda")

    def run(self, stream=None):
        L, wl, d = self.L, self.wl, self.d
        L.dsa_index_score_topk(d["q"], d["k"], d["w"], self.idx, wl.top_k, scores=self.scores, kv_len=d["kv_len"],
                               scale=wl.scale, workspace=self.ws_f, stream=stream)
        L.dsa_sparse_mla_attn(d["qa"], d["latent"], self.idx, self.out, wl.d_latent, wl.sm_scale, lse=self.lse,
                              kv_len=d["kv_len"], workspace=self.ws_m, stream=stream)

    def results(self):
        return [t.clone() for t in (self.scores, self.idx, self.out, self.lse)]


def test_threads_on_their_own_streams_match_serial_calls():
    L = binding()
    shapes = [workloads.GLM_DECODE_8K.scaled(B=2, n_kv=6000, top_k=1024),
              workloads.GLM_DECODE_8K.scaled(B=4, n_kv=3000, top_k=512, Hm=32),
              workloads.LONG_DECODE_128K.scaled(B=2, n_kv=9000),
              workloads.CHUNKED_PREFILL_16K.scaled(n_q=24, n_kv=800, q_pos_start=None, top_k=256)]
    steps = [_Step(L, wl, 40 + i) for i, wl in enumerate(shapes)]
    want = []
    for s in steps:  # serial reference on the current stream
        s.run()
        torch.cuda.synchronize()
        want.append(s.results())
    errors = []

    def worker(i):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for _ in range(20):
                    steps[i].run(stream)
            stream.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(steps))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, s in enumerate(steps):
        got = s.results()
        for g, w, name in zip(got, want[i], ("scores", "idx", "out", "lse")):
            same = torch.equal(g.view(torch.int32), w.view(torch.int32)) if g.dtype == torch.float32 else \
                torch.equal(g, w)
            assert same, f"thread {i}: {name} differs from the serial call"
