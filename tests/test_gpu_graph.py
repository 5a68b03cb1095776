"""Run calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The run calls allocate nothing, never synchronise and launch only kernels
(no memset nodes), so a serving loop can capture them.  Each test captures
one call on static buffers, then replays the graph several times with
eager work in between (new inputs copied into the static buffers, a host
synchronisation) and checks every replay bit for bit against an eager call
on the same inputs.
"""

import sys

import pytest
import torch

from workloads import make_sparse_workload, make_workload

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def mla():
    import paged_mla_decode_05_amd as m

    m.load_library()
    assert torch.cuda.is_available()
    return m


def _replay_and_check(graph, set_inputs, eager, outputs, rounds=3):
    for k in range(rounds):
        set_inputs(k)
        torch.cuda.synchronize()
        ref = [t.clone() for t in eager()]
        torch.cuda.synchronize()
        for t in outputs:
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(outputs, ref):
            assert torch.equal(got, want), f"replay {k} differs from the eager call"


def test_split_decode_graph_replays(mla):
    say("graph: bf16 decode with forced splits (attention + combine)")
    w = make_workload(kv_lens=[900, 130, 2000], heads=128, page_size=64, seed=90, device=DEV)
    plan = mla.mla_plan_create(mla.MLA_KIND_DECODE, w.batch, w.num_heads, w.page_size, w.num_pages, w.kv_len,
                               w.kv_indptr, force_splits=3)
    assert plan.num_split_groups > 0
    ip, ix = w.kv_indptr.to(DEV), w.kv_indices.to(DEV)
    qn, qp = w.q_nope.clone(), w.q_pe.clone()
    out = torch.empty((w.batch, w.num_heads, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((w.batch, w.num_heads), dtype=torch.float32, device=DEV)
    ws = plan.workspace(DEV)  # uploaded before capture
    torch.cuda.synchronize()

    def call(o, l):
        return mla.mla_decode(plan, qn, qp, w.ckv, w.kpe, ip, ix, w.sm_scale, out=o, lse=l, workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(out, lse)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, lse)
    gen = torch.Generator(device=DEV).manual_seed(5)

    def set_inputs(k):
        qn.copy_(torch.randn(qn.shape, generator=gen, device=DEV).to(torch.bfloat16))
        qp.copy_(torch.randn(qp.shape, generator=gen, device=DEV).to(torch.bfloat16))

    out_e = torch.empty_like(out)
    lse_e = torch.empty_like(lse)
    _replay_and_check(g, set_inputs, lambda: call(out_e, lse_e), [out, lse])


def test_sparse_decode_graph_replays(mla):
    say("graph: token-sparse fp8 decode (list compaction + attention + combine)")
    w = make_sparse_workload(kv_lens=[1500, 700], s_q=2, heads=128, topk=512, page_size=64, seed=91,
                             invalid_frac=0.2, sink=True, device=DEV)
    plan = mla.mla_sparse_plan_create(w.tokens, w.num_heads, w.num_slots, w.topk,
                                      kv_format=mla.MLA_KV_FP8_E4M3_T128, force_splits=2)
    idx = w.indices.to(DEV)
    sink = w.attn_sink.to(DEV)
    q = w.q.clone()
    out = torch.empty((w.tokens, w.num_heads, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((w.tokens, w.num_heads), dtype=torch.float32, device=DEV)
    mx = torch.empty_like(lse)
    ws = plan.workspace(DEV)
    torch.cuda.synchronize()

    def call(o, l, m):
        return mla.mla_sparse_decode_fp8(plan, q, w.kv_fp8, idx, w.sm_scale, attn_sink=sink, out=o, lse=l,
                                         max_logits=m, workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(out, lse, mx)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, lse, mx)
    perm_gen = torch.Generator().manual_seed(6)

    def set_inputs(k):
        # new lists (a permutation of each row's entries) and a new query
        p = torch.randperm(w.topk, generator=perm_gen)
        idx.copy_(w.indices[:, p].to(DEV))
        q.copy_(torch.roll(w.q, shifts=k + 1, dims=0))

    out_e, lse_e, mx_e = torch.empty_like(out), torch.empty_like(lse), torch.empty_like(mx)
    _replay_and_check(g, set_inputs, lambda: call(out_e, lse_e, mx_e), [out, lse, mx])
