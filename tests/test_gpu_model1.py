"""GPU parity of the MODEL1 record path (FlashMLA FP8 section,
MODEL1_FP8Sparse): the record expansion is byte work and must equal the
oracle's dequantisation bit for bit (bf16 bits, signed zeros included);
decode over the expanded rows and queries, through the concatenated-layout
entry point, is checked against the MODEL1 oracle (q.k over 512 dims,
V = the 448 NoPE dims) with the bf16 tolerances, since both sides attend
over the same bf16 keys.  Output dims 448..511 must be exactly 0."""

import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import make_model1_workload

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = dict(max_abs=2e-2, rel_l2=1e-2, lse=1e-3)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def mla():
    import paged_mla_decode_05_amd as m

    m.load_library()
    assert torch.cuda.is_available()
    return m


def bf16_bits(x64):
    return torch.from_numpy(np.ascontiguousarray(x64)).to(torch.bfloat16).view(torch.int16).numpy()


def test_expand_records_bit_exact(mla):
    say("model1: record expansion, 2 requests, page size 16")
    w = make_model1_workload([300, 5], heads=2, page_size=16, seed=21)
    rec = w.records.clone()
    # hand-placed codes: subnormals, the largest code, signed zeros, a zero tile
    rec[0, 0, :8] = torch.tensor([0x01, 0x81, 0x07, 0x7E, 0xFE, 0x00, 0x80, 0x38], dtype=torch.uint8)
    rec[0, 1, 64:128] = 0
    rec[0, 1, 448 + 4:448 + 8] = 0  # scale of tile 1 = 0
    rows = mla.mla_model1_expand_records(rec.to(DEV))
    torch.cuda.synchronize()
    got = rows.cpu().view(torch.int16).numpy()
    nope, rope = oracle.model1_record_decode(rec)
    assert np.array_equal(got[..., :448], bf16_bits(nope))
    assert (got[..., 448:512] == 0).all()
    assert np.array_equal(got[..., 512:], rec[..., 476:].contiguous().view(torch.int16).numpy())


def test_expand_q_bit_exact(mla):
    g = torch.Generator().manual_seed(4)
    q = torch.randn((3, 5, 512), generator=g).to(torch.bfloat16)
    q576 = mla.mla_model1_expand_q(q.to(DEV)).cpu()
    assert torch.equal(q576[..., :448].view(torch.int16), q[..., :448].view(torch.int16))
    assert (q576[..., 448:512].view(torch.int16) == 0).all()
    assert torch.equal(q576[..., 512:].view(torch.int16), q[..., 448:].view(torch.int16))


CASES = [
    # (heads, page_size, kv_lens, tile_mode, force_splits)
    (16, 64, [1, 37, 64, 200], 0, 0),
    (16, 16, [5, 300, 0, 1], 2, 3),
    (128, 16, [700, 3, 65], 1, 3),
    (128, 64, [1000, 1, 257], 0, 0),
]


@pytest.mark.parametrize("case", CASES, ids=[f"H{c[0]}-ps{c[1]}-m{c[3]}-s{c[4]}" for c in CASES])
def test_decode_over_expanded_records(mla, case):
    H, ps, lens, mode, fs = case
    say(f"model1 decode H={H} page_size={ps} lens={lens} tile_mode={mode} force_splits={fs}")
    w = make_model1_workload(lens, heads=H, page_size=ps, seed=40 + H + ps)
    rows = mla.mla_model1_expand_records(w.records.to(DEV))
    q576 = mla.mla_model1_expand_q(w.q.to(DEV))
    plan = mla.mla_plan_create(mla.MLA_KIND_DECODE, w.batch, H, ps, w.num_pages, w.kv_len, w.kv_indptr,
                               tile_mode=mode, force_splits=fs)
    out, lse = mla.mla_decode_packed(plan, q576, rows, w.kv_indptr.to(DEV), w.kv_indices.to(DEV), w.sm_scale)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.mla_decode_model1_ref(w.q, w.records, w.kv_indptr, w.kv_indices, w.kv_len, w.sm_scale)
    o = out.double().cpu().numpy()
    l = lse.double().cpu().numpy()
    assert (o[..., 448:] == 0).all()
    o = o[..., :448]
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(l), empty) and np.all(o[empty] == 0)
    err = np.abs(o - ref_o).max()
    rel = np.linalg.norm(o - ref_o) / np.linalg.norm(ref_o)
    lerr = np.abs(l[~empty] - ref_l[~empty]).max()
    say(f"    max|dout|={err:.3e} relL2={rel:.3e} max|dlse|={lerr:.3e}")
    assert err <= TOL["max_abs"] and rel <= TOL["rel_l2"] and lerr <= TOL["lse"]


def test_sparse_attention_over_expanded_records(mla):
    """The token-sparse form (MODEL1_FP8Sparse): per-query key lists with
    invalid entries, an attention sink and forced splits, over rows expanded
    from MODEL1 records, against the oracle's sparse attention over its own
    dequantised keys (widened with zeros in dims 448..511, the form the
    dense MODEL1 oracle test pins as the same attention)."""
    from workloads import quantize_model1_records

    say("model1 sparse: s_q=6 H=32 s_kv=700 topk=96, sink, 2 splits")
    g = torch.Generator().manual_seed(77)
    s_q, H, s_kv, topk = 6, 32, 700, 96
    src = torch.randn((s_kv, 512), generator=g).to(torch.bfloat16)
    rec = quantize_model1_records(src)
    q = torch.randn((s_q, H, 512), generator=g).to(torch.bfloat16)
    idx = torch.randint(0, s_kv, (s_q, topk), generator=g, dtype=torch.int64).to(torch.int32)
    idx[:, ::7] = -1
    sink = (torch.randn(H, generator=g) + 4.0).to(torch.float32)
    scale = 0.07
    rows = mla.mla_model1_expand_records(rec.to(DEV))
    q576 = mla.mla_model1_expand_q(q.to(DEV))
    plan = mla.mla_sparse_plan_create(s_q, H, s_kv, topk, kv_format=mla.MLA_KV_BF16, force_splits=2)
    out, lse, mx = mla.mla_sparse_prefill(plan, q576, rows, idx.to(DEV), scale, attn_sink=sink.to(DEV))
    torch.cuda.synchronize()
    nope, rope = oracle.model1_record_decode(rec)
    kv = np.zeros((s_kv, 576))
    kv[:, :448], kv[:, 512:] = nope, rope
    qq = np.zeros((s_q, H, 576))
    qq[..., :448], qq[..., 512:] = q[..., :448].double().numpy(), q[..., 448:].double().numpy()
    ref_o, ref_l, ref_m = oracle.mla_sparse_prefill_ref(qq, kv, idx.numpy(), scale, attn_sink=sink.numpy())
    o = out.double().cpu().numpy()
    assert (o[..., 448:] == 0).all()
    err = np.abs(o[..., :448] - ref_o[..., :448]).max()
    rel = np.linalg.norm(o[..., :448] - ref_o[..., :448]) / np.linalg.norm(ref_o[..., :448])
    lerr = np.abs(lse.double().cpu().numpy() - ref_l).max()
    merr = np.abs(mx.double().cpu().numpy() - ref_m).max()
    say(f"    max|dout|={err:.3e} relL2={rel:.3e} max|dlse|={lerr:.3e} max|dmax|={merr:.3e}")
    assert err <= TOL["max_abs"] and rel <= TOL["rel_l2"] and lerr <= TOL["lse"] and merr <= TOL["lse"]
