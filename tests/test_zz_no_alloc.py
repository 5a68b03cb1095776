"""mla_decode_noalloc (the decode that allocates nothing and uses the
library's fixed device scratch array) against mla_decode with a caller
workspace: the same kernels on the same plan, so the results must agree bit
for bit, on two calls in a row (the second with a smaller input, so the
array still holds the first call's larger contents), and both must be
within the bf16 gate of the float64 oracle.  A plan too large for the array
is refused before anything is enqueued."""

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import make_workload

DEV = "cuda:0"
TOL = dict(max_abs=2e-2, rel_l2=1e-2, lse=1e-3)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def mla():
    import paged_mla_decode_05_amd as m

    m.load_library()
    return m


def _inputs(w):
    return (w.q_nope.to(DEV), w.q_pe.to(DEV), w.ckv.to(DEV), w.kpe.to(DEV), w.kv_indptr.to(DEV),
            w.kv_indices.to(DEV))


def _oracle_gate(out, lse, w):
    ref_o, ref_l = oracle.mla_decode_ref(w.q_nope, w.q_pe, w.ckv, w.kpe, w.kv_indptr, w.kv_indices, w.kv_len,
                                         w.sm_scale)
    o = out.double().cpu().numpy()
    l = lse.double().cpu().numpy()
    assert np.all(np.isfinite(o))
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(l), empty)
    err = np.abs(o - ref_o).max()
    rel = np.linalg.norm(o - ref_o) / np.linalg.norm(ref_o)
    lerr = np.abs(l[~empty] - ref_l[~empty]).max()
    say(f"    vs oracle: max|dout|={err:.3e} relL2={rel:.3e} max|dlse|={lerr:.3e}")
    assert err <= TOL["max_abs"] and rel <= TOL["rel_l2"] and lerr <= TOL["lse"]


@pytest.mark.gpu
def test_noalloc_decode_matches_workspace_decode(mla):
    cases = [
        # (heads, page size, kv lens, tile mode, forced splits): the first is the larger
        (128, 64, [3000, 17, 1200, 640, 0, 2049], 1, 3),
        (16, 16, [5, 300, 64], 2, 2),
    ]
    for H, ps, lens, mode, fs in cases:
        say(f"noalloc decode H={H} page_size={ps} lens={lens} tile_mode={mode} force_splits={fs}")
        w = make_workload(kv_lens=lens, heads=H, page_size=ps, seed=900 + H)
        plan = mla.mla_plan_create(mla.MLA_KIND_DECODE, w.batch, w.num_heads, w.page_size, w.num_pages, w.kv_len,
                                   w.kv_indptr, tile_mode=mode, force_splits=fs)
        assert plan.num_split_groups > 0
        qn, qp, ckv, kpe, ip, ix = _inputs(w)
        o_ws, l_ws = mla.mla_decode(plan, qn, qp, ckv, kpe, ip, ix, w.sm_scale)
        o_na, l_na = mla.mla_decode_noalloc(plan, qn, qp, ckv, kpe, ip, ix, w.sm_scale)
        torch.cuda.synchronize()
        assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16))
        assert torch.equal(l_ws.view(torch.int32), l_na.view(torch.int32))
        _oracle_gate(o_na, l_na, w)


@pytest.mark.gpu
def test_noalloc_rejects_a_plan_larger_than_its_array(mla):
    lib = mla.load_library()
    # 128 requests x 128 heads cut into 64 pieces each: 8192 partial slots of
    # 128 rows x 1 KB, far above the 64 MiB array
    B, H = 128, 128
    lens = np.full(B, 64 * 64)
    indptr = np.concatenate([[0], np.cumsum(lens // 64)])
    plan = mla.mla_plan_create(mla.MLA_KIND_DECODE, B, H, 64, int(indptr[-1]), lens, indptr, tile_mode=1,
                               force_splits=64, num_cus=256)
    assert plan.workspace_bytes > mla.NOALLOC_SCRATCH_BYTES
    st = lib.mla_decode_noalloc(plan.handle, 1, 1, 1, 1, 1, 1, ctypes.c_float(1.0), 1, 0, 1, None)
    assert st == -3  # MLA_ERR_WORKSPACE, nothing enqueued
