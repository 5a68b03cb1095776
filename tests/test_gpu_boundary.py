"""The boundary's run-time options, through the C ABI on the GPU:

* validate = 1 ("batch_mla_decode_with_paged_kv_cache": pre-planned runs may
  skip the checks with run(validate=False)): a bad page id, page offset,
  query offset or live length is refused with MLA_ERR_INVALID_ARGUMENT
  before any attention kernel runs (the outputs keep their sentinel bits);
  good arrays give bitwise the results of an unchecked call;
* the lse layout [batch, H, s_q] of FlashMLA's "flash_mla_with_kvcache
  (Dense Attention)" is bitwise the transposed [rows, H] layout;
* capacity plans (max_kv_len, max_seq_len_q of the same FlashInfer page):
  one plan serves several steps of different live lengths, each within the
  bf16 gate of the float64 oracle; rows past the live query tokens are not
  written.

Only the small check kernel ever sees a bad array: the attention kernel is
never launched on one.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import make_workload

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = dict(max_abs=2e-2, rel_l2=1e-2, lse=1e-3)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def mla():
    import paged_mla_decode_05_amd as m

    m.load_library()
    return m


def compare(out, lse, ref_o, ref_l):
    o = out.double().cpu().numpy()
    l = lse.double().cpu().numpy()
    assert np.all(np.isfinite(o))
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(l), empty)
    assert np.all(o[empty] == 0)
    err = np.abs(o - ref_o).max()
    den = np.linalg.norm(ref_o)
    rel = np.linalg.norm(o - ref_o) / den if den > 0 else 0.0
    lerr = np.abs(l[~empty] - ref_l[~empty]).max() if (~empty).any() else 0.0
    say(f"    max|dout|={err:.3e} relL2={rel:.3e} max|dlse|={lerr:.3e}")
    assert err <= TOL["max_abs"] and rel <= TOL["rel_l2"] and lerr <= TOL["lse"]


def _dev_inputs(w):
    return dict(q_nope=w.q_nope.to(DEV), q_pe=w.q_pe.to(DEV), ckv=w.ckv.to(DEV), kpe=w.kpe.to(DEV),
                kv_indptr=w.kv_indptr.to(DEV), kv_indices=w.kv_indices.to(DEV),
                qo_indptr=w.qo_indptr.to(DEV) if w.qo_indptr is not None else None)


# ---------------------------------------------------------------------------
# validate = 1
# ---------------------------------------------------------------------------

def _decode_call(mla, plan, w, x, kv_indices=None, kv_indptr=None):
    """(status, out, lse) of one decode call on sentinel-filled outputs."""
    lib = mla.load_library()
    out = torch.full((w.batch, w.num_heads, 512), 7.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((w.batch, w.num_heads), 7.0, dtype=torch.float32, device=DEV)
    ws = plan.workspace(DEV)
    ip = x["kv_indptr"] if kv_indptr is None else kv_indptr
    ix = x["kv_indices"] if kv_indices is None else kv_indices
    st = lib.mla_decode(plan.handle, x["q_nope"].data_ptr(), x["q_pe"].data_ptr(), x["ckv"].data_ptr(),
                        x["kpe"].data_ptr(), ip.data_ptr(), ix.data_ptr(), float(w.sm_scale), out.data_ptr(), 0,
                        lse.data_ptr(), ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return st, out, lse


@pytest.mark.parametrize("mode", [1, 2, 3])
def test_validate_passes_good_arrays_bitwise(mla, mode):
    w = make_workload(kv_lens=[300, 1, 0, 1200], heads=64, page_size=16, seed=501)
    x = _dev_inputs(w)
    outs = []
    for v in (False, True):
        plan = mla.mla_plan_create(mla.MLA_KIND_DECODE, w.batch, w.num_heads, w.page_size, w.num_pages, w.kv_len,
                                   w.kv_indptr, tile_mode=mode, force_splits=3, validate=v)
        st, out, lse = _decode_call(mla, plan, w, x)
        assert st == 0
        outs.append((out, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("bad", ["page_past_pool", "negative_page", "indptr_shifted", "indptr_start"])
def test_validate_refuses_bad_decode_arrays(mla, bad):
    say(f"validate decode: {bad}")
    w = make_workload(kv_lens=[300, 77, 1000], heads=128, page_size=64, seed=502)
    x = _dev_inputs(w)
    plan = mla.mla_plan_create(mla.MLA_KIND_DECODE, w.batch, w.num_heads, w.page_size, w.num_pages, w.kv_len,
                               w.kv_indptr, validate=True)
    ix = x["kv_indices"].clone()
    ip = x["kv_indptr"].clone()
    if bad == "page_past_pool":
        ix[-1] = w.num_pages
    elif bad == "negative_page":
        ix[3] = -1
    elif bad == "indptr_shifted":
        ip[1] += 1
    else:
        ip[0] = 1
    st, out, lse = _decode_call(mla, plan, w, x, kv_indices=ix, kv_indptr=ip)
    assert st == mla.MLA_ERR_INVALID_ARGUMENT
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)  # nothing was launched past the check


def test_validate_refuses_bad_prefill_offsets(mla):
    w = make_workload(kind="prefill", kv_lens=[300, 77], q_lens=[3, 2], heads=32, page_size=16, seed=503)
    x = _dev_inputs(w)
    plan = mla.mla_plan_create(mla.MLA_KIND_PREFILL, w.batch, w.num_heads, w.page_size, w.num_pages, w.kv_len,
                               w.kv_indptr, qo_indptr=w.qo_indptr, validate=True)
    out, lse = mla.mla_prefill(plan, x["q_nope"], x["q_pe"], x["ckv"], x["kpe"], x["qo_indptr"], x["kv_indptr"],
                               x["kv_indices"], w.sm_scale)
    compare(out, lse, *oracle.mla_prefill_ref(w.q_nope, w.q_pe, w.ckv, w.kpe, w.qo_indptr, w.kv_indptr,
                                              w.kv_indices, w.kv_len, w.sm_scale))
    qo = x["qo_indptr"].clone()
    qo[1] -= 1
    with pytest.raises(mla.MLAError) as e:
        mla.mla_prefill(plan, x["q_nope"], x["q_pe"], x["ckv"], x["kpe"], qo, x["kv_indptr"], x["kv_indices"],
                        w.sm_scale)
    assert e.value.status == mla.MLA_ERR_INVALID_ARGUMENT


# ---------------------------------------------------------------------------
# lse layout [batch, H, s_q]
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode,splits", [(1, 0), (1, 3), (2, 2), (3, 2)])
def test_lse_heads_first_is_the_transposed_rows_layout(mla, mode, splits):
    s_q, H = 3, 32
    w = make_workload(kind="prefill", kv_lens=[300, 77, 1000], q_lens=[s_q] * 3, heads=H, page_size=16, seed=504)
    x = _dev_inputs(w)
    res = []
    for layout in (mla.MLA_LSE_ROWS, mla.MLA_LSE_HEADS_FIRST):
        plan = mla.mla_plan_create(mla.MLA_KIND_PREFILL, w.batch, H, w.page_size, w.num_pages, w.kv_len, w.kv_indptr,
                                   qo_indptr=w.qo_indptr, tile_mode=mode, force_splits=splits, lse_layout=layout)
        res.append(mla.mla_prefill(plan, x["q_nope"], x["q_pe"], x["ckv"], x["kpe"], x["qo_indptr"],
                                   x["kv_indptr"], x["kv_indices"], w.sm_scale))
    torch.cuda.synchronize()
    (o_rows, l_rows), (o_hf, l_hf) = res
    assert l_hf.shape == (3, H, s_q)
    assert torch.equal(o_rows, o_hf)
    assert torch.equal(l_rows.view(3, s_q, H).permute(0, 2, 1), l_hf)


def test_lse_heads_first_decode_equals_rows(mla):
    w = make_workload(kv_lens=[300, 5, 2000], heads=128, page_size=64, seed=505)
    x = _dev_inputs(w)
    res = []
    for layout in (mla.MLA_LSE_ROWS, mla.MLA_LSE_HEADS_FIRST):
        plan = mla.mla_plan_create(mla.MLA_KIND_DECODE, w.batch, w.num_heads, w.page_size, w.num_pages, w.kv_len,
                                   w.kv_indptr, force_splits=2, lse_layout=layout)
        res.append(mla.mla_decode(plan, x["q_nope"], x["q_pe"], x["ckv"], x["kpe"], x["kv_indptr"],
                                  x["kv_indices"], w.sm_scale))
    torch.cuda.synchronize()
    assert torch.equal(res[0][0], res[1][0])
    assert torch.equal(res[0][1], res[1][1].view(w.batch, w.num_heads))


# ---------------------------------------------------------------------------
# capacity plans
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("H,mode,splits", [(128, 1, 0), (128, 1, 4), (16, 2, 3), (128, 3, 2), (40, 0, 0)])
def test_capacity_decode_live_lengths(mla, H, mode, splits):
    max_kv = 1500
    for step, lens in enumerate([[1500, 3, 0, 777], [64, 1499, 1, 1200], [0, 0, 0, 0]]):
        say(f"capacity decode H={H} mode={mode} splits={splits} step {step} lens={lens}")
        w = make_workload(kv_lens=lens, heads=H, page_size=16, seed=506 + step)
        x = _dev_inputs(w)
        plan = mla.mla_plan_create(mla.MLA_KIND_DECODE, 4, H, 16, w.num_pages, None, None, tile_mode=mode,
                                   force_splits=splits, max_kv_len=max_kv, validate=True)
        out, lse = mla.mla_decode_live(plan, x["q_nope"], x["q_pe"], x["ckv"], x["kpe"], w.kv_len.to(DEV),
                                       x["kv_indptr"], x["kv_indices"], w.sm_scale)
        torch.cuda.synchronize()
        compare(out, lse, *oracle.mla_decode_ref(w.q_nope, w.q_pe, w.ckv, w.kpe, w.kv_indptr, w.kv_indices,
                                                 w.kv_len, w.sm_scale))


def test_capacity_decode_one_plan_many_steps(mla):
    # one plan object and one workspace reused across steps on one pool
    H, ps, max_kv = 128, 64, 2048
    pool = make_workload(kv_lens=[max_kv] * 3, heads=H, page_size=ps, seed=510)
    plan = mla.mla_plan_create(mla.MLA_KIND_DECODE, 3, H, ps, pool.num_pages, None, None, max_kv_len=max_kv)
    x = _dev_inputs(pool)
    for step, lens in enumerate([[2048, 1, 700], [65, 2000, 0], [1, 1, 1]]):
        say(f"one capacity plan, step {step}: live lens {lens}")
        kl = torch.tensor(lens, dtype=torch.int32)
        out, lse = mla.mla_decode_live(plan, x["q_nope"], x["q_pe"], x["ckv"], x["kpe"], kl.to(DEV), x["kv_indptr"],
                                       x["kv_indices"], pool.sm_scale)
        torch.cuda.synchronize()
        # the live keys are the first kv_len[b] of each request's pages
        compare(out, lse, *oracle.mla_decode_ref(pool.q_nope, pool.q_pe, pool.ckv, pool.kpe,
                                                 _trim_indptr(pool.kv_indptr, kl, ps), _trim_indices(pool, kl, ps),
                                                 kl, pool.sm_scale))


def _trim_indptr(indptr, kl, ps):
    pages = (kl.to(torch.int64) + ps - 1) // ps
    out = torch.zeros(len(kl) + 1, dtype=torch.int32)
    out[1:] = torch.cumsum(pages, 0).to(torch.int32)
    return out


def _trim_indices(w, kl, ps):
    parts = []
    for b in range(len(kl)):
        n = (int(kl[b]) + ps - 1) // ps
        parts.append(w.kv_indices[int(w.kv_indptr[b]):int(w.kv_indptr[b]) + n])
    return torch.cat(parts) if parts else torch.zeros(0, dtype=torch.int32)


@pytest.mark.parametrize("mode,layout", [(1, 0), (1, 1), (2, 0), (3, 1)])
def test_capacity_prefill_live_queries(mla, mode, layout):
    H, ps, max_kv, max_q = 32, 16, 900, 4
    plan = None
    for step, (qlens, lens) in enumerate([([4, 1, 2], [900, 40, 2]), ([0, 4, 3], [5, 600, 3])]):
        say(f"capacity prefill mode={mode} layout={layout} step {step}: q {qlens} kv {lens}")
        w = make_workload(kind="prefill", kv_lens=lens, q_lens=qlens, heads=H, page_size=ps, seed=520 + step)
        x = _dev_inputs(w)
        plan = mla.mla_plan_create(mla.MLA_KIND_PREFILL, 3, H, ps, w.num_pages, None, None, tile_mode=mode,
                                   max_kv_len=max_kv, max_seq_len_q=max_q, lse_layout=layout, validate=True)
        lse = None
        if layout == mla.MLA_LSE_HEADS_FIRST:
            lse = torch.full((3, H, max_q), 7.0, dtype=torch.float32, device=DEV)
        out, lse = mla.mla_prefill_live(plan, x["q_nope"], x["q_pe"], x["ckv"], x["kpe"], x["qo_indptr"],
                                        w.kv_len.to(DEV), x["kv_indptr"], x["kv_indices"], w.sm_scale, lse=lse)
        torch.cuda.synchronize()
        ro, rl = oracle.mla_prefill_ref(w.q_nope, w.q_pe, w.ckv, w.kpe, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                        w.kv_len, w.sm_scale)
        if layout == mla.MLA_LSE_HEADS_FIRST:
            qo = w.qo_indptr.numpy()
            rows = torch.full((int(qo[-1]), H), float("nan"))
            for b in range(3):
                n = qo[b + 1] - qo[b]
                assert torch.all(lse[b, :, n:] == 7.0)  # past the live tokens: not written
                rows[qo[b]:qo[b + 1]] = lse[b, :, :n].t().cpu()
            lse = rows
        compare(out, lse, ro, rl)


def test_capacity_live_lengths_are_validated(mla):
    w = make_workload(kv_lens=[100, 50], heads=16, page_size=16, seed=530)
    x = _dev_inputs(w)
    plan = mla.mla_plan_create(mla.MLA_KIND_DECODE, 2, 16, 16, w.num_pages, None, None, max_kv_len=100,
                               validate=True)
    for lens in ([101, 50], [-1, 50], [100, 65]):  # over the bound, negative, more keys than pages
        with pytest.raises(mla.MLAError) as e:
            mla.mla_decode_live(plan, x["q_nope"], x["q_pe"], x["ckv"], x["kpe"],
                                torch.tensor(lens, dtype=torch.int32, device=DEV), x["kv_indptr"], x["kv_indices"],
                                w.sm_scale)
        assert e.value.status == mla.MLA_ERR_INVALID_ARGUMENT
    # a capacity plan cannot run through the exact-length calls, nor an exact plan through the live ones
    with pytest.raises(mla.MLAError):
        mla.mla_decode(plan, x["q_nope"], x["q_pe"], x["ckv"], x["kpe"], x["kv_indptr"], x["kv_indices"], w.sm_scale)


# ---------------------------------------------------------------------------
# gang-packed prefill plans (128 heads, several query tokens per request:
# each token's 128-row block gets the same key pieces on neighbouring lists)
# ---------------------------------------------------------------------------

def _is_ganged(plan, H):
    items = plan.work_items().numpy()
    ptr = plan.workgroup_ptr().numpy()
    first = {}
    for w in range(len(ptr) - 1):
        for pos, it in enumerate(items[ptr[w]:ptr[w + 1]]):
            first.setdefault((int(it[0]), int(it[1])), (w, pos, int(it[3])))
    return any(first.get((b, r0 + H)) == (w + 1, pos, t0) for (b, r0), (w, pos, t0) in first.items())


@pytest.mark.parametrize("layout", [0, 1])
def test_gang_prefill(mla, layout):
    H, s_q = 128, 4
    w = make_workload(kind="prefill", kv_lens=[700, 2100, 64, 1500], q_lens=[s_q] * 4, heads=H, page_size=64,
                      seed=540 + layout)
    x = _dev_inputs(w)
    plan = mla.mla_plan_create(mla.MLA_KIND_PREFILL, w.batch, H, w.page_size, w.num_pages, w.kv_len, w.kv_indptr,
                               qo_indptr=w.qo_indptr, lse_layout=layout)
    assert _is_ganged(plan, H)
    out, lse = mla.mla_prefill(plan, x["q_nope"], x["q_pe"], x["ckv"], x["kpe"], x["qo_indptr"], x["kv_indptr"],
                               x["kv_indices"], w.sm_scale)
    torch.cuda.synchronize()
    if layout == mla.MLA_LSE_HEADS_FIRST:
        lse = lse.permute(0, 2, 1).reshape(-1, H)
    compare(out, lse, *oracle.mla_prefill_ref(w.q_nope, w.q_pe, w.ckv, w.kpe, w.qo_indptr, w.kv_indptr,
                                              w.kv_indices, w.kv_len, w.sm_scale))


def test_gang_capacity_prefill(mla):
    H, max_kv, max_q = 128, 4096, 4
    plan = mla.mla_plan_create(mla.MLA_KIND_PREFILL, 3, H, 64, 200, None, None, max_kv_len=max_kv,
                               max_seq_len_q=max_q, validate=True)
    assert _is_ganged(plan, H)
    for step, (qlens, lens) in enumerate([([4, 2, 4], [4096, 900, 4]), ([1, 4, 3], [64, 4000, 1500])]):
        say(f"gang capacity prefill step {step}: q {qlens} kv {lens}")
        w = make_workload(kind="prefill", kv_lens=lens, q_lens=qlens, heads=H, page_size=64, seed=545 + step,
                          pool_pages=200)
        x = _dev_inputs(w)
        out, lse = mla.mla_prefill_live(plan, x["q_nope"], x["q_pe"], x["ckv"], x["kpe"], x["qo_indptr"],
                                        w.kv_len.to(DEV), x["kv_indptr"], x["kv_indices"], w.sm_scale)
        torch.cuda.synchronize()
        compare(out, lse, *oracle.mla_prefill_ref(w.q_nope, w.q_pe, w.ckv, w.kpe, w.qo_indptr, w.kv_indptr,
                                                  w.kv_indices, w.kv_len, w.sm_scale))
