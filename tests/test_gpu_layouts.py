"""GPU tests of the interface adapters: the concatenated 576-wide q / cache
layout, the output scale, and page lists built from a dense block table.

The concatenated layout reads the same numbers as the split layout through
other row strides, so with an output scale of 1 its results must match the
split entry points bit for bit; they are also compared with the float64
oracle on the split views.  An output scale s multiplies the output only
(lse is unchanged bit for bit); it is checked against s times the oracle's
output, with the bf16 tolerances scaled by |s|.  The block-table conversion
is integer work and is checked bit-exactly against a gather on the host.
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
    assert torch.cuda.is_available()
    return m


def check(out, lse, ref_o, ref_l, scale=1.0):
    o = out.double().cpu().numpy()
    l = lse.double().cpu().numpy()
    ref_o = ref_o * scale
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(l), empty)
    assert np.all(np.isfinite(o)) and np.all(o[empty] == 0)
    err = np.abs(o - ref_o).max() if o.size else 0.0
    den = np.linalg.norm(ref_o)
    rel = np.linalg.norm(o - ref_o) / den if den > 0 else 0.0
    lerr = np.abs(l[~empty] - ref_l[~empty]).max() if (~empty).any() else 0.0
    say(f"    max|dout|={err:.3e} relL2={rel:.3e} max|dlse|={lerr:.3e}")
    assert err <= TOL["max_abs"] * max(1.0, abs(scale)) and rel <= TOL["rel_l2"] and lerr <= TOL["lse"]


def packed(w):
    q = torch.cat([w.q_nope, w.q_pe], dim=-1).contiguous()
    kv = torch.cat([w.ckv, w.kpe], dim=-1).contiguous()
    return q.to(DEV), kv.to(DEV)


def decode_plan(mla, w, **kw):
    return mla.mla_plan_create(mla.MLA_KIND_DECODE, w.batch, w.num_heads, w.page_size, w.num_pages, w.kv_len,
                               w.kv_indptr, num_cus=0, **kw)


def prefill_plan(mla, w, **kw):
    return mla.mla_plan_create(mla.MLA_KIND_PREFILL, w.batch, w.num_heads, w.page_size, w.num_pages, w.kv_len,
                               w.kv_indptr, qo_indptr=w.qo_indptr, causal=w.causal, **kw)


DECODE_CASES = [
    # (heads, page_size, kv_lens, tile_mode, force_splits, out fp32)
    (128, 64, [1, 37, 64, 700], 1, 0, False),
    (128, 16, [900, 3, 65], 1, 3, True),
    (16, 64, [5, 300, 64, 1], 2, 0, False),
    (16, 1, [3, 70, 129], 2, 2, True),
    (128, 64, [1000, 1, 257], 3, 4, False),
    (40, 8, [100, 400, 0, 33], 3, 2, False),
    (24, 4, [90, 31], 0, 0, True),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[f"H{c[0]}-ps{c[1]}-m{c[3]}-s{c[4]}" for c in DECODE_CASES])
def test_packed_decode_matches_split_bitwise(mla, case):
    H, ps, lens, mode, fs, f32 = case
    say(f"packed decode H={H} page_size={ps} lens={lens} tile_mode={mode} force_splits={fs}")
    w = make_workload(kv_lens=lens, heads=H, page_size=ps, seed=400 + H + ps,
                      out_dtype=torch.float32 if f32 else torch.bfloat16)
    plan = decode_plan(mla, w, tile_mode=mode, force_splits=fs)
    ip, ix = w.kv_indptr.to(DEV), w.kv_indices.to(DEV)
    o1, l1 = mla.mla_decode(plan, w.q_nope.to(DEV), w.q_pe.to(DEV), w.ckv.to(DEV), w.kpe.to(DEV), ip, ix,
                            w.sm_scale, out_dtype=w.out_dtype)
    q, kv = packed(w)
    o2, l2 = mla.mla_decode_packed(plan, q, kv, ip, ix, w.sm_scale, out_dtype=w.out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    check(o2, l2, *oracle.mla_decode_ref(w.q_nope, w.q_pe, w.ckv, w.kpe, w.kv_indptr, w.kv_indices, w.kv_len,
                                         w.sm_scale))


@pytest.mark.parametrize("mode,fs", [(1, 0), (1, 3), (3, 2), (2, 0)])
def test_packed_prefill_matches_split_bitwise(mla, mode, fs):
    H = 16 if mode == 2 else 128
    say(f"packed prefill H={H} tile_mode={mode} force_splits={fs}")
    w = make_workload(kind="prefill", kv_lens=[64, 100, 700, 5], q_lens=[3, 1, 8, 5], heads=H, page_size=64,
                      causal=True, seed=41 + mode)
    plan = prefill_plan(mla, w, tile_mode=mode, force_splits=fs)
    qo, ip, ix = w.qo_indptr.to(DEV), w.kv_indptr.to(DEV), w.kv_indices.to(DEV)
    o1, l1 = mla.mla_prefill(plan, w.q_nope.to(DEV), w.q_pe.to(DEV), w.ckv.to(DEV), w.kpe.to(DEV), qo, ip, ix,
                             w.sm_scale)
    q, kv = packed(w)
    o2, l2 = mla.mla_prefill_packed(plan, q, kv, qo, ip, ix, w.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    check(o2, l2, *oracle.mla_prefill_ref(w.q_nope, w.q_pe, w.ckv, w.kpe, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                          w.kv_len, w.sm_scale, causal=True))


@pytest.mark.parametrize("mode,fs,scale", [(1, 0, 0.5), (1, 3, 3.0), (2, 2, -1.25), (3, 0, 2.0), (3, 3, 0.0)])
def test_output_scale(mla, mode, fs, scale):
    # Final rows are written directly (no split) or by the combine pass (split
    # requests); both must apply the scale once.
    H = 16 if mode == 2 else 128
    say(f"output scale {scale} H={H} tile_mode={mode} force_splits={fs}")
    w = make_workload(kv_lens=[2000, 37, 0, 600], heads=H, page_size=64, seed=77 + mode,
                      out_dtype=torch.float32)
    plan = decode_plan(mla, w, tile_mode=mode, force_splits=fs)
    q, kv = packed(w)
    ip, ix = w.kv_indptr.to(DEV), w.kv_indices.to(DEV)
    o1, l1 = mla.mla_decode_packed(plan, q, kv, ip, ix, w.sm_scale, out_dtype=torch.float32)
    o2, l2 = mla.mla_decode_packed(plan, q, kv, ip, ix, w.sm_scale, out_scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(l1, l2), "the output scale must not touch lse"
    ref_o, ref_l = oracle.mla_decode_ref(w.q_nope, w.q_pe, w.ckv, w.kpe, w.kv_indptr, w.kv_indices, w.kv_len,
                                         w.sm_scale)
    check(o2, l2, ref_o, ref_l, scale=scale)
    # fp32 output: one extra rounding at most between s*(o/l) and (s/l)*o
    np.testing.assert_allclose(o2.double().cpu().numpy(), scale * o1.double().cpu().numpy(), rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("batch,max_blocks", [(4, 40), (1, 1), (33, 300)])
def test_block_table_to_indices_is_exact(mla, batch, max_blocks):
    say(f"block table batch={batch} max_blocks={max_blocks}")
    g = np.random.default_rng(batch * 1000 + max_blocks)
    pages = g.integers(0, max_blocks + 1, size=batch)
    pages[0] = max_blocks  # one full row
    indptr = np.concatenate([[0], np.cumsum(pages)]).astype(np.int32)
    table = g.integers(0, 1 << 30, size=(batch, max_blocks)).astype(np.int32)
    lens = [int(p) * 64 for p in pages]
    plan = mla.mla_plan_create(mla.MLA_KIND_DECODE, batch, 128, 64, 1 << 30, lens, indptr)
    sentinel = -7
    out = torch.full((int(indptr[-1]) + 5,), sentinel, dtype=torch.int32, device=DEV)
    mla.mla_block_table_to_indices(plan, torch.from_numpy(table).to(DEV), torch.from_numpy(indptr).to(DEV), out)
    torch.cuda.synchronize()
    want = np.concatenate([table[b, :pages[b]] for b in range(batch)] + [np.full(5, sentinel, np.int32)])
    assert np.array_equal(out.cpu().numpy(), want)


def test_block_table_decode_equals_page_list_decode(mla):
    say("decode through a block table, H=128 page_size=16")
    w = make_workload(kv_lens=[130, 64, 1, 900], heads=128, page_size=16, seed=61)
    B = w.batch
    counts = (w.kv_indptr[1:] - w.kv_indptr[:-1]).numpy()
    maxb = int(counts.max()) + 3
    table = torch.full((B, maxb), -1, dtype=torch.int32)  # columns past a request's pages are never read
    for b in range(B):
        table[b, :counts[b]] = w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]
    plan = decode_plan(mla, w)
    ip = w.kv_indptr.to(DEV)
    ix = mla.mla_block_table_to_indices(plan, table.to(DEV), ip)
    q, kv = packed(w)
    o1, l1 = mla.mla_decode_packed(plan, q, kv, ip, w.kv_indices.to(DEV), w.sm_scale)
    o2, l2 = mla.mla_decode_packed(plan, q, kv, ip, ix, w.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(ix[: int(w.kv_indptr[-1])].cpu(), w.kv_indices[: int(w.kv_indptr[-1])])
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
