"""GPU parity of the fp8-query decode (mla_decode_fp8_q8, through the C ABI)
against the float64 oracle on the same seeded inputs.

The query is e4m3 codes taken at their values; the oracle decodes them
exactly, so the gate is the fp8-cache one (output max |err| <= 6e-2,
relative L2 <= 3e-2, lse <= 1e-3 against the oracle on the dequantised
records).  Unused pool slots hold NaN codes, scales and rope values.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import make_workload, quantize_q_e4m3

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = dict(max_abs=6e-2, rel_l2=3e-2, lse=1e-3)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def mla():
    import paged_mla_decode_05_amd as m

    m.load_library()
    assert torch.cuda.is_available()
    return m


def compare(out, lse, ref_o, ref_l, rows=None):
    o = out.double().cpu().numpy()
    l = lse.double().cpu().numpy()
    assert np.all(np.isfinite(o)) and not np.any(np.isnan(l)) and not np.any(np.isposinf(l))
    if rows is not None:
        o, l, ref_o, ref_l = o[rows], l[rows], ref_o[rows], ref_l[rows]
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(l), empty) and np.all(o[empty] == 0)
    err = np.abs(o - ref_o).max()
    rel = np.linalg.norm(o - ref_o) / np.linalg.norm(ref_o)
    lerr = np.abs(l[~empty] - ref_l[~empty]).max() if (~empty).any() else 0.0
    say(f"    max|dout|={err:.3e} relL2={rel:.3e} max|dlse|={lerr:.3e}")
    assert err <= TOL["max_abs"] and rel <= TOL["rel_l2"] and lerr <= TOL["lse"]


def run_q8(mla, w, q8, **plan_kw):
    plan = mla.mla_plan_create(mla.MLA_KIND_DECODE, w.batch, w.num_heads, w.page_size, w.num_pages, w.kv_len,
                               w.kv_indptr, kv_format=mla.MLA_KV_FP8_E4M3_T128, tile_mode=mla.MLA_TILE_WIDE,
                               **plan_kw)
    out, lse = mla.mla_decode_fp8_q8(plan, q8.to(DEV), w.kv_fp8.to(DEV), w.kv_indptr.to(DEV),
                                     w.kv_indices.to(DEV), w.sm_scale, out_dtype=w.out_dtype)
    torch.cuda.synchronize()
    return out, lse


CASES = [
    # (heads, page_size, kv_lens, force_splits, out fp32)
    (128, 64, [1, 37, 64, 200], 0, False),
    (128, 16, [700, 3, 65], 3, True),
    (128, 1, [2, 130], 2, False),
    (128, 256, [1000, 33], 2, False),
    (64, 64, [300, 5000], 0, False),
    (16, 8, [100, 400, 0, 33], 2, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"H{c[0]}-ps{c[1]}-s{c[3]}" for c in CASES])
def test_q8_small_cases(mla, case):
    H, ps, lens, fs, f32 = case
    say(f"fp8-query decode H={H} page_size={ps} lens={lens} force_splits={fs}")
    w = make_workload(kv_lens=lens, heads=H, page_size=ps, seed=800 + H + ps, kv_format="fp8",
                      out_dtype=torch.float32 if f32 else torch.bfloat16)
    q8 = quantize_q_e4m3(w.q_nope, w.q_pe)
    out, lse = run_q8(mla, w, q8, num_cus=0, force_splits=fs)
    compare(out, lse, *oracle.mla_decode_fp8_q8_ref(q8, w.kv_fp8, w.kv_indptr, w.kv_indices, w.kv_len, w.sm_scale))


def test_q8_needs_the_wide_tile(mla):
    w = make_workload(kv_lens=[100, 5], heads=16, page_size=64, seed=81, kv_format="fp8")
    plan = mla.mla_plan_create(mla.MLA_KIND_DECODE, w.batch, 16, 64, w.num_pages, w.kv_len, w.kv_indptr,
                               kv_format=mla.MLA_KV_FP8_E4M3_T128, tile_mode=mla.MLA_TILE_NARROW)
    q8 = quantize_q_e4m3(w.q_nope, w.q_pe).to(DEV)
    with pytest.raises(mla.MLAError) as e:
        mla.mla_decode_fp8_q8(plan, q8, w.kv_fp8.to(DEV), w.kv_indptr.to(DEV), w.kv_indices.to(DEV), w.sm_scale)
    assert e.value.status == -2


def test_q8_full_size(mla):
    say("decode_fp8_b128_h128 with an e4m3 query (bench launch configuration), every request")
    w = make_workload("decode_fp8_b128_h128", device=DEV)
    q8 = quantize_q_e4m3(w.q_nope, w.q_pe)
    out, lse = run_q8(mla, w, q8)
    ref = oracle.mla_decode_fp8_q8_ref(q8.cpu(), w.kv_fp8, w.kv_indptr, w.kv_indices, w.kv_len, w.sm_scale)
    compare(out, lse, *ref)
