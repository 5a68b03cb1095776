"""Pins of the oracle's fp8 pieces: the e4m3 codec, the 656-byte record, and
the fp8 decode built on them."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_special_codes_match_the_format_definition():
    spec = json.load(open(os.path.join(GOLDEN, "e4m3_special_codes.json")))
    for item in spec["codes"]:
        v = oracle.e4m3_decode(np.array([int(item["code"], 16)]))[0]
        if item["value"] == "nan":
            assert math.isnan(v)
        else:
            assert v == item["value"] and math.copysign(1, v) == math.copysign(1, item["value"])


def test_all_codes_match_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()


def test_encoder_matches_torch_cast_after_clamp():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000) * 50,
        rng.standard_normal(20000) * 1e-3,            # subnormal range
        oracle.e4m3_all_finite_values(),               # exact codes
        (oracle.e4m3_all_finite_values()[1:] + oracle.e4m3_all_finite_values()[:-1]) / 2,  # ties
        [600.0, -1000.0, 448.0, 464.0, 0.0],
    ]).astype(np.float32)
    mine = oracle.e4m3_encode(x.astype(np.float64))
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # +-0 may differ only in the sign bit of a zero
    both_zero = (oracle.e4m3_decode(mine) == 0) & (oracle.e4m3_decode(ref) == 0)
    assert np.all((mine == ref) | both_zero)


def test_encoder_roundtrip_error_bound():
    rng = np.random.default_rng(1)
    x = rng.uniform(-448, 448, 100000)
    y = oracle.e4m3_decode(oracle.e4m3_encode(x))
    big = np.abs(x) >= 2.0 ** -6
    # 3 mantissa bits: half an ulp is 2^-4 relative for normals, 2^-10 absolute for subnormals
    assert np.all(np.abs(y - x)[big] <= 2.0 ** -4 * np.abs(x)[big])
    assert np.all(np.abs(y - x)[~big] <= 2.0 ** -10)


def test_hand_built_record_decodes_as_the_layout_says():
    spec = json.load(open(os.path.join(GOLDEN, "fp8_record_656.json")))
    rec = np.zeros(656, dtype=np.uint8)
    for off, byte in spec["bytes"]:
        rec[off] = int(byte, 16)
    nope, rope = oracle.fp8_record_decode(rec[None])
    for d, v in spec["expected_nope"].items():
        assert nope[0, int(d)] == v
    for d, v in spec["expected_rope"].items():
        assert rope[0, int(d)] == v


def test_record_encoder_layout_and_scales():
    rng = np.random.default_rng(2)
    tok = torch.from_numpy(rng.standard_normal((50, 576)).astype(np.float32)).to(torch.bfloat16)
    tok[3, 128:256] = 0  # an all-zero tile: scale 0, codes 0
    rec = oracle.fp8_record_encode(tok)
    assert rec.shape == (50, 656)
    x = oracle.as_f64(tok)
    scales = rec[:, 512:528].copy().view("<f4")
    amax = np.abs(x[:, :512].reshape(50, 4, 128)).max(axis=2)
    assert np.array_equal(scales, (amax.astype(np.float32) / np.float32(448)).astype(np.float32))
    assert scales[3, 1] == 0 and np.all(rec[3, 128:256] == 0)
    nope, rope = oracle.fp8_record_decode(rec)
    assert np.array_equal(rope, x[:, 512:])              # RoPE kept exactly
    # each tile's largest element comes back as amax to within one fp32 ulp of it
    for t in range(4):
        i = np.abs(x[:, 128 * t:128 * (t + 1)]).argmax(axis=1)
        got = np.abs(nope[np.arange(50), 128 * t + i])
        want = amax[:, t]
        assert np.all(np.abs(got - want) <= np.spacing(want.astype(np.float32)).astype(np.float64) + 0.0)
    # elementwise: relative error of e4m3 rounding, scaled
    err = np.abs(nope - x[:, :512]).reshape(50, 4, 128)
    s = scales.astype(np.float64)[:, :, None]
    bound = np.maximum(2.0 ** -4 * np.abs(x[:, :512]).reshape(50, 4, 128), 2.0 ** -10 * s) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_generator_records_agree_with_oracle_encoder():
    # the seeded generator quantises with torch's cast; the oracle's own
    # encoder must produce the same bytes from the same bf16 source
    from workloads import quantize_fp8_records

    g = torch.Generator().manual_seed(3)
    src = torch.randn((6, 16, 576), generator=g).to(torch.bfloat16)
    src[0, 0, :128] = 0
    rec_gen = quantize_fp8_records(src).numpy()
    rec_orc = oracle.fp8_record_encode(src)
    codes_g = rec_gen[..., :512]
    codes_o = rec_orc[..., :512]
    zero = (oracle.e4m3_decode(codes_g) == 0) & (oracle.e4m3_decode(codes_o) == 0)
    assert np.all((codes_g == codes_o) | zero)
    assert np.array_equal(rec_gen[..., 512:], rec_orc[..., 512:])


def test_fp8_decode_equals_bf16_decode_on_dequantised_cache():
    from workloads import make_workload

    w = make_workload(kind="decode", kv_format="fp8", kv_lens=[3, 70, 130], heads=8,
                      page_size=16, seed=4)
    out8, lse8 = oracle.mla_decode_fp8_ref(w.q_nope, w.q_pe, w.kv_fp8, w.kv_indptr, w.kv_indices,
                                           w.kv_len, w.sm_scale)
    assert np.all(np.isfinite(out8))  # poisoned slots never read
    nope, rope = oracle.fp8_record_decode(w.kv_fp8)
    out, lse = oracle.mla_decode_ref(w.q_nope, w.q_pe, nope, rope, w.kv_indptr, w.kv_indices,
                                     w.kv_len, w.sm_scale)
    assert np.array_equal(out, out8) and np.array_equal(lse, lse8)


def test_fp8_query_decode_reduces_to_the_fp8_decode():
    # Every e4m3 value is a bf16 value: the fp8-query oracle must equal the
    # (pinned) fp8-cache decode fed the decoded query as bf16 tensors.
    import torch

    from workloads import make_workload, quantize_q_e4m3

    w = make_workload(kv_lens=[1, 70, 300], heads=8, page_size=16, seed=31, kv_format="fp8")
    q8 = quantize_q_e4m3(w.q_nope, w.q_pe)
    qv = torch.from_numpy(oracle.e4m3_decode(q8.numpy())).to(torch.bfloat16)
    assert torch.equal(qv.to(torch.float64), torch.from_numpy(oracle.e4m3_decode(q8.numpy())))
    o1, l1 = oracle.mla_decode_fp8_q8_ref(q8, w.kv_fp8, w.kv_indptr, w.kv_indices, w.kv_len, w.sm_scale)
    o2, l2 = oracle.mla_decode_fp8_ref(qv[..., :512], qv[..., 512:], w.kv_fp8, w.kv_indptr, w.kv_indices, w.kv_len,
                                       w.sm_scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # the codes are the round-to-nearest e4m3 of the bf16 query (within half an e4m3 step)
    q = torch.cat([w.q_nope, w.q_pe], dim=-1).double().numpy()
    err = np.abs(oracle.e4m3_decode(q8.numpy()) - q)
    assert np.all(err <= np.maximum(np.abs(q) * 2.0 ** -4, 2.0 ** -10) + 1e-12)
