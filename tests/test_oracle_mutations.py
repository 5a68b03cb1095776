"""Planted mistakes in the oracle must be caught by its pins.

Each case swaps one oracle function for a copy with a plausible mistake (a
dropped term, a wrong sign, an off-by-one, a transposed index, a wrong
base, a wrong tile, a missing renormalisation) and checks that at least one
of the pins in test_oracle_pins / test_oracle_fp8 then fails.  Everything
runs on the CPU.
"""

import math

import numpy as np
import pytest

import oracle
import oracle.mla_oracle as om
from tests import test_oracle_fp8 as fp8pins
from tests import test_oracle_pins as pins


def _pin_suite():
    checks = [
        lambda: pins.test_decode_matches_torch_sdpa(16),
        lambda: pins.test_decode_matches_torch_sdpa(1),
        lambda: pins.test_prefill_matches_torch_sdpa(True),
        lambda: pins.test_single_key_returns_its_row(),
        lambda: pins.test_zero_scale_gives_mean_and_log_count(),
        lambda: pins.test_split_merge_equals_unsplit([64, 128, 129]),
        lambda: pins.test_causal_visibility_boundary(),
        lambda: fp8pins.test_hand_built_record_decodes_as_the_layout_says(),
        lambda: fp8pins.test_record_encoder_layout_and_scales(),
        lambda: fp8pins.test_all_codes_match_torch_float8_e4m3fn(),
    ]
    failed = 0
    for c in checks:
        try:
            c()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    return failed


def _attend_variant(mistake):
    def attend(qn, qp, ckv, kpe, sm_scale, n_visible):
        qn = np.asarray(qn, dtype=np.float64)
        qp = np.asarray(qp, dtype=np.float64)
        R, L = qn.shape[0], ckv.shape[0]
        n_visible = np.broadcast_to(np.asarray(n_visible, dtype=np.int64), (R,))
        if L == 0:
            return np.zeros((R, 512)), np.full(R, -np.inf)
        if mistake == "drop_rope":
            s = sm_scale * (qn @ ckv.T)
        elif mistake == "scale_one_term":
            s = sm_scale * (qn @ ckv.T) + qp @ kpe.T
        elif mistake == "sign":
            s = -sm_scale * (qn @ ckv.T + qp @ kpe.T)
        else:
            s = sm_scale * (qn @ ckv.T + qp @ kpe.T)
        vis_n = n_visible - 1 if mistake == "off_by_one" else n_visible
        visible = np.arange(L)[None, :] < vis_n[:, None]
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, initial=-np.inf)
        m = np.where(np.isfinite(m), m, 0.0)
        z = np.exp(s - m[:, None]).sum(axis=1)
        lse = m + np.log(np.maximum(z, 1e-300))
        if mistake == "base2_lse":
            lse = lse / math.log(2.0)
        w = np.where(visible, np.exp(s - (m if mistake == "unnormalised" else lse)[:, None]), 0.0)
        return w @ ckv, lse
    return attend


@pytest.mark.parametrize("mistake", ["drop_rope", "scale_one_term", "sign", "off_by_one",
                                     "base2_lse", "unnormalised"])
def test_attend_mistakes_are_caught(monkeypatch, mistake):
    assert _pin_suite() == 0  # the real oracle passes
    bad = _attend_variant(mistake)
    monkeypatch.setattr(om, "attend", bad)
    monkeypatch.setattr(oracle, "attend", bad)
    assert _pin_suite() > 0


def test_transposed_slot_mapping_is_caught(monkeypatch):
    def slots(kv_indptr, kv_indices, b, kv_len, page_size):
        pages = kv_indices[kv_indptr[b]:kv_indptr[b + 1]]
        j = np.arange(kv_len)
        return pages[np.minimum(j % page_size, len(pages) - 1)], np.minimum(j // page_size, page_size - 1)
    monkeypatch.setattr(om, "_token_slots", slots)
    assert _pin_suite() > 0


def test_causal_alignment_mistake_is_caught(monkeypatch):
    # top-left instead of bottom-right alignment
    monkeypatch.setattr(om, "prefill_visible", lambda L, n, causal: np.arange(n) + 1 if causal else np.full(n, L))
    assert _pin_suite() > 0


@pytest.mark.parametrize("mistake", ["tile64", "inverse_scale", "rope_big_endian"])
def test_fp8_record_mistakes_are_caught(monkeypatch, mistake):
    real = om.fp8_record_decode

    def decode(records):
        r = om._as_u8(records)
        flat = r.reshape(-1, 656)
        codes = flat[:, :512]
        scales = np.ascontiguousarray(flat[:, 512:528]).view("<f4").astype(np.float64)
        rope_bits = np.ascontiguousarray(flat[:, 528:]).view(">u2" if mistake == "rope_big_endian" else "<u2")
        vals = om.e4m3_decode(codes)
        d = np.arange(512)
        tile = (d // 64) % 4 if mistake == "tile64" else d // 128
        sc = scales[:, tile]
        nope = vals / sc if mistake == "inverse_scale" else vals * sc
        rope = om.bf16_bits_to_f64(rope_bits.astype(np.uint16))
        return nope.reshape(*r.shape[:-1], 512), rope.reshape(*r.shape[:-1], 64)

    assert real is not decode
    monkeypatch.setattr(om, "fp8_record_decode", decode)
    monkeypatch.setattr(oracle, "fp8_record_decode", decode)
    with np.errstate(all="ignore"):
        assert _pin_suite() > 0


def test_merge_without_renormalisation_is_caught(monkeypatch):
    def merge(outs, lses):
        outs = np.asarray(outs)
        lses = np.asarray(lses)
        M = lses.max(axis=0)
        w = np.exp(lses - M[None])
        return (w[:, :, None] * outs).sum(axis=0), M + np.log(w.sum(axis=0))
    monkeypatch.setattr(om, "merge_partials", merge)
    monkeypatch.setattr(oracle, "merge_partials", merge)
    assert _pin_suite() > 0


def test_e4m3_exponent_bias_mistake_is_caught(monkeypatch):
    real = om.e4m3_decode
    monkeypatch.setattr(om, "e4m3_decode", lambda c: real(c) * 2.0)
    monkeypatch.setattr(oracle, "e4m3_decode", lambda c: real(c) * 2.0)
    assert _pin_suite() > 0


# ---------------------------------------------------------------------------
# token-sparse oracle
# ---------------------------------------------------------------------------

from tests import test_oracle_sparse as sparsepins  # noqa: E402


def _sparse_pin_suite():
    checks = [
        sparsepins.test_sparse_fp8_matches_bruteforce,
        sparsepins.test_sparse_list_of_all_keys_equals_dense_fp8_decode,
        sparsepins.test_sparse_prefill_matches_torch_sdpa,
        sparsepins.test_sink_only_rescales_the_output,
        sparsepins.test_sink_equals_an_extra_key_with_a_zero_value_row,
        sparsepins.test_single_key_and_zero_scale_closed_forms,
    ]
    failed = 0
    for c in checks:
        try:
            c()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    return failed


def _valid_variant(mistake):
    def sparse_valid_indices(index_row, num_slots, topk_length=None):
        idx = np.asarray(index_row, dtype=np.int64).reshape(-1)
        if topk_length is not None and mistake != "ignore_topk_length":
            idx = idx[:max(0, int(topk_length) + (1 if mistake == "topk_length_plus_one" else 0))]
        if mistake == "keep_end_slot":
            return idx[(idx >= 0) & (idx <= num_slots)]
        sel = idx[(idx >= 0) & (idx < num_slots)]
        return np.unique(sel) if mistake == "drop_duplicates" else sel
    return sparse_valid_indices


@pytest.mark.parametrize("mistake", ["ignore_topk_length", "topk_length_plus_one", "keep_end_slot",
                                     "drop_duplicates"])
def test_sparse_index_mistakes_are_caught(monkeypatch, mistake):
    assert _sparse_pin_suite() == 0
    monkeypatch.setattr(om, "sparse_valid_indices", _valid_variant(mistake))
    assert _sparse_pin_suite() > 0


def _sparse_attend_variant(mistake):
    def sparse_attend(qn, qp, kn, kp, sm_scale, attn_sink=None):
        qn = np.asarray(qn, dtype=np.float64)
        qp = np.asarray(qp, dtype=np.float64)
        H = qn.shape[0]
        if kn.shape[0] == 0:
            return np.zeros((H, 512)), np.full(H, -np.inf), np.full(H, -np.inf)
        s = sm_scale * (qn @ kn.T + (0 if mistake == "drop_rope" else qp @ kp.T))
        mx = s.max(axis=1)
        lse = mx + np.log(np.exp(s - mx[:, None]).sum(axis=1))
        denom = lse
        if attn_sink is not None and mistake != "sink_ignored":
            sink = np.asarray(attn_sink, dtype=np.float64).reshape(H)
            denom = np.logaddexp(lse, -sink if mistake == "sink_sign" else sink)
        out = np.exp(s - denom[:, None]) @ kn
        if mistake == "sink_in_lse":
            lse = denom
        if mistake == "max_base2":
            mx = mx / math.log(2.0)
        return out, lse, mx
    return sparse_attend


@pytest.mark.parametrize("mistake", ["drop_rope", "sink_ignored", "sink_sign", "sink_in_lse", "max_base2"])
def test_sparse_attend_mistakes_are_caught(monkeypatch, mistake):
    assert _sparse_pin_suite() == 0
    monkeypatch.setattr(om, "sparse_attend", _sparse_attend_variant(mistake))
    assert _sparse_pin_suite() > 0


# ---------------------------------------------------------------------------
# MODEL1 records: planted mistakes in the record decoder and in the decode
# ---------------------------------------------------------------------------

def _model1_pin_suite():
    from tests import test_oracle_model1 as m1

    checks = [
        m1.test_hand_built_record,
        m1.test_hand_built_record_bf16_dequantisation,
        m1.test_round_trip_within_the_quantisation_bound,
        m1.test_sparse_decode_matches_brute_force,
        m1.test_decode_matches_torch_sdpa_on_the_dequantised_keys,
        m1.test_input_quantiser_matches_the_oracle_encoder,
        m1.test_bf16_rounding_matches_torch_and_ties_go_to_even,
    ]
    failed = 0
    for c in checks:
        try:
            c()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    return failed


def _model1_decode_variant(mistake):
    M1, REC = om.M1_NOPE, om.M1_RECORD_BYTES

    def decode(records):
        r = om._as_u8(records)
        lead = r.shape[:-1]
        flat = r.reshape(-1, REC)
        codes = flat[:, :M1]
        s0 = M1 + (4 if mistake == "scale_offset" else 0)
        sc = np.ascontiguousarray(flat[:, s0:s0 + 28]) if mistake != "scale_offset" else \
            np.ascontiguousarray(np.concatenate([flat[:, s0:s0 + 24], flat[:, M1:M1 + 4]], axis=1))
        scales = sc.view("<f4")
        r0 = M1 + 28 + (2 if mistake == "rope_offset" else 0)
        rope_bytes = np.ascontiguousarray(flat[:, r0:r0 + 128]) if mistake != "rope_offset" else \
            np.ascontiguousarray(np.concatenate([flat[:, r0:REC], flat[:, M1 + 28:M1 + 30]], axis=1))
        rope = om.bf16_bits_to_f64(rope_bytes.view("<u2"))
        vals = om.e4m3_decode(codes)
        if mistake == "tile_128":
            tiles = np.repeat(scales[:, :4], 2, axis=1)[:, :7]  # each scale covering 128 dims
        else:
            tiles = scales
        prod = vals.reshape(-1, 7, 64) * tiles.astype(np.float64)[:, :, None]
        if mistake == "bf16_keys":  # the keys rounded as the page's BF16 utility returns them
            prod = om.f32_to_bf16_rne(prod.astype(np.float32))
        elif mistake == "fp32_product":
            prod = prod.astype(np.float32).astype(np.float64)
        nope = prod.reshape(-1, M1)
        return nope.reshape(*lead, M1), rope.reshape(*lead, 64)

    return decode


def _model1_bf16_variant(mistake):
    exact = om.model1_record_decode

    def dequant(records):
        nope, rope = exact(records)
        prod = nope.astype(np.float32)
        if mistake == "no_bf16_rounding":
            out = prod.astype(np.float64)
        else:  # truncate instead of rounding
            u = prod.view(np.uint32) & np.uint32(0xFFFF0000)
            out = u.view(np.float32).astype(np.float64)
        return out, rope

    return dequant


@pytest.mark.parametrize("mistake", ["scale_offset", "rope_offset", "tile_128", "bf16_keys", "fp32_product"])
def test_model1_record_mistakes_are_caught(monkeypatch, mistake):
    assert _model1_pin_suite() == 0  # the real decoder passes every pin
    bad = _model1_decode_variant(mistake)
    monkeypatch.setattr(om, "model1_record_decode", bad)
    monkeypatch.setattr(oracle, "model1_record_decode", bad)
    assert _model1_pin_suite() > 0


@pytest.mark.parametrize("mistake", ["no_bf16_rounding", "truncate"])
def test_model1_bf16_dequantisation_mistakes_are_caught(monkeypatch, mistake):
    assert _model1_pin_suite() == 0
    bad = _model1_bf16_variant(mistake)
    monkeypatch.setattr(om, "model1_dequantize_bf16", bad)
    monkeypatch.setattr(oracle, "model1_dequantize_bf16", bad)
    assert _model1_pin_suite() > 0


def test_model1_decode_without_the_rope_term_is_caught(monkeypatch):
    """A MODEL1 decode whose logits miss the 64 RoPE dims (q.k over the 448
    NoPE dims only)."""
    def decode(q, kv_records, kv_indptr, kv_indices, kv_len, sm_scale, requests=None):
        qf = om.as_f64(q)
        B, H, _ = qf.shape
        kvl = om._as_int(kv_len)
        out = np.zeros((B, H, om.M1_NOPE))
        lse = np.full((B, H), -np.inf)
        for b in range(B):
            L = int(kvl[b])
            if L == 0:
                continue
            page, slot = om._token_slots(om._as_int(kv_indptr), om._as_int(kv_indices), b, L, kv_records.shape[1])
            kn, kp = om.model1_record_decode(om._take_rows(kv_records, page, slot))
            o, l = om.attend(qf[b, :, :om.M1_NOPE], np.zeros_like(qf[b, :, om.M1_NOPE:]), kn, kp, sm_scale, L)
            out[b], lse[b] = o[:, :om.M1_NOPE], l
        return out, lse
    monkeypatch.setattr(om, "mla_decode_model1_ref", decode)
    monkeypatch.setattr(oracle, "mla_decode_model1_ref", decode)
    assert _model1_pin_suite() > 0
