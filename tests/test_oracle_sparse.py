"""Pins of the token-sparse oracle (CPU only).

The sparse oracle is checked against things other than itself:
* brute force with explicit loops and math.fsum on tiny inputs (invalid
  entries, duplicates, a topk_length cut, an attention sink);
* the dense fp8 decode oracle (itself pinned to torch's SDPA and to brute
  force) when a query token's list is exactly its request's keys in order;
* torch's scaled_dot_product_attention / logsumexp / max in float64 for the
  bf16 sparse prefill form;
* closed forms of the sink (it only rescales the output by
  1 / (1 + exp(sink - lse)); a sink equal to one more key with a zero value
  row, built through the rope dims, through the pinned dense ``attend``);
* invariants: list order, dropping invalid or cut entries, no valid key.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from workloads import make_sparse_workload, make_workload


def _tokens_bf16(n, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((n, 576), generator=g).to(torch.bfloat16)


def _q_bf16(t, h, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((t, h, 576), generator=g).to(torch.bfloat16)


def _brute(q, kn, kp, valid_lists, sm_scale, sink):
    """Explicit loops: logits, max, lse and output with the sink as an extra denominator term."""
    q = oracle.as_f64(q)
    T, H, _ = q.shape
    out = np.zeros((T, H, 512))
    lse = np.full((T, H), -math.inf)
    mx = np.full((T, H), -math.inf)
    for t in range(T):
        sel = valid_lists[t]
        for h in range(H):
            if not sel:
                continue
            logits = [sm_scale * math.fsum([q[t, h, d] * kn[j, d] for d in range(512)]
                                           + [q[t, h, 512 + d] * kp[j, d] for d in range(64)]) for j in sel]
            m = max(logits)
            z = math.fsum(math.exp(x - m) for x in logits)
            lse[t, h] = m + math.log(z)
            mx[t, h] = m
            den = z + (math.exp(sink[h] - m) if sink is not None else 0.0)
            for d in range(512):
                out[t, h, d] = math.fsum(math.exp(x - m) * kn[j, d] for x, j in zip(logits, sel)) / den
    return out, lse, mx


def test_sparse_fp8_matches_bruteforce():
    n_slots, H = 12, 2
    rec = oracle.fp8_record_encode(_tokens_bf16(n_slots, 1)).reshape(3, 4, 656)
    kn, kp = oracle.fp8_record_decode(rec.reshape(-1, 656))
    q = _q_bf16(4, H, 2)
    indices = np.array([[3, -1, 7, 3, 12, 0],      # a duplicate, -1, one past the end
                        [11, 10, 9, 8, 7, 6],     # cut to 4 by topk_length
                        [-1, -1, -1, -1, -1, -1],  # nothing valid
                        [5, 99, -7, 2, 1, 4]], dtype=np.int32)
    topk_length = np.array([6, 4, 6, 5], dtype=np.int32)
    valid = [[3, 7, 3, 0], [11, 10, 9, 8], [], [5, 2, 1]]
    sink = np.array([0.7, -1.3])
    for s in (None, sink):
        o, l, m = oracle.mla_sparse_decode_fp8_ref(q, rec, indices, 0.09, topk_length=topk_length, attn_sink=s)
        bo, bl, bm = _brute(q, kn, kp, valid, 0.09, s)
        assert np.allclose(o, bo, rtol=0, atol=1e-12)
        assert np.array_equal(np.isneginf(l), np.isneginf(bl)) and np.array_equal(np.isneginf(m), np.isneginf(bm))
        f = np.isfinite(bl)
        assert np.allclose(l[f], bl[f], rtol=0, atol=1e-12) and np.allclose(m[f], bm[f], rtol=0, atol=1e-12)
        assert np.all(o[2] == 0)


def test_sparse_list_of_all_keys_equals_dense_fp8_decode():
    w = make_workload(kv_lens=[1, 70, 200], heads=8, page_size=16, seed=21, kv_format="fp8")
    ref_o, ref_l = oracle.mla_decode_fp8_ref(w.q_nope, w.q_pe, w.kv_fp8, w.kv_indptr, w.kv_indices, w.kv_len,
                                             w.sm_scale)
    topk = 256
    idx = np.full((w.batch, topk), -1, dtype=np.int64)
    for b in range(w.batch):
        L = int(w.kv_len[b])
        pages = w.kv_indices[int(w.kv_indptr[b]):int(w.kv_indptr[b + 1])].numpy().astype(np.int64)
        j = np.arange(L)
        idx[b, :L] = pages[j // 16] * 16 + j % 16
    q = torch.cat([w.q_nope, w.q_pe], dim=-1)
    o, l, m = oracle.mla_sparse_decode_fp8_ref(q, w.kv_fp8, idx, w.sm_scale)
    assert np.abs(o - ref_o).max() < 1e-12 and np.abs(l - ref_l).max() < 1e-12
    assert np.all(m <= l) and np.all(l - m <= np.log(w.kv_len.numpy())[:, None] + 1e-12)


def test_sparse_prefill_matches_torch_sdpa():
    s_kv, s_q, H, topk = 40, 5, 4, 12
    kv = _tokens_bf16(s_kv, 3)
    q = _q_bf16(s_q, H, 4)
    g = np.random.default_rng(5)
    idx = g.integers(-3, s_kv + 3, size=(s_q, 1, topk)).astype(np.int32)  # [s_q, h_kv, topk]
    idx[1] = -1
    sm = 576 ** -0.5
    o, l, m = oracle.mla_sparse_prefill_ref(q, kv.reshape(s_kv, 1, 576), idx, sm)
    k64 = kv.double()
    for t in range(s_q):
        sel = [int(i) for i in idx[t, 0] if 0 <= i < s_kv]
        if not sel:
            assert np.all(o[t] == 0) and np.all(np.isneginf(l[t])) and np.all(np.isneginf(m[t]))
            continue
        K = k64[torch.tensor(sel)]                           # [n, 576]
        qq = q[t].double()                                   # [H, 576]
        ref = torch.nn.functional.scaled_dot_product_attention(qq[None, :, None, :], K[None, None].expand(1, H, -1, -1),
                                                               K[None, None, :, :512].expand(1, H, -1, -1),
                                                               scale=sm)[0, :, 0]
        logits = (qq @ K.T) * sm
        assert np.abs(o[t] - ref.numpy()).max() < 1e-12
        assert np.abs(l[t] - torch.logsumexp(logits, dim=1).numpy()).max() < 1e-12
        assert np.abs(m[t] - logits.max(dim=1).values.numpy()).max() < 1e-12


def test_sink_only_rescales_the_output():
    w = make_sparse_workload(kv_lens=[300, 90], s_q=2, heads=4, topk=64, page_size=16, seed=7, sink=True,
                             invalid_frac=0.2)
    o0, l0, m0 = oracle.mla_sparse_decode_fp8_ref(w.q, w.kv_fp8, w.indices, w.sm_scale)
    o1, l1, m1 = oracle.mla_sparse_decode_fp8_ref(w.q, w.kv_fp8, w.indices, w.sm_scale, attn_sink=w.attn_sink)
    sink = w.attn_sink.double().numpy()
    assert np.array_equal(l0, l1) and np.array_equal(m0, m1)
    factor = 1.0 / (1.0 + np.exp(sink[None, :] - l0))
    assert np.abs(o1 - o0 * factor[:, :, None]).max() < 1e-12
    # a sink of -inf is no sink; a sink equal to lse halves the output
    oi, _, _ = oracle.mla_sparse_decode_fp8_ref(w.q, w.kv_fp8, w.indices, w.sm_scale,
                                                attn_sink=np.full(4, -np.inf))
    assert np.abs(oi - o0).max() < 1e-15
    oh, _, _ = oracle.mla_sparse_decode_fp8_ref(w.q[:1], w.kv_fp8, w.indices[:1], w.sm_scale, attn_sink=l0[0])
    assert np.abs(oh - 0.5 * o0[:1]).max() < 1e-12


def test_sink_equals_an_extra_key_with_a_zero_value_row():
    # One head: the extra key has nope = 0 and a rope row along q_pe, so its
    # logit x is known exactly; attention over keys + that key (the pinned
    # dense `attend`) equals the sparse result with sink = x.
    rec = oracle.fp8_record_encode(_tokens_bf16(20, 8)).reshape(20, 656)
    q = _q_bf16(1, 1, 9)
    sel = [4, 9, 13, 2, 17]
    idx = np.array([sel + [-1]], dtype=np.int32)
    sm = 0.07
    o, l, _ = oracle.mla_sparse_decode_fp8_ref(q, rec, idx, sm, attn_sink=None)
    qp = oracle.as_f64(q)[0, 0, 512:]
    for c in (0.02, 0.05, -0.03):
        kp_x = oracle.as_f64(torch.from_numpy(c * qp).to(torch.bfloat16))
        x = sm * math.fsum(qp * kp_x)
        kn, kp = oracle.fp8_record_decode(rec[sel])
        kn2 = np.vstack([kn, np.zeros((1, 512))])
        kp2 = np.vstack([kp, kp_x[None, :]])
        qq = oracle.as_f64(q)[0]
        ref_o, ref_l = oracle.attend(qq[:, :512], qq[:, 512:], kn2, kp2, sm, len(sel) + 1)
        so, sl, _ = oracle.mla_sparse_decode_fp8_ref(q, rec, idx, sm, attn_sink=np.array([x]))
        assert np.abs(so[0] - ref_o).max() < 1e-12
        assert abs(np.logaddexp(sl[0, 0], x) - ref_l[0]) < 1e-12 and sl[0, 0] == l[0, 0]


def test_invalid_and_cut_entries_are_ignored_and_order_does_not_matter():
    w = make_sparse_workload(kv_lens=[500, 64, 1], s_q=2, heads=4, topk=96, page_size=16, seed=11,
                             invalid_frac=0.3, topk_min=40)
    o, l, m = oracle.mla_sparse_decode_fp8_ref(w.q, w.kv_fp8, w.indices, w.sm_scale, topk_length=w.topk_length)
    T = w.tokens
    g = np.random.default_rng(12)
    idx = w.indices.numpy().astype(np.int64)
    kept = np.full_like(idx, -1)
    for t in range(T):
        n = int(w.topk_length[t])
        v = idx[t, :n][(idx[t, :n] >= 0) & (idx[t, :n] < w.num_slots)]
        v = v[g.permutation(len(v))]           # another order
        kept[t, :len(v)] = v
        # entries past the cut may hold any slot: they are not read
        idx[t, n:] = g.integers(0, w.num_slots, size=idx.shape[1] - n)
    o2, l2, m2 = oracle.mla_sparse_decode_fp8_ref(w.q, w.kv_fp8, kept, w.sm_scale)
    o3, l3, m3 = oracle.mla_sparse_decode_fp8_ref(w.q, w.kv_fp8, idx, w.sm_scale, topk_length=w.topk_length)
    for a, b in ((o, o2), (l, l2), (m, m2), (o, o3), (l, l3), (m, m3)):
        assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_single_key_and_zero_scale_closed_forms():
    rec = oracle.fp8_record_encode(_tokens_bf16(6, 13)).reshape(6, 656)
    kn, kp = oracle.fp8_record_decode(rec)
    q = _q_bf16(2, 3, 14)
    idx = np.array([[4, -1, -1], [0, 2, 5]], dtype=np.int32)
    o, l, m = oracle.mla_sparse_decode_fp8_ref(q, rec, idx, 0.1)
    qq = oracle.as_f64(q)
    s0 = 0.1 * (qq[0, :, :512] @ kn[4] + qq[0, :, 512:] @ kp[4])
    assert np.abs(o[0] - kn[4][None, :]).max() < 1e-12 and np.abs(l[0] - s0).max() < 1e-12
    assert np.abs(m[0] - s0).max() < 1e-12
    o, l, m = oracle.mla_sparse_decode_fp8_ref(q, rec, idx, 0.0)
    assert np.abs(o[1] - kn[[0, 2, 5]].mean(axis=0)[None, :]).max() < 1e-12
    assert np.abs(l[1] - math.log(3)).max() < 1e-12 and np.all(m[1] == 0)


def test_bad_shapes_are_rejected():
    rec = np.zeros((4, 656), dtype=np.uint8)
    with pytest.raises(ValueError):
        oracle.mla_sparse_decode_fp8_ref(_q_bf16(1, 2, 1)[..., :512], rec, np.zeros((1, 2), np.int32), 0.1)
    with pytest.raises(ValueError):
        oracle.mla_sparse_decode_fp8_ref(_q_bf16(1, 2, 1), rec[:, :600], np.zeros((1, 2), np.int32), 0.1)
