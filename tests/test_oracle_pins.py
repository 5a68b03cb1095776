"""Pins of the float64 oracle against things other than itself.

* brute force (explicit loops, math.fsum) on tiny inputs;
* torch's scaled_dot_product_attention and logsumexp in float64 on CPU,
  fed a dense K/V built here by an independent page scatter;
* closed forms (single key, sm_scale = 0, identical logits, logit shift);
* invariants (physical page permutation, key order, split merge, prefill
  with one query = decode, last causal row = decode, page_size re-view,
  head permutation, causal visibility boundary).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.mla_oracle import prefill_visible

D_CKV, D_KPE = 512, 64


def dense_to_paged(K_list, page_size, pool_pages, rng):
    """Scatter each request's dense keys [L, 576] into a permuted page pool.

    Written independently of the oracle's gather: pages are handed out from a
    random permutation, token j of a request goes to (its (j // ps)-th page,
    slot j % ps).  Unused slots are NaN.
    """
    need = [-(-len(K) // page_size) for K in K_list]
    perm = rng.permutation(pool_pages)
    pool = np.full((pool_pages, page_size, D_CKV + D_KPE), np.nan)
    indptr = [0]
    indices = []
    off = 0
    for K, n in zip(K_list, need):
        pages = perm[off:off + n]
        off += n
        for j in range(len(K)):
            pool[pages[j // page_size], j % page_size] = K[j]
        indices.extend(pages.tolist())
        indptr.append(indptr[-1] + n)
    return (pool[..., :D_CKV], pool[..., D_CKV:], np.array(indptr, dtype=np.int32),
            np.array(indices, dtype=np.int32))


def sdpa_f64(q576, K576, sm_scale, mask):
    """torch SDPA (math path, float64, CPU); V = first 512 dims of K."""
    q = torch.from_numpy(q576)[None]          # [1, R, 576]
    k = torch.from_numpy(K576)[None]          # [1, L, 576]
    v = torch.from_numpy(np.ascontiguousarray(K576[:, :D_CKV]))[None]
    m = torch.from_numpy(mask)[None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=sm_scale)
    return o[0].numpy()


def lse_f64(q576, K576, sm_scale, mask):
    s = torch.from_numpy(sm_scale * (q576 @ K576.T))
    s = s.masked_fill(~torch.from_numpy(mask), -math.inf)
    return torch.logsumexp(s, dim=-1).numpy()


def rand(rng, *shape):
    return rng.standard_normal(shape)


# --------------------------------------------------------------------------
# brute force
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_attend_matches_bruteforce(seed):
    rng = np.random.default_rng(seed)
    R, L = 4, 7
    qn, qp = rand(rng, R, D_CKV), rand(rng, R, D_KPE)
    Kn, Kp = rand(rng, L, D_CKV), rand(rng, L, D_KPE)
    vis = np.array([7, 1, 4, 0])
    o1, l1 = oracle.attend(qn, qp, Kn, Kp, 0.05, vis)
    o2, l2 = oracle.attend_bruteforce(qn, qp, Kn, Kp, 0.05, vis)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    assert np.max(np.abs(l1[:3] - l2[:3])) < 1e-12
    assert l1[3] == -np.inf and l2[3] == -np.inf and np.all(o1[3] == 0)


def test_decode_matches_bruteforce_through_pages():
    rng = np.random.default_rng(3)
    lens = [1, 5, 9]
    H = 2
    K_list = [rand(rng, L, D_CKV + D_KPE) for L in lens]
    ckv, kpe, indptr, indices = dense_to_paged(K_list, 4, 12, rng)
    qn, qp = rand(rng, 3, H, D_CKV), rand(rng, 3, H, D_KPE)
    out, lse = oracle.mla_decode_ref(qn, qp, ckv, kpe, indptr, indices, lens, 0.1)
    for b, K in enumerate(K_list):
        o2, l2 = oracle.attend_bruteforce(qn[b], qp[b], K[:, :D_CKV], K[:, D_CKV:], 0.1, len(K))
        assert np.max(np.abs(out[b] - o2)) < 1e-12
        assert np.max(np.abs(lse[b] - l2)) < 1e-12


# --------------------------------------------------------------------------
# library routines (torch SDPA / logsumexp, float64, CPU)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("page_size", [1, 16, 64])
def test_decode_matches_torch_sdpa(page_size):
    rng = np.random.default_rng(10 + page_size)
    lens = [1, 37, 64, 200]
    H = 16
    sm = 1 / math.sqrt(192)
    K_list = [rand(rng, L, D_CKV + D_KPE) for L in lens]
    need = sum(-(-L // page_size) for L in lens)
    ckv, kpe, indptr, indices = dense_to_paged(K_list, page_size, 2 * need, rng)
    qn, qp = rand(rng, 4, H, D_CKV), rand(rng, 4, H, D_KPE)
    out, lse = oracle.mla_decode_ref(qn, qp, ckv, kpe, indptr, indices, lens, sm)
    for b, K in enumerate(K_list):
        q = np.concatenate([qn[b], qp[b]], axis=1)
        mask = np.ones((H, len(K)), dtype=bool)
        ref_o = sdpa_f64(q, K, sm, mask)
        ref_l = lse_f64(q, K, sm, mask)
        assert np.max(np.abs(out[b] - ref_o)) < 1e-12
        assert np.max(np.abs(lse[b] - ref_l)) < 1e-12


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_matches_torch_sdpa(causal):
    rng = np.random.default_rng(20 + causal)
    lens = [3, 40, 70]
    qlens = [3, 1, 5]
    H = 4
    sm = 0.09
    K_list = [rand(rng, L, D_CKV + D_KPE) for L in lens]
    ckv, kpe, indptr, indices = dense_to_paged(K_list, 16, 16, rng)
    qo = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    T = int(qo[-1])
    qn, qp = rand(rng, T, H, D_CKV), rand(rng, T, H, D_KPE)
    out, lse = oracle.mla_prefill_ref(qn, qp, ckv, kpe, qo, indptr, indices, lens, sm, causal=causal)
    for b, K in enumerate(K_list):
        L, n = len(K), qlens[b]
        for i in range(n):
            r = qo[b] + i
            q = np.concatenate([qn[r], qp[r]], axis=1)
            # bottom-right causal: query i sits at key position L - n + i
            mask = np.tile(np.arange(L) <= (L - n + i) if causal else np.ones(L, bool), (H, 1))
            assert np.max(np.abs(out[r] - sdpa_f64(q, K, sm, mask))) < 1e-12
            assert np.max(np.abs(lse[r] - lse_f64(q, K, sm, mask))) < 1e-12


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def test_single_key_returns_its_row():
    rng = np.random.default_rng(5)
    qn, qp = rand(rng, 3, D_CKV), rand(rng, 3, D_KPE)
    Kn, Kp = rand(rng, 1, D_CKV), rand(rng, 1, D_KPE)
    o, l = oracle.attend(qn, qp, Kn, Kp, 0.3, 1)
    assert np.array_equal(o, np.repeat(Kn, 3, axis=0))
    s0 = 0.3 * (qn @ Kn[0] + qp @ Kp[0])
    assert np.max(np.abs(l - s0)) < 1e-12


def test_zero_scale_gives_mean_and_log_count():
    rng = np.random.default_rng(6)
    L = 33
    qn, qp = rand(rng, 2, D_CKV), rand(rng, 2, D_KPE)
    Kn, Kp = rand(rng, L, D_CKV), rand(rng, L, D_KPE)
    o, l = oracle.attend(qn, qp, Kn, Kp, 0.0, L)
    assert np.max(np.abs(o - Kn.mean(axis=0))) < 1e-13
    assert np.max(np.abs(l - math.log(L))) < 1e-13


def test_identical_logits_give_mean_of_values():
    # q_nope = 0 and all kpe rows equal: every key has the same logit, the
    # values (ckv rows) differ -> the output is their mean.
    rng = np.random.default_rng(7)
    L = 17
    qn = np.zeros((2, D_CKV))
    qp = rand(rng, 2, D_KPE)
    Kn = rand(rng, L, D_CKV)
    Kp = np.tile(rand(rng, 1, D_KPE), (L, 1))
    o, l = oracle.attend(qn, qp, Kn, Kp, 0.2, L)
    assert np.max(np.abs(o - Kn.mean(axis=0))) < 1e-13
    s = 0.2 * (qp @ Kp[0])
    assert np.max(np.abs(l - (s + math.log(L)))) < 1e-12


def test_logit_shift_moves_lse_only():
    rng = np.random.default_rng(8)
    L = 20
    qn, qp = rand(rng, 3, D_CKV), rand(rng, 3, D_KPE)
    Kn, Kp = rand(rng, L, D_CKV), rand(rng, L, D_KPE)
    Kp[:, 0] = 1.0  # a constant feature: q_pe[:, 0] adds the same amount to every logit
    o1, l1 = oracle.attend(qn, qp, Kn, Kp, 0.1, L)
    qp2 = qp.copy()
    qp2[:, 0] += 7.0
    o2, l2 = oracle.attend(qn, qp2, Kn, Kp, 0.1, L)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    assert np.max(np.abs((l2 - l1) - 0.7)) < 1e-12


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def _small_paged(seed, lens, page_size=16, H=4):
    rng = np.random.default_rng(seed)
    K_list = [rand(rng, L, D_CKV + D_KPE) for L in lens]
    need = sum(-(-L // page_size) for L in lens)
    ckv, kpe, indptr, indices = dense_to_paged(K_list, page_size, 2 * need + 1, rng)
    qn, qp = rand(rng, len(lens), H, D_CKV), rand(rng, len(lens), H, D_KPE)
    return rng, K_list, ckv, kpe, indptr, indices, qn, qp


def test_physical_page_permutation_is_exact():
    lens = [5, 33, 64]
    rng, K_list, ckv, kpe, indptr, indices, qn, qp = _small_paged(11, lens)
    o1, l1 = oracle.mla_decode_ref(qn, qp, ckv, kpe, indptr, indices, lens, 0.1)
    P = ckv.shape[0]
    perm = rng.permutation(P)          # new position of old page p is perm[p]
    ckv2 = np.empty_like(ckv)
    kpe2 = np.empty_like(kpe)
    ckv2[perm] = ckv
    kpe2[perm] = kpe
    o2, l2 = oracle.mla_decode_ref(qn, qp, ckv2, kpe2, indptr, perm[indices], lens, 0.1)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_key_order_does_not_matter_in_decode():
    rng = np.random.default_rng(12)
    L = 50
    qn, qp = rand(rng, 4, D_CKV), rand(rng, 4, D_KPE)
    Kn, Kp = rand(rng, L, D_CKV), rand(rng, L, D_KPE)
    p = rng.permutation(L)
    o1, l1 = oracle.attend(qn, qp, Kn, Kp, 0.1, L)
    o2, l2 = oracle.attend(qn, qp, Kn[p], Kp[p], 0.1, L)
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12


@pytest.mark.parametrize("cuts", [[10], [1, 2, 3], [64, 128, 129], [0, 0, 200]])
def test_split_merge_equals_unsplit(cuts):
    rng = np.random.default_rng(13)
    L = 200
    qn, qp = rand(rng, 5, D_CKV), rand(rng, 5, D_KPE)
    Kn, Kp = rand(rng, L, D_CKV) * 3, rand(rng, L, D_KPE) * 3
    o, l = oracle.attend(qn, qp, Kn, Kp, 0.2, L)
    bounds = [0] + list(cuts) + [L]
    outs, lses = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        oc, lc = oracle.attend(qn, qp, Kn[a:b], Kp[a:b], 0.2, b - a)
        outs.append(oc)
        lses.append(lc)
    om, lm = oracle.merge_partials(outs, lses)
    assert np.max(np.abs(om - o)) < 1e-12 and np.max(np.abs(lm - l)) < 1e-12


def test_merge_of_all_empty_is_empty():
    om, lm = oracle.merge_partials(np.zeros((2, 3, 4)), np.full((2, 3), -np.inf))
    assert np.all(om == 0) and np.all(lm == -np.inf)


def test_prefill_single_query_equals_decode_and_last_row_equals_decode():
    lens = [9, 40]
    rng, K_list, ckv, kpe, indptr, indices, qn, qp = _small_paged(14, lens)
    od, ld = oracle.mla_decode_ref(qn, qp, ckv, kpe, indptr, indices, lens, 0.1)
    qo = np.array([0, 1, 2], dtype=np.int32)
    op, lp = oracle.mla_prefill_ref(qn, qp, ckv, kpe, qo, indptr, indices, lens, 0.1, causal=True)
    assert np.max(np.abs(op - od)) < 1e-14 and np.max(np.abs(lp - ld)) < 1e-14
    # three queries for request 1: its last row sees all keys, like decode
    H = qn.shape[1]
    q3n = np.concatenate([qn[:1], rand(rng, 2, H, D_CKV), qn[1:2]])
    q3p = np.concatenate([qp[:1], rand(rng, 2, H, D_KPE), qp[1:2]])
    qo3 = np.array([0, 1, 4], dtype=np.int32)
    o3, l3 = oracle.mla_prefill_ref(q3n, q3p, ckv, kpe, qo3, indptr, indices, lens, 0.1, causal=True)
    assert np.max(np.abs(o3[3] - od[1])) < 1e-14 and np.max(np.abs(l3[3] - ld[1])) < 1e-14


def test_causal_visibility_boundary():
    # changing key L-n+i changes row i; changing key L-n+i+1 does not
    L, n = 30, 4
    rng = np.random.default_rng(15)
    K = rand(rng, L, D_CKV + D_KPE)
    ckv, kpe, indptr, indices = dense_to_paged([K], 8, 8, rng)
    qn, qp = rand(rng, n, 2, D_CKV), rand(rng, n, 2, D_KPE)
    qo = np.array([0, n], dtype=np.int32)
    o1, _ = oracle.mla_prefill_ref(qn, qp, ckv, kpe, qo, indptr, indices, [L], 0.1)
    assert list(prefill_visible(L, n, True)) == [27, 28, 29, 30]
    i = 1
    edge = L - n + i
    for j, changes in [(edge, True), (edge + 1, False)]:
        K2 = K.copy()
        K2[j] += 1.0
        # same page placement as the first call, one key changed
        c2 = ckv.copy()
        k2 = kpe.copy()
        page = indices[j // 8]
        c2[page, j % 8] = K2[j, :D_CKV]
        k2[page, j % 8] = K2[j, D_CKV:]
        o2, _ = oracle.mla_prefill_ref(qn, qp, c2, k2, qo, indptr, indices, [L], 0.1)
        assert (np.max(np.abs(o2[i] - o1[i])) > 1e-6) == changes


def test_page_size_review_is_exact():
    # the same pool viewed with page_size 1 and expanded indices
    lens = [7, 40]
    rng, K_list, ckv, kpe, indptr, indices, qn, qp = _small_paged(16, lens, page_size=16)
    o1, l1 = oracle.mla_decode_ref(qn, qp, ckv, kpe, indptr, indices, lens, 0.1)
    ckv1 = ckv.reshape(-1, 1, D_CKV)
    kpe1 = kpe.reshape(-1, 1, D_KPE)
    idx1, ptr1 = [], [0]
    for b, L in enumerate(lens):
        pages = indices[indptr[b]:indptr[b + 1]]
        idx1.extend(int(pages[j // 16]) * 16 + j % 16 for j in range(L))
        ptr1.append(len(idx1))
    o2, l2 = oracle.mla_decode_ref(qn, qp, ckv1, kpe1, np.array(ptr1), np.array(idx1), lens, 0.1)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_head_permutation_permutes_outputs():
    lens = [12, 20]
    rng, K_list, ckv, kpe, indptr, indices, qn, qp = _small_paged(17, lens)
    o1, l1 = oracle.mla_decode_ref(qn, qp, ckv, kpe, indptr, indices, lens, 0.1)
    p = rng.permutation(qn.shape[1])
    o2, l2 = oracle.mla_decode_ref(qn[:, p], qp[:, p], ckv, kpe, indptr, indices, lens, 0.1)
    assert np.array_equal(o1[:, p], o2) and np.array_equal(l1[:, p], l2)


def test_page_count_mismatch_is_rejected():
    lens = [20]
    rng, K_list, ckv, kpe, indptr, indices, qn, qp = _small_paged(18, lens)
    with pytest.raises(ValueError):
        oracle.mla_decode_ref(qn, qp, ckv, kpe, indptr, indices, [40], 0.1)


def test_bf16_widening_is_exact():
    x = torch.randn(1000).to(torch.bfloat16)
    assert np.array_equal(oracle.as_f64(x), x.to(torch.float64).numpy())


def test_workload_inputs_feed_the_oracle():
    # the seeded generator and the oracle agree on shapes / page bookkeeping
    from workloads import make_workload

    w = make_workload("tiny_decode")
    assert w.kv_len.tolist() == [1, 37, 64, 200]
    assert w.kv_indptr.tolist() == [0, 1, 2, 3, 7]
    assert sorted(set(w.kv_indices.tolist())) == sorted(w.kv_indices.tolist())
    out, lse = oracle.mla_decode_ref(w.q_nope, w.q_pe, w.ckv, w.kpe, w.kv_indptr, w.kv_indices,
                                     w.kv_len, w.sm_scale)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))  # poison never read
    # request 0 has a single key: its output is that key's ckv row
    p0 = int(w.kv_indices[0])
    row = oracle.as_f64(w.ckv[p0, 0])
    assert np.array_equal(out[0], np.tile(row, (w.num_heads, 1)))
