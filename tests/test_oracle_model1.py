"""Pins of the oracle's MODEL1 pieces: the 604-byte record (448 e4m3 NoPE
codes in 7 tiles of 64, 7 fp32 scales, 64 bf16 RoPE values) decoded to the
exact keys code * scale, the page's BF16 dequantisation of it (with its
rounding), and the decode and token-sparse decode over it (d = 512 for q.k,
V = the 448 NoPE dims)."""

import math
import struct

import numpy as np
import torch

import oracle

M1 = oracle.M1_NOPE
REC = oracle.M1_RECORD_BYTES


def test_record_size():
    assert M1 == 448 and REC == 448 + 7 * 4 + 64 * 2 == 604


def test_bf16_rounding_matches_torch_and_ties_go_to_even():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000) * 100, rng.standard_normal(1000) * 1e-30]).astype(np.float32)
    mine = oracle.f32_to_bf16_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(mine, ref)
    # exact ties between neighbouring bf16 values (spacing 2^-7 in [1, 2))
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 2 + 2.0 ** -7], dtype=np.float32)
    assert list(oracle.f32_to_bf16_rne(ties)) == [1.0, 1 + 2.0 ** -6, -1.0, 2.0]


def _record(codes, scales, rope_bits):
    r = bytearray(REC)
    r[:M1] = bytes(codes)
    r[M1:M1 + 28] = struct.pack("<7f", *scales)
    r[M1 + 28:] = struct.pack("<64H", *rope_bits)
    return np.frombuffer(bytes(r), dtype=np.uint8)


def _hand_built():
    # code 0x38 = 1.0, 0x3C = 1.5, 0xB8 = -1.0, 0x7E = 448, 0x01 = 2^-9 (e4m3 definition)
    codes = [0x38] * M1
    codes[0] = 0x3C          # tile 0
    codes[63] = 0xB8         # last dim of tile 0
    codes[64] = 0x7E         # first dim of tile 1
    codes[6 * 64] = 0x01     # first dim of tile 6
    scales = [0.75, 1.1, 2.0, 0.5, 3.0, 0.25, 1024.0]
    rope_bits = [0x3F80] * 64  # bf16 1.0
    rope_bits[5] = 0xC000      # bf16 -2.0
    return _record(codes, scales, rope_bits)


def test_hand_built_record():
    nope, rope = oracle.model1_record_decode(_hand_built())
    assert nope.shape == (M1,) and rope.shape == (64,)
    s11 = float(np.float32(1.1))                  # the stored fp32 scale of tile 1
    assert nope[0] == 1.125                       # 1.5 * 0.75
    assert nope[1] == 0.75 and nope[63] == -0.75  # tile 0 scale on its dims only
    assert nope[64] == 448 * s11                  # exact product, not rounded: 492.8000106...
    assert nope[64] != 492.0 and abs(nope[64] - 492.80001068115234) < 1e-9
    assert nope[65] == s11 and nope[127] == s11   # code 1.0 times tile 1's scale
    assert nope[128] == 2.0 and nope[191] == 2.0  # tile 2 starts at dim 128
    assert nope[3 * 64] == 0.5 and nope[4 * 64] == 3.0 and nope[5 * 64] == 0.25
    assert nope[6 * 64] == 2.0 ** -9 * 1024 and nope[6 * 64 + 1] == 1024.0
    assert rope[5] == -2.0 and rope[0] == 1.0 and rope[63] == 1.0


def test_hand_built_record_bf16_dequantisation():
    # the page's dequantize_k_cache: fp32 product, then bf16, both to nearest even
    nope, rope = oracle.model1_dequantize_bf16(_hand_built())
    assert nope[0] == 1.125
    assert nope[1] == 0.75 and nope[63] == -0.75
    # 448 * fp32(1.1) = 492.8000106... in fp32; bf16 spacing at 2^8 is 2: nearest is 492
    assert nope[64] == 492.0
    assert nope[65] == oracle.f32_to_bf16_rne(np.float32(1.1))  # code 1.0 * 1.1, then bf16
    assert nope[65] == 1.1015625 and nope[127] == nope[65]
    assert nope[6 * 64] == 2.0 and nope[6 * 64 + 1] == 1024.0
    assert rope[5] == -2.0 and rope[0] == 1.0
    exact, _ = oracle.model1_record_decode(_hand_built())
    assert np.array_equal(nope, oracle.f32_to_bf16_rne(exact.astype(np.float32)))


def test_nan_code_decodes_to_nan():
    codes = [0x38] * M1
    codes[10] = 0x7F
    nope, _ = oracle.model1_record_decode(_record(codes, [1.0] * 7, [0] * 64))
    assert math.isnan(nope[10]) and np.isfinite(np.delete(nope, 10)).all()


def test_round_trip_within_the_quantisation_bound():
    g = torch.Generator().manual_seed(3)
    x = torch.randn((300, M1 + 64), generator=g).to(torch.bfloat16)
    x[7, :64] = 0                      # a zero tile: scale 0, codes 0
    rec = oracle.model1_record_encode(x)
    nope, rope = oracle.model1_record_decode(rec)
    nope16, rope16 = oracle.model1_dequantize_bf16(rec)
    src = x.double().numpy()
    assert np.array_equal(rope, src[:, M1:]) and np.array_equal(rope16, rope)
    assert (nope[7, :64] == 0).all() and (nope16[7, :64] == 0).all()
    tiles = src[:, :M1].reshape(300, 7, 64)
    scale = np.abs(tiles).max(axis=2, keepdims=True) / 448.0
    # e4m3 rounding: 2^-4 relative for normal codes, half a subnormal step
    # 2^-10 * scale below 2^-6 * scale; the scale itself is amax/448 rounded
    # to fp32 (2^-24 relative)
    bound = np.where(np.abs(tiles) >= 2.0 ** -6 * scale, 2.0 ** -4 * np.abs(tiles), 2.0 ** -10 * scale)
    bound = bound * (1 + 2.0 ** -20) + 1e-30
    assert (np.abs(nope.reshape(300, 7, 64) - tiles) <= bound).all()
    # the bf16 dequantisation adds at most half a bf16 ulp (2^-9 relative, with the fp32 step)
    bound16 = bound * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(tiles)
    assert (np.abs(nope16.reshape(300, 7, 64) - tiles) <= bound16).all()
    assert np.array_equal(nope16, oracle.f32_to_bf16_rne(nope.astype(np.float32)))
    # each tile's largest magnitude: 448 * fp32(amax / 448) is amax within one fp32 rounding
    idx = np.abs(tiles).argmax(axis=2)
    got = np.take_along_axis(nope.reshape(300, 7, 64), idx[..., None], 2)
    want = np.take_along_axis(tiles, idx[..., None], 2)
    assert (np.abs(got - want) <= 2.0 ** -23 * np.abs(want)).all()


def _paged(records, lens, page_size, seed):
    """Scatter per-request token records into a shuffled page pool."""
    rng = np.random.default_rng(seed)
    need = [-(-L // page_size) for L in lens]
    P = 2 * sum(need) + 1
    perm = rng.permutation(P)
    pool = np.zeros((P, page_size, REC), dtype=np.uint8)
    indptr = [0]
    indices = []
    t = 0
    for L, n in zip(lens, need):
        pages = perm[len(indices):len(indices) + n]
        for j in range(L):
            pool[pages[j // page_size], j % page_size] = records[t + j]
        indices.extend(pages.tolist())
        indptr.append(len(indices))
        t += L
    return pool, np.array(indptr), np.array(indices)


def test_decode_matches_torch_sdpa_on_the_dequantised_keys():
    g = torch.Generator().manual_seed(5)
    lens, H, ps = [1, 37, 70], 4, 16
    tokens = torch.randn((sum(lens), M1 + 64), generator=g).to(torch.bfloat16)
    rec = oracle.model1_record_encode(tokens)
    pool, indptr, indices = _paged(rec, lens, ps, 6)
    q = torch.randn((len(lens), H, M1 + 64), generator=g).to(torch.bfloat16)
    scale = 1 / math.sqrt(192)
    out, lse = oracle.mla_decode_model1_ref(q, pool, indptr, indices, np.array(lens), scale)
    assert out.shape == (3, H, M1)
    t = 0
    for b, L in enumerate(lens):
        kn, kp = oracle.model1_record_decode(rec[t:t + L])
        k = torch.from_numpy(np.concatenate([kn, kp], axis=1))
        v = torch.from_numpy(kn)
        qb = q[b].double()
        ref = torch.nn.functional.scaled_dot_product_attention(qb[None], k[None], v[None], scale=scale)[0]
        assert np.abs(out[b] - ref.numpy()).max() < 1e-12
        logits = scale * (qb @ k.T)
        assert np.abs(lse[b] - torch.logsumexp(logits, dim=1).numpy()).max() < 1e-12
        t += L
    # one key: the output is that key's NoPE row, lse its logit
    kn0, kp0 = oracle.model1_record_decode(rec[0])
    assert np.abs(out[0] - kn0[None]).max() < 1e-12


def test_padded_576_form_is_the_same_attention():
    """q and keys widened to 576 dims with zeros in dims 448..511 give the
    same output (dims 448..511 zero) and lse through the 576-dim oracle."""
    g = torch.Generator().manual_seed(8)
    lens, H, ps = [5, 90], 3, 8
    tokens = torch.randn((sum(lens), M1 + 64), generator=g).to(torch.bfloat16)
    rec = oracle.model1_record_encode(tokens)
    pool, indptr, indices = _paged(rec, lens, ps, 9)
    q = torch.randn((len(lens), H, M1 + 64), generator=g).to(torch.bfloat16)
    out, lse = oracle.mla_decode_model1_ref(q, pool, indptr, indices, np.array(lens), 0.1)
    kn, kp = oracle.model1_record_decode(pool)
    ckv = np.zeros(pool.shape[:2] + (512,))
    ckv[..., :M1] = kn
    qn = np.zeros((len(lens), H, 512))
    qn[..., :M1] = q[..., :M1].double().numpy()
    o2, l2 = oracle.mla_decode_ref(qn, q[..., M1:].double().numpy(), ckv, kp, indptr, indices, np.array(lens), 0.1)
    assert np.abs(o2[..., :M1] - out).max() < 1e-12 and (o2[..., M1:] == 0).all()
    assert np.abs(l2 - lse).max() < 1e-12


def test_input_quantiser_matches_the_oracle_encoder():
    """workloads.quantize_model1_records (torch casts, input preparation) and
    the oracle's encoder (a search over the code table) write the same bytes."""
    from workloads import quantize_model1_records

    g = torch.Generator().manual_seed(11)
    x = torch.randn((64, 512), generator=g).to(torch.bfloat16)
    x[3, 64:128] = 0
    x[5, :64] *= 1e-3
    a = quantize_model1_records(x).numpy()
    b = oracle.model1_record_encode(x)
    assert np.array_equal(a, b)


def test_sparse_decode_matches_brute_force():
    """Token-sparse decode over MODEL1 records: each query token attends to
    its listed slots (invalid entries skipped, repeats counted), with a sink."""
    g = torch.Generator().manual_seed(12)
    n_slots, T, H, topk = 40, 3, 4, 10
    tokens = torch.randn((n_slots, M1 + 64), generator=g).to(torch.bfloat16)
    rec = oracle.model1_record_encode(tokens).reshape(10, 4, REC)
    q = torch.randn((T, H, M1 + 64), generator=g).to(torch.bfloat16)
    idx = np.array([[0, 5, 5, -1, 39, 40, 7, 1, 2, 3],
                    [-1] * 10,
                    [9, 8, 7, 6, 5, 4, 3, 2, 1, 0]], dtype=np.int32)
    sink = np.array([0.5, -1.0, 3.0, 10.0])
    out, lse, mx = oracle.mla_sparse_decode_model1_ref(q, rec, idx, 0.2, topk_length=np.array([10, 4, 6]),
                                                       attn_sink=sink)
    assert out.shape == (T, H, M1)
    kn_all, kp_all = oracle.model1_record_decode(rec.reshape(-1, REC))
    qd = q.double().numpy()
    for t in range(T):
        sel = [i for i in idx[t][:[10, 4, 6][t]] if 0 <= i < n_slots]
        if not sel:
            assert (out[t] == 0).all() and np.isneginf(lse[t]).all() and np.isneginf(mx[t]).all()
            continue
        s = 0.2 * (qd[t, :, :M1] @ kn_all[sel].T + qd[t, :, M1:] @ kp_all[sel].T)
        for h in range(H):
            m = max(s[h])
            z = math.fsum(math.exp(x - m) for x in s[h])
            assert abs(lse[t, h] - (m + math.log(z))) < 1e-12 and mx[t, h] == m
            den = z * math.exp(m) + math.exp(sink[h])
            want = sum(math.exp(s[h][j]) * kn_all[sel[j]] for j in range(len(sel))) / den
            assert np.abs(out[t, h] - want).max() < 1e-12
