"""Pins of the oracle's MODEL1 pieces: the bf16 rounding, the 604-byte
record (448 e4m3 NoPE codes in 7 tiles of 64, 7 fp32 scales, 64 bf16 RoPE
values) and the decode over it (d = 512 for q.k, V = the 448 NoPE dims)."""

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


def test_hand_built_record():
    # code 0x38 = 1.0, 0x3C = 1.5, 0xB8 = -1.0, 0x7E = 448, 0x01 = 2^-9 (e4m3 definition)
    codes = [0x38] * M1
    codes[0] = 0x3C          # tile 0
    codes[63] = 0xB8         # last dim of tile 0
    codes[64] = 0x7E         # first dim of tile 1
    codes[6 * 64] = 0x01     # first dim of tile 6
    scales = [0.75, 1.1, 2.0, 0.5, 3.0, 0.25, 1024.0]
    rope_bits = [0x3F80] * 64  # bf16 1.0
    rope_bits[5] = 0xC000      # bf16 -2.0
    nope, rope = oracle.model1_record_decode(_record(codes, scales, rope_bits))
    assert nope.shape == (M1,) and rope.shape == (64,)
    assert nope[0] == 1.125                       # 1.5 * 0.75, exact
    assert nope[1] == 0.75 and nope[63] == -0.75  # tile 0 scale on its dims only
    # 448 * fp32(1.1) = 492.8000106... in fp32; bf16 spacing at 2^8 is 2: nearest is 492
    assert nope[64] == 492.0
    assert nope[65] == oracle.f32_to_bf16_rne(np.float32(1.1))  # code 1.0 * 1.1, then bf16
    assert nope[127] == nope[65] and nope[128] == 2.0 and nope[191] == 2.0  # tile 2 starts at dim 128
    assert nope[3 * 64] == 0.5 and nope[4 * 64] == 3.0 and nope[5 * 64] == 0.25
    assert nope[6 * 64] == 2.0 ** -9 * 1024 and nope[6 * 64 + 1] == 1024.0
    assert rope[5] == -2.0 and rope[0] == 1.0 and rope[63] == 1.0


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
    src = x.double().numpy()
    assert np.array_equal(rope, src[:, M1:])
    assert (nope[7, :64] == 0).all()
    tiles = src[:, :M1].reshape(300, 7, 64)
    scale = np.abs(tiles).max(axis=2, keepdims=True) / 448.0
    err = np.abs(nope.reshape(300, 7, 64) - tiles)
    # e4m3 rounding (2^-4 relative for normal codes, half a subnormal step
    # 2^-10 * scale below 2^-6 * scale) plus the bf16 rounding (2^-9 relative)
    bound = np.where(np.abs(tiles) >= 2.0 ** -6 * scale, 2.0 ** -4 * np.abs(tiles), 2.0 ** -10 * scale)
    bound = bound * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(tiles) + 1e-30
    assert (err <= bound).all()
    # each tile's largest magnitude comes back exactly (448 * amax / 448)
    idx = np.abs(tiles).argmax(axis=2)
    got = np.take_along_axis(nope.reshape(300, 7, 64), idx[..., None], 2)
    want = np.take_along_axis(tiles, idx[..., None], 2)
    assert np.array_equal(got, want)


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
