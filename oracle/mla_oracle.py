"""Plain, slow, float64 CPU oracle for paged absorbed-MLA attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Written from the
definition, not from any algorithm for computing it fast: there is no
tiling, no online softmax and no split-K here except in
:func:`merge_partials`, which states the merge identity so tests can check
it.

What is computed (one query row ``r``, one head ``h``):

    s_j   = sm_scale * (q_nope[r,h] . ckv_j + q_pe[r,h] . kpe_j)   j visible
    lse   = ln sum_j exp(s_j)
    out   = sum_j exp(s_j - lse) * ckv_j

Sources, all on the pages named in ``oracle/__init__.py``:

* shapes and the paged inputs: "MLA Paged", sections "decode" and "prefill"
  (``q_nope [.., H, 512]``, ``q_pe [.., H, 64]``,
  ``ckv_cache [num_pages, page_size, 512]``,
  ``kpe_cache [num_pages, page_size, 64]``, ``kv_indptr``/``kv_indices``,
  ``qo_indptr``, outputs ``output [.., H, 512]`` and ``lse [.., H]``);
* the formula: FlashMLA "Sparse MLA Prefill Kernel" (scaled ``Q K^T``, its
  log-sum-exp, ``exp(P - lse)`` weights times the gathered KV).  That
  passage works in base 2 on logits pre-multiplied by log2(e); the natural
  form used here is the same quantity divided by ln 2 (reading: the lse we
  return is the natural log-sum-exp of the ``sm_scale``-scaled logits);
* V is the first 512 dims of the latent key: "mla_decoding_single_batch"
  (V derived as ``K[:, :depth_v]``, not loaded separately);
* causal mask for packed queries: "batch_mla_decode_with_paged_kv_cache"
  (``mask_type`` 'causal' by default).  Reading: bottom-right aligned, i.e.
  query ``i`` of ``n`` in a request with ``L`` keys sees keys
  ``j <= L - n + i``;
* fp8 record: FlashMLA "FP8 KV Cache Quantization and Dequantization"
  (656 bytes per token: 512 e4m3 NoPE codes, 4 fp32 scales, 64 bf16 RoPE;
  tile size 128, four tiles).

Per-request key counts ``kv_len`` are explicit inputs (the pages give
``seq_lens`` / ``cache_seqlens`` for this); a request's logical token ``j``
lives in page ``kv_indices[kv_indptr[b] + j // page_size]`` at slot
``j % page_size`` (the block/offset mapping of FlashMLA's
``abs_indices2indices_in_kvcache``).

Token-sparse attention (:func:`mla_sparse_decode_fp8_ref`,
:func:`mla_sparse_prefill_ref`): the same formula over a per-query-token
list of key slots instead of a request's keys, as in FlashMLA "Sparse MLA
Prefill Kernel" (``focused_kv = kv[indices]``; -1 or an index past the end
is invalid) and "flash_mla_with_kvcache (Sparse Attention with FP8 KV
Cache)" (flat slots ``block * block_size + offset`` into the 656-byte
record cache).  It also returns ``max_logits`` (the largest logit, natural
units) and takes the optional ``topk_length`` and ``attn_sink`` of those
passages; the readings are stated on :func:`sparse_valid_indices` and
:func:`sparse_attend`.
"""

from __future__ import annotations

import math

import numpy as np

HEAD_DIM_CKV = 512
HEAD_DIM_KPE = 64
FP8_TILE = 128
FP8_NUM_TILES = HEAD_DIM_CKV // FP8_TILE
FP8_RECORD_BYTES = HEAD_DIM_CKV + 4 * FP8_NUM_TILES + 2 * HEAD_DIM_KPE  # 656
# MODEL1_FP8Sparse ("FP8 KV Cache Quantization and Dequantization"): 448 NoPE
# dims in 7 tiles of 64, 64 RoPE dims, d = 512 for q.k
M1_NOPE = 448
M1_TILE = 64
M1_NUM_TILES = M1_NOPE // M1_TILE
M1_RECORD_BYTES = M1_NOPE + 4 * M1_NUM_TILES + 2 * HEAD_DIM_KPE  # 604


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16/int16) -> float64, exactly.

    bfloat16 is the upper half of an IEEE binary32: shift the 16 bits up by
    16 and reinterpret as float32 (exact), then widen to float64 (exact).
    """
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def as_f64(x) -> np.ndarray:
    """Any input array (torch CPU tensor or NumPy) -> float64 NumPy, exactly.

    torch bfloat16 tensors are read through their raw bits (the widening is
    done by :func:`bf16_bits_to_f64`, not by torch).  NumPy uint16 arrays are
    taken as bfloat16 bit patterns.
    """
    try:
        import torch  # only used as a container here

        if isinstance(x, torch.Tensor):
            x = x.detach().cpu()
            if x.dtype == torch.bfloat16:
                return bf16_bits_to_f64(x.contiguous().view(torch.int16).numpy())
            return x.numpy().astype(np.float64)
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def _as_int(x) -> np.ndarray:
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().cpu().numpy().astype(np.int64)
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x).astype(np.int64)


def _as_u8(x) -> np.ndarray:
    try:
        import torch

        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype != torch.uint8:
                x = x.view(torch.uint8)
            return x.numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x).view(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """OCP FP8 E4M3 ('fn': finite, no infinities) codes -> float64.

    The pages name ``float8_e4m3`` for the NoPE codes and use
    ``torch.float8_e4m3fn`` for the cache dtype (FlashMLA FP8 sections).
    Bit 7 sign, bits 6..3 exponent with bias 7, bits 2..0 mantissa.
    Exponent 0 is subnormal: m/8 * 2^-6.  Exponent 15 with mantissa 7
    (codes 0x7F, 0xFF) is NaN; every other code is finite (max 448).
    """
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, out)


def e4m3_all_finite_values() -> np.ndarray:
    """Values of the non-negative finite codes 0x00..0x7E, increasing."""
    return e4m3_decode(np.arange(0x7F))


def e4m3_encode(x) -> np.ndarray:
    """float -> E4M3 code: clamp to [-448, 448], then round to nearest, ties
    to the code with even mantissa (round-half-to-even on the significand).

    Written as a search over the table of representable magnitudes, which
    is obviously correct if slow.  Reading (the pages give no rounding
    rule): saturate, then RNE; NaN input is not expected.
    """
    x = np.asarray(x, dtype=np.float64)
    table = e4m3_all_finite_values()  # 127 increasing magnitudes, codes 0..126
    mag = np.minimum(np.abs(x), 448.0)
    hi = np.searchsorted(table, mag, side="left")  # first table >= mag
    hi = np.clip(hi, 0, len(table) - 1)
    lo = np.clip(hi - 1, 0, len(table) - 1)
    d_lo = mag - table[lo]
    d_hi = table[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(mag == table[hi], hi, code)
    neg = np.signbit(x)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def fp8_record_decode(records) -> tuple[np.ndarray, np.ndarray]:
    """656-byte token records -> (nope float64 [..., 512], rope float64 [..., 64]).

    Layout ("FP8 KV Cache Quantization and Dequantization", V32_FP8Sparse):
    bytes 0..511 are 512 e4m3 codes of the NoPE part; bytes 512..527 are
    four little-endian fp32 scales, one per 128-dim tile (tile t covers
    dims [128t, 128t+128)); bytes 528..655 are 64 little-endian bf16 RoPE
    values, stored unquantised.  Dequantised NoPE = code value * scale.
    """
    r = _as_u8(records)
    assert r.shape[-1] == FP8_RECORD_BYTES
    lead = r.shape[:-1]
    flat = r.reshape(-1, FP8_RECORD_BYTES)
    codes = flat[:, :HEAD_DIM_CKV]
    scales = np.ascontiguousarray(flat[:, HEAD_DIM_CKV:HEAD_DIM_CKV + 16]).view("<f4").astype(np.float64)
    rope_bits = np.ascontiguousarray(flat[:, HEAD_DIM_CKV + 16:]).view("<u2")
    vals = e4m3_decode(codes).reshape(-1, FP8_NUM_TILES, FP8_TILE)
    nope = (vals * scales[:, :, None]).reshape(-1, HEAD_DIM_CKV)
    rope = bf16_bits_to_f64(rope_bits)
    return nope.reshape(*lead, HEAD_DIM_CKV), rope.reshape(*lead, HEAD_DIM_KPE)


def fp8_record_encode(tokens) -> np.ndarray:
    """bf16 token rows [..., 576] -> 656-byte records (used only by tests).

    Reading of the quantiser (the pages show only its layout): per token and
    128-dim tile, ``scale = fp32(amax) / 448`` in fp32 (round to nearest),
    codes = e4m3_encode(fp32(x / scale)); a tile of zeros has scale 0 and
    codes 0.  RoPE dims are stored as their bf16 bits.
    """
    x = as_f64(tokens)
    assert x.shape[-1] == HEAD_DIM_CKV + HEAD_DIM_KPE
    lead = x.shape[:-1]
    x = x.reshape(-1, HEAD_DIM_CKV + HEAD_DIM_KPE)
    n = x.shape[0]
    nope = x[:, :HEAD_DIM_CKV].astype(np.float32).reshape(n, FP8_NUM_TILES, FP8_TILE)
    amax = np.abs(nope).max(axis=2)  # exact in fp32
    scale = (amax / np.float32(448.0)).astype(np.float32)  # IEEE fp32 division
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (nope / scale[:, :, None]).astype(np.float32)
    q = np.where(scale[:, :, None] == 0, np.float32(0.0), q)
    codes = e4m3_encode(q.astype(np.float64)).reshape(n, HEAD_DIM_CKV)
    out = np.zeros((n, FP8_RECORD_BYTES), dtype=np.uint8)
    out[:, :HEAD_DIM_CKV] = codes
    out[:, HEAD_DIM_CKV:HEAD_DIM_CKV + 16] = scale.astype("<f4").view(np.uint8).reshape(n, 16)
    rope_f32 = x[:, HEAD_DIM_CKV:].astype(np.float32)
    rope_bits = (rope_f32.view(np.uint32) >> np.uint32(16)).astype("<u2")
    # the rows came from bf16 so the low half is zero: truncation is exact
    out[:, HEAD_DIM_CKV + 16:] = rope_bits.view(np.uint8).reshape(n, 2 * HEAD_DIM_KPE)
    return out.reshape(*lead, FP8_RECORD_BYTES)


def f32_to_bf16_rne(x) -> np.ndarray:
    """float32 values -> the nearest bfloat16 values (ties to even mantissa),
    returned as float64.  Written out on the fp32 bit pattern: add
    0x7FFF plus the lowest kept bit, then clear the low 16 bits (finite
    inputs only; the dequantised keys are bounded by the bf16 source)."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _model1_fields(records):
    """604-byte MODEL1 records -> (codes [n, 448] uint8, scales [n, 7] fp32,
    RoPE float64 [n, 64], leading shape).

    "FP8 KV Cache Quantization and Dequantization" names the MODEL1_FP8Sparse
    layout by its sizes only (d = 512, d_nope = 448, d_rope = 64, tile 64,
    7 tiles); it prints the byte layout of V32_FP8Sparse alone.  Reading:
    the same order as the printed one, packed: bytes 0..447 are the e4m3
    codes (tile t = dims [64t, 64t+64)), bytes 448..475 seven little-endian
    fp32 scales, bytes 476..603 the 64 RoPE values as little-endian bf16.
    """
    r = _as_u8(records)
    assert r.shape[-1] == M1_RECORD_BYTES
    lead = r.shape[:-1]
    flat = r.reshape(-1, M1_RECORD_BYTES)
    codes = flat[:, :M1_NOPE]
    scales = np.ascontiguousarray(flat[:, M1_NOPE:M1_NOPE + 4 * M1_NUM_TILES]).view("<f4")
    rope_bits = np.ascontiguousarray(flat[:, M1_NOPE + 4 * M1_NUM_TILES:]).view("<u2")
    return codes, scales, bf16_bits_to_f64(rope_bits), lead


def model1_record_decode(records) -> tuple[np.ndarray, np.ndarray]:
    """604-byte MODEL1 token records -> (NoPE [..., 448], RoPE [..., 64]) float64.

    The key the attention uses, read as for the 656-byte records: NoPE value
    = code value * its tile's fp32 scale, exactly (an e4m3 value has 4
    significant bits and the scale 24, so the float64 product is exact).
    One reading serves both record formats; the page's dequantize_k_cache,
    which rounds these values to BF16, is :func:`model1_dequantize_bf16`.
    """
    codes, scales, rope, lead = _model1_fields(records)
    vals = e4m3_decode(codes).reshape(-1, M1_NUM_TILES, M1_TILE)
    nope = (vals * scales.astype(np.float64)[:, :, None]).reshape(-1, M1_NOPE)
    return nope.reshape(*lead, M1_NOPE), rope.reshape(*lead, HEAD_DIM_KPE)


def model1_dequantize_bf16(records) -> tuple[np.ndarray, np.ndarray]:
    """The page's dequantize_k_cache for MODEL1 records ("FP8 KV Cache
    Quantization Utilities": it returns the BF16 dequantised cache): NoPE
    value = bf16(fp32(code) * scale), the product rounded to fp32, then to
    bf16, both to nearest even.  (NoPE [..., 448], RoPE [..., 64]) as the
    float64 values of those bf16 numbers.  Not the attention's keys: those
    are the exact products of :func:`model1_record_decode`.
    """
    codes, scales, rope, lead = _model1_fields(records)
    vals = e4m3_decode(codes).astype(np.float32).reshape(-1, M1_NUM_TILES, M1_TILE)
    prod = (vals * scales[:, :, None]).astype(np.float32)  # fp32 multiply
    nope = f32_to_bf16_rne(prod).reshape(-1, M1_NOPE)
    return nope.reshape(*lead, M1_NOPE), rope.reshape(*lead, HEAD_DIM_KPE)


def model1_record_encode(tokens) -> np.ndarray:
    """bf16 token rows [..., 512] (448 NoPE + 64 RoPE) -> 604-byte records
    (used only by tests).  Quantiser as for the 656-byte records, per
    64-dim tile: scale = fp32(amax) / 448, codes = e4m3_encode(fp32(x / scale)),
    a zero tile has scale 0 and codes 0; RoPE stored as its bf16 bits."""
    x = as_f64(tokens)
    assert x.shape[-1] == M1_NOPE + HEAD_DIM_KPE
    lead = x.shape[:-1]
    x = x.reshape(-1, M1_NOPE + HEAD_DIM_KPE)
    n = x.shape[0]
    nope = x[:, :M1_NOPE].astype(np.float32).reshape(n, M1_NUM_TILES, M1_TILE)
    amax = np.abs(nope).max(axis=2)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (nope / scale[:, :, None]).astype(np.float32)
    q = np.where(scale[:, :, None] == 0, np.float32(0.0), q)
    codes = e4m3_encode(q.astype(np.float64)).reshape(n, M1_NOPE)
    out = np.zeros((n, M1_RECORD_BYTES), dtype=np.uint8)
    out[:, :M1_NOPE] = codes
    out[:, M1_NOPE:M1_NOPE + 4 * M1_NUM_TILES] = scale.astype("<f4").view(np.uint8).reshape(n, 4 * M1_NUM_TILES)
    rope_bits = (x[:, M1_NOPE:].astype(np.float32).view(np.uint32) >> np.uint32(16)).astype("<u2")
    out[:, M1_NOPE + 4 * M1_NUM_TILES:] = rope_bits.view(np.uint8).reshape(n, 2 * HEAD_DIM_KPE)
    return out.reshape(*lead, M1_RECORD_BYTES)


def mla_decode_model1_ref(q, kv_records, kv_indptr, kv_indices, kv_len, sm_scale: float, requests=None):
    """Paged decode over MODEL1 records: q [B, H, 512] (448 NoPE + 64 RoPE
    dims), records [num_pages, page_size, 604].  Returns out [B, H, 448],
    lse [B, H] in float64.

    Definition as for the 656-byte records ("MLA Paged" decode; slot
    mapping and sizes from the FlashMLA FP8 section), with d = 512 for
    q . k and, reading, V = the 448 NoPE dims (as V = the 512 NoPE dims
    of the 656-byte layout).  Keys are the exact products code * scale of
    :func:`model1_record_decode`.
    """
    qf = as_f64(q)
    B, H, D = qf.shape
    assert D == M1_NOPE + HEAD_DIM_KPE
    kvl = _as_int(kv_len)
    kv_records = _host(kv_records)
    out = np.zeros((B, H, M1_NOPE))
    lse = np.full((B, H), -np.inf)
    for b in (range(B) if requests is None else requests):
        L = int(kvl[b])
        if L == 0:
            continue
        page, slot = _token_slots(_as_int(kv_indptr), _as_int(kv_indices), b, L, kv_records.shape[1])
        kn, kp = model1_record_decode(_take_rows(kv_records, page, slot))
        o, l = attend(qf[b, :, :M1_NOPE], qf[b, :, M1_NOPE:], kn, kp, sm_scale, L)
        out[b] = o[:, :M1_NOPE]
        lse[b] = l
    return out, lse


# ---------------------------------------------------------------------------
# Paged gather
# ---------------------------------------------------------------------------

def _token_slots(kv_indptr, kv_indices, b: int, kv_len: int, page_size: int):
    """(page, slot) of the logical tokens 0..kv_len-1 of request b.

    "MLA Paged": request b owns pages kv_indices[kv_indptr[b]:kv_indptr[b+1]];
    FlashMLA's slot mapping is block * block_size + offset, i.e. token j is
    at (page j // page_size, offset j % page_size) of that list.
    """
    pages = kv_indices[kv_indptr[b]:kv_indptr[b + 1]]
    need = -(-kv_len // page_size)
    if len(pages) != need:
        raise ValueError(f"request {b}: {len(pages)} pages given for kv_len {kv_len} (need {need})")
    j = np.arange(kv_len)
    return pages[j // page_size], j % page_size


def _host(x):
    """A torch tensor on a device -> one host copy of it (every gather then
    runs on the CPU, so nothing the oracle reads is computed on the device
    under test); anything else as it is."""
    try:
        import torch

        if isinstance(x, torch.Tensor) and x.device.type != "cpu":
            return x.detach().cpu()
    except ImportError:  # pragma: no cover
        pass
    return x


def _take_rows(cache, page, slot):
    """cache[page[i], slot[i], :] for every i, without widening the rest
    (host arrays only: callers pass device tensors through :func:`_host`)."""
    try:
        import torch

        if isinstance(cache, torch.Tensor):
            if cache.device.type != "cpu":
                raise ValueError("the oracle gathers from host memory only")
            return cache.detach()[torch.from_numpy(page), torch.from_numpy(slot)]
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(cache)[page, slot]


def gather_request(ckv_cache, kpe_cache, kv_indptr, kv_indices, b: int, kv_len: int):
    """Logical keys of request b: (ckv [L, 512], kpe [L, 64]) in float64."""
    page, slot = _token_slots(_as_int(kv_indptr), _as_int(kv_indices), b, kv_len, ckv_cache.shape[1])
    return as_f64(_take_rows(ckv_cache, page, slot)), as_f64(_take_rows(kpe_cache, page, slot))


def gather_request_fp8(kv_cache_fp8, kv_indptr, kv_indices, b: int, kv_len: int):
    """Logical keys of request b from 656-byte records, dequantised (float64)."""
    page, slot = _token_slots(_as_int(kv_indptr), _as_int(kv_indices), b, kv_len, kv_cache_fp8.shape[1])
    return fp8_record_decode(_take_rows(kv_cache_fp8, page, slot))


# ---------------------------------------------------------------------------
# Attention for a block of query rows against one request's keys
# ---------------------------------------------------------------------------

def attend(qn, qp, ckv, kpe, sm_scale: float, n_visible):
    """out [R, 512], lse [R] for query rows against keys 0..n_visible[r]-1.

    Definition as in FlashMLA "Sparse MLA Prefill Kernel" (natural-log
    form): logits = sm_scale * (q_nope . ckv + q_pe . kpe) over the 576
    concatenated dims, lse = log-sum-exp of the visible logits, weights
    exp(logit - lse), output = weights @ ckv (V = first 512 dims, per
    "mla_decoding_single_batch").  A row with no visible key gets out = 0
    and lse = -inf (reading: the pages never produce such a row).
    """
    qn = np.asarray(qn, dtype=np.float64)
    qp = np.asarray(qp, dtype=np.float64)
    R = qn.shape[0]
    L = ckv.shape[0]
    n_visible = np.broadcast_to(np.asarray(n_visible, dtype=np.int64), (R,))
    out = np.zeros((R, HEAD_DIM_CKV))
    lse = np.full(R, -np.inf)
    if L == 0:
        return out, lse
    s = sm_scale * (qn @ ckv.T + qp @ kpe.T)  # [R, L]
    visible = np.arange(L)[None, :] < n_visible[:, None]
    s = np.where(visible, s, -np.inf)
    has = n_visible > 0
    m = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
    with np.errstate(invalid="ignore"):
        z = np.exp(s - m[:, None]).sum(axis=1)
    lse = np.where(has, m + np.log(np.where(has, z, 1.0)), -np.inf)
    w = np.where(visible, np.exp(s - np.where(has, lse, 0.0)[:, None]), 0.0)
    out = w @ ckv
    return out, lse


def attend_bruteforce(qn, qp, ckv, kpe, sm_scale: float, n_visible):
    """The same as :func:`attend` with explicit Python loops and math.fsum.

    Only for tiny inputs; it exists to pin :func:`attend`.
    """
    qn = np.asarray(qn, dtype=np.float64)
    qp = np.asarray(qp, dtype=np.float64)
    R = qn.shape[0]
    n_visible = np.broadcast_to(np.asarray(n_visible, dtype=np.int64), (R,))
    out = np.zeros((R, ckv.shape[1]))
    lse = np.full(R, -math.inf)
    for r in range(R):
        n = int(n_visible[r])
        if n == 0:
            continue
        logits = []
        for j in range(n):
            dot = math.fsum([qn[r, d] * ckv[j, d] for d in range(ckv.shape[1])]
                            + [qp[r, d] * kpe[j, d] for d in range(kpe.shape[1])])
            logits.append(sm_scale * dot)
        mx = max(logits)
        total = math.fsum(math.exp(x - mx) for x in logits)
        lse[r] = mx + math.log(total)
        for d in range(ckv.shape[1]):
            out[r, d] = math.fsum(math.exp(logits[j] - lse[r]) * ckv[j, d] for j in range(n))
    return out, lse


def merge_partials(outs, lses):
    """Merge per-chunk results of one row set into the whole-range result.

    "mla_decoding_single_batch" keeps per-row exp-sum and max statistics
    "used for split-K reduction" without printing the merge; it follows from
    the log-sum-exp identity.  With chunk results (o_c normalised within
    the chunk, lse_c):  M = max_c lse_c, w_c = exp(lse_c - M),
    lse = M + ln sum_c w_c, out = sum_c (w_c / sum w) o_c.
    outs: [C, R, D], lses: [C, R].  Chunks with lse = -inf get weight 0.
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    M = lses.max(axis=0)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - Ms[None, :]), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(finite, Ms + np.log(np.where(finite, tot, 1.0)), -np.inf)
    coef = np.where(finite[None, :], w / np.where(finite, tot, 1.0)[None, :], 0.0)
    out = (coef[:, :, None] * outs).sum(axis=0)
    return out, lse


# ---------------------------------------------------------------------------
# The three variants
# ---------------------------------------------------------------------------

def _check_heads(q_nope, q_pe):
    if q_nope.shape[-1] != HEAD_DIM_CKV or q_pe.shape[-1] != HEAD_DIM_KPE:
        raise ValueError("head_dim_ckv must be 512 and head_dim_kpe 64")
    if q_nope.shape[:-1] != q_pe.shape[:-1]:
        raise ValueError("q_nope and q_pe disagree on [rows, heads]")


def mla_decode_ref(q_nope, q_pe, ckv_cache, kpe_cache, kv_indptr, kv_indices, kv_len,
                   sm_scale: float, requests=None):
    """"MLA Paged" decode: one query row per request.

    q_nope [B, H, 512], q_pe [B, H, 64]; returns out [B, H, 512] and
    lse [B, H] in float64.  ``requests`` restricts the work to those
    request indices (other rows are NaN), for sampled checks at full size.
    """
    qn = as_f64(q_nope)
    qp = as_f64(q_pe)
    _check_heads(qn, qp)
    ckv_cache, kpe_cache = _host(ckv_cache), _host(kpe_cache)
    lens = _as_int(kv_len)
    B, H, _ = qn.shape
    out = np.full((B, H, HEAD_DIM_CKV), np.nan)
    lse = np.full((B, H), np.nan)
    for b in (range(B) if requests is None else requests):
        L = int(lens[b])
        Kn, Kp = gather_request(ckv_cache, kpe_cache, kv_indptr, kv_indices, b, L)
        out[b], lse[b] = attend(qn[b], qp[b], Kn, Kp, sm_scale, L)
    return out, lse


def prefill_visible(L: int, n: int, causal: bool) -> np.ndarray:
    """Keys visible to each of the n queries of a request with L keys.

    Causal (the default ``mask_type`` of "batch_mla_decode_with_paged_kv_cache"),
    bottom-right aligned: query i (0-based) sits at position L - n + i and
    sees keys 0..L-n+i.  'dense' sees all L keys.
    """
    i = np.arange(n)
    return (L - n + i + 1) if causal else np.full(n, L)


def mla_prefill_ref(q_nope, q_pe, ckv_cache, kpe_cache, qo_indptr, kv_indptr, kv_indices,
                    kv_len, sm_scale: float, causal: bool = True, requests=None):
    """"MLA Paged" prefill: packed query rows, request b owning rows
    qo_indptr[b]..qo_indptr[b+1]-1 (total_q == qo_indptr[-1]).

    Returns out [total_q, H, 512], lse [total_q, H] in float64.
    """
    qn = as_f64(q_nope)
    qp = as_f64(q_pe)
    _check_heads(qn, qp)
    ckv_cache, kpe_cache = _host(ckv_cache), _host(kpe_cache)
    qo = _as_int(qo_indptr)
    lens = _as_int(kv_len)
    T, H, _ = qn.shape
    if qo[-1] != T:
        raise ValueError("total_q must equal qo_indptr[-1]")
    out = np.full((T, H, HEAD_DIM_CKV), np.nan)
    lse = np.full((T, H), np.nan)
    B = len(qo) - 1
    for b in (range(B) if requests is None else requests):
        L = int(lens[b])
        r0, r1 = int(qo[b]), int(qo[b + 1])
        n = r1 - r0
        if n == 0:
            continue
        if causal and n > L:
            raise ValueError(f"request {b}: {n} queries but only {L} keys under the causal mask")
        Kn, Kp = gather_request(ckv_cache, kpe_cache, kv_indptr, kv_indices, b, L)
        vis = np.repeat(prefill_visible(L, n, causal), H)
        o, l = attend(qn[r0:r1].reshape(n * H, -1), qp[r0:r1].reshape(n * H, -1), Kn, Kp, sm_scale, vis)
        out[r0:r1] = o.reshape(n, H, -1)
        lse[r0:r1] = l.reshape(n, H)
    return out, lse


def mla_decode_fp8_ref(q_nope, q_pe, kv_cache_fp8, kv_indptr, kv_indices, kv_len,
                       sm_scale: float, requests=None):
    """Decode over the 656-byte fp8 record cache [num_pages, page_size, 656].

    The keys are the dequantised records (:func:`fp8_record_decode`); the
    attention is then exactly :func:`mla_decode_ref`'s.
    """
    qn = as_f64(q_nope)
    qp = as_f64(q_pe)
    _check_heads(qn, qp)
    kv_cache_fp8 = _host(kv_cache_fp8)
    lens = _as_int(kv_len)
    B, H, _ = qn.shape
    out = np.full((B, H, HEAD_DIM_CKV), np.nan)
    lse = np.full((B, H), np.nan)
    for b in (range(B) if requests is None else requests):
        L = int(lens[b])
        Kn, Kp = gather_request_fp8(kv_cache_fp8, kv_indptr, kv_indices, b, L)
        out[b], lse[b] = attend(qn[b], qp[b], Kn, Kp, sm_scale, L)
    return out, lse



def mla_decode_fp8_q8_ref(q_codes, kv_cache_fp8, kv_indptr, kv_indices, kv_len, sm_scale: float,
                          requests=None):
    """Decode over the 656-byte records with an fp8 query.

    "mla_decoding_single_batch" allows q_type float8_e4m3fn (output bf16).
    Reading: q_codes [B, H, 576] are e4m3 codes of the 576 query dims
    (latent, then rope), taken at their exact values with no scale; the
    attention is then exactly :func:`mla_decode_fp8_ref`'s.
    """
    q = e4m3_decode(_as_u8(q_codes))
    if q.shape[-1] != HEAD_DIM_CKV + HEAD_DIM_KPE:
        raise ValueError("q must hold 576 codes per head")
    return mla_decode_fp8_ref(q[..., :HEAD_DIM_CKV], q[..., HEAD_DIM_CKV:], kv_cache_fp8, kv_indptr, kv_indices,
                              kv_len, sm_scale, requests=requests)

# ---------------------------------------------------------------------------
# Token-sparse attention (DSA): each query token attends to its own key list
# ---------------------------------------------------------------------------

def sparse_valid_indices(index_row, num_slots: int, topk_length=None) -> np.ndarray:
    """The key slots one query token attends to, in list order.

    FlashMLA "Sparse MLA Prefill Kernel": query i attends to the KV rows
    named by indices[i, :]; an entry of -1, or one at or past the number of
    KV rows, is invalid and ignored.  The optional ``topk_length`` of
    flash_mla_sparse_fwd bounds the entries used; reading: the first
    topk_length[i] entries of row i.  A slot listed twice counts twice (the
    selection is a gather, kv[indices]).
    """
    idx = np.asarray(index_row, dtype=np.int64).reshape(-1)
    if topk_length is not None:
        idx = idx[:max(0, int(topk_length))]
    return idx[(idx >= 0) & (idx < num_slots)]


def sparse_attend(qn, qp, kn, kp, sm_scale: float, attn_sink=None):
    """out [H, 512], lse [H], max_logits [H] of one query token's H heads
    against its gathered keys kn [n, 512], kp [n, 64] (float64).

    The "Sparse MLA Prefill Kernel" formula in natural-log units: logits
    s_j = sm_scale * (q_nope . kn_j + q_pe . kp_j), max_logits = max_j s_j,
    lse = ln sum_j exp(s_j), out = sum_j exp(s_j - lse) kn_j (V = the first
    512 dims).  ``attn_sink`` [H] (reading of the optional per-head sink "for
    output scaling"): one more logit per head that joins the softmax
    denominator and has no value row, out = sum_j exp(s_j) kn_j /
    (sum_j exp(s_j) + exp(sink_h)); lse and max_logits are those of the keys
    alone.  No key: out = 0, lse = max_logits = -inf.
    """
    qn = np.asarray(qn, dtype=np.float64)
    qp = np.asarray(qp, dtype=np.float64)
    H = qn.shape[0]
    if kn.shape[0] == 0:
        return np.zeros((H, kn.shape[1])), np.full(H, -np.inf), np.full(H, -np.inf)
    s = sm_scale * (qn @ kn.T + qp @ kp.T)  # [H, n]
    mx = s.max(axis=1)
    lse = mx + np.log(np.exp(s - mx[:, None]).sum(axis=1))
    denom = lse
    if attn_sink is not None:
        sink = np.asarray(attn_sink, dtype=np.float64).reshape(H)
        denom = np.logaddexp(lse, sink)  # ln(sum_j exp(s_j) + exp(sink))
    out = np.exp(s - denom[:, None]) @ kn
    return out, lse, mx


def _sparse_run(q, indices, num_slots, gather, sm_scale, topk_length, attn_sink, tokens, nope=HEAD_DIM_CKV):
    qq = as_f64(q)
    if qq.shape[-1] != nope + HEAD_DIM_KPE:
        raise ValueError(f"q must hold {nope + HEAD_DIM_KPE} dims per head (latent, then rope)")
    H = qq.shape[-2]
    qq = qq.reshape(-1, H, nope + HEAD_DIM_KPE)
    T = qq.shape[0]
    idx = _as_int(indices)
    idx = idx.reshape(T, -1)
    lens = None if topk_length is None else _as_int(topk_length).reshape(T)
    sink = None if attn_sink is None else as_f64(attn_sink).reshape(H)
    out = np.full((T, H, nope), np.nan)
    lse = np.full((T, H), np.nan)
    mx = np.full((T, H), np.nan)
    for t in (range(T) if tokens is None else tokens):
        sel = sparse_valid_indices(idx[t], num_slots, None if lens is None else lens[t])
        kn, kp = gather(sel)
        out[t], lse[t], mx[t] = sparse_attend(qq[t, :, :nope], qq[t, :, nope:], kn, kp, sm_scale, sink)
    return out, lse, mx


def _flat_rows(cache, width: int, sel):
    """Rows sel of a cache viewed as [num_slots, width] (no widening; host
    arrays only, see :func:`_host`)."""
    try:
        import torch

        if isinstance(cache, torch.Tensor):
            if cache.device.type != "cpu":
                raise ValueError("the oracle gathers from host memory only")
            flat = cache.detach().reshape(-1, width)
            return flat[torch.from_numpy(np.asarray(sel, dtype=np.int64))]
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(cache).reshape(-1, width)[sel]


def mla_sparse_decode_fp8_ref(q, kv_cache_fp8, indices, sm_scale: float, topk_length=None, attn_sink=None,
                              tokens=None):
    """Token-sparse decode over the 656-byte fp8 record cache, as in FlashMLA
    "flash_mla_with_kvcache (Sparse Attention with FP8 KV Cache)".

    q [..., H, 576] bf16 (latent dims, then rope); kv_cache_fp8
    [num_blocks, block_size, (1,) 656]; indices [..., topk] int of flat token
    slots block * block_size + offset (the mapping of
    abs_indices2indices_in_kvcache).  The leading dims of q and indices
    (batch, s_q) are flattened into T query tokens.  topk_length [T] and
    attn_sink [H] are optional.  Returns out [T, H, 512], lse [T, H] and
    max_logits [T, H] in float64; ``tokens`` restricts the work to those
    query tokens (the others are NaN).
    """
    num_slots = int(np.prod(kv_cache_fp8.shape[:-1]))
    if kv_cache_fp8.shape[-1] != FP8_RECORD_BYTES:
        raise ValueError("fp8 records must be 656 bytes")
    kv_cache_fp8 = _host(kv_cache_fp8)
    return _sparse_run(q, indices, num_slots,
                       lambda sel: fp8_record_decode(_flat_rows(kv_cache_fp8, FP8_RECORD_BYTES, sel)),
                       sm_scale, topk_length, attn_sink, tokens)


def mla_sparse_prefill_ref(q, kv, indices, sm_scale: float, topk_length=None, attn_sink=None, tokens=None):
    """FlashMLA "Sparse MLA Prefill Kernel" (flash_mla_sparse_fwd): q [s_q, H, 576]
    bf16, kv [s_kv, (1,) 576] bf16 (one KV head, no paging), indices
    [s_q, (1,) topk] int into the s_kv rows.  Returns out [s_q, H, 512],
    lse [s_q, H], max_logits [s_q, H] in float64 (natural-log units).
    """
    width = HEAD_DIM_CKV + HEAD_DIM_KPE
    if kv.shape[-1] != width:
        raise ValueError("kv must hold 576 dims per token")
    num_slots = int(np.prod(kv.shape[:-1]))
    kv = _host(kv)

    def gather(sel):
        rows = as_f64(_flat_rows(kv, width, sel))
        return rows[:, :HEAD_DIM_CKV], rows[:, HEAD_DIM_CKV:]

    return _sparse_run(q, indices, num_slots, gather, sm_scale, topk_length, attn_sink, tokens)


def mla_sparse_decode_model1_ref(q, kv_records, indices, sm_scale: float, topk_length=None, attn_sink=None,
                                 tokens=None):
    """Token-sparse decode over MODEL1 records ("FP8 KV Cache Quantization and
    Dequantization", MODEL1_FP8Sparse; the sparse decoding passages as for
    :func:`mla_sparse_decode_fp8_ref`): q [..., H, 512] (448 NoPE + 64 RoPE
    dims), kv_records [num_blocks, block_size, (1,) 604], indices [..., topk]
    flat slots.  Keys are the exact products of :func:`model1_record_decode`,
    V = the 448 NoPE dims.  Returns out [T, H, 448], lse [T, H],
    max_logits [T, H] in float64.
    """
    num_slots = int(np.prod(kv_records.shape[:-1]))
    if kv_records.shape[-1] != M1_RECORD_BYTES:
        raise ValueError("MODEL1 records must be 604 bytes")
    kv_records = _host(kv_records)
    return _sparse_run(q, indices, num_slots,
                       lambda sel: model1_record_decode(_flat_rows(kv_records, M1_RECORD_BYTES, sel)),
                       sm_scale, topk_length, attn_sink, tokens, nope=M1_NOPE)
