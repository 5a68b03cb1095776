"""Seeded synthetic inputs for paged MLA decode / prefill.

This module only makes inputs.  It holds none of the attention arithmetic
and is shared, as the one common piece, by the tests (which feed the same
bytes to the CPU oracle and to the HIP library), ``bench.py`` and
``__graft_entry__.smoke()``.

Recipe (for workload seed ``k``):

* CPU ``torch.Generator().manual_seed(k)`` draws, in this order: the
  per-request query counts (prefill only), the per-request key counts, and
  the physical page permutation (``randperm`` of the pool).
* Values come next from a generator seeded with ``k`` on the target device
  (the same CPU generator when ``device='cpu'``): ``q_nope``, ``q_pe``, then
  the ckv pool and the kpe pool (fp8: one 576-wide bf16 source pool, which is
  then quantised).  Every value is ``randn`` in fp32 rounded to bf16 (RNE),
  i.e. N(0, 1).
* The pool holds ``pool_factor`` x the pages needed (or an explicit count);
  live pages are taken from the permutation in request order, so request b
  owns ``perm[off_b : off_b + ceil(L_b / page_size)]``.
* With ``poison=True`` every slot no request reads (unused pages and the
  slots past ``kv_len`` in each last page) is NaN (fp8: all-ones bytes, which
  are NaN codes, NaN scales and NaN bf16).  Results must not depend on them.

Token-sparse workloads (:func:`make_sparse_workload`) start from the fp8
decode workload of the same seed (lengths, pages, pool) and then draw from a
second CPU generator seeded ``k + 1`` on the host: for each query token
(request b, MTP position i < s_q) ``min(topk, L_b)`` distinct positions of
``randperm(L_b)``, mapped to flat slots ``page * page_size + offset``
through b's page list and padded with -1 to ``topk``; a fraction
``invalid_frac`` of entries replaced by -1 or by a slot at or past the pool
end (half each); ``topk_length`` ~ U[topk_min, topk] when asked for; the
attention sink ln(topk) + 1.5 + 2 N(0, 1) per head (near the lse of topk
N(0,1) keys at sm_scale 1/sqrt(192), so that it matters); then q [T, H, 576] as N(0,1) bf16 on the target
device from a generator seeded ``k + 1``.

Token-sparse prefill workloads (:func:`make_sparse_prefill_workload`, bf16
KV rows without paging): a CPU generator seeded ``k`` draws the key lists
as ``randint(0, s_kv)`` per entry (repeats allowed, as in the FlashMLA
sparse-prefill example), then invalid entries, ``topk_length`` and the sink
as above; then q [s_q, H, 576] and kv [s_kv, 576] as N(0,1) bf16 from a
generator seeded ``k`` on the target device.

fp8 quantisation of the source pool (the 656-byte record of FlashMLA's
"FP8 KV Cache Quantization and Dequantization"): per token and 128-dim tile,
``scale = amax / 448`` in fp32 and ``code = e4m3(clamp(x / scale, +-448))``
through torch's own ``float8_e4m3fn`` cast (round to nearest even); a
zero tile has scale 0 and codes 0.  Bytes 0..511 codes, 512..527 the four
fp32 scales, 528..655 the 64 bf16 RoPE values.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Union

import torch

HEAD_DIM_CKV = 512
HEAD_DIM_KPE = 64
FP8_RECORD_BYTES = 656

# The five workloads.  Sizes follow the paged-MLA problem statement; names
# say what they are.
CONFIGS = {
    # B=4, H=16, lens [1, 37, 64, 200] over a 16-page permuted pool, fp32 out
    "tiny_decode": dict(seed=1, kind="decode", batch=4, heads=16, page_size=64,
                        kv_lens=[1, 37, 64, 200], pool_pages=16, out_dtype=torch.float32),
    # B=64, H=128, L ~ U[512, 4096], pool 2x the pages needed
    "decode_b64_h128": dict(seed=2, kind="decode", batch=64, heads=128, page_size=64,
                            kv_lens=("uniform", 512, 4096), pool_factor=2),
    # B=128, H=16: 120 requests at 8192 keys + 8 (seeded choice) at 32768
    "decode_b128_h16_skew": dict(seed=3, kind="decode", batch=128, heads=16, page_size=64,
                                 kv_lens=("skew", 8192, 32768, 8), pool_factor=2),
    # 32 requests, q len ~ U[1, 8], L ~ U[1024, 4096], causal, H=128
    "prefill_causal_h128": dict(seed=4, kind="prefill", batch=32, heads=128, page_size=64,
                                q_lens=("uniform", 1, 8), kv_lens=("uniform", 1024, 4096),
                                pool_factor=2, causal=True),
    # B=128, H=128, L ~ U[4096, 16384], 656-byte fp8 records
    "decode_fp8_b128_h128": dict(seed=5, kind="decode", kv_format="fp8", batch=128, heads=128,
                                 page_size=64, kv_lens=("uniform", 4096, 16384), pool_factor=2),
}

# Token-sparse decode over the fp8 records: B=128 requests with L ~ U[4096,
# 16384], s_q = 2 query tokens each (MTP), H=128, 2048 keys per query token
SPARSE_CONFIGS = {
    "sparse_fp8_b128_sq2_h128_topk2048": dict(seed=6, batch=128, s_q=2, heads=128, topk=2048, page_size=64,
                                              kv_lens=("uniform", 4096, 16384), pool_factor=2),
}

# Token-sparse prefill over bf16 KV rows: 4096 query tokens, 32768 KV rows,
# H=128, 2048 keys per query token
SPARSE_PREFILL_CONFIGS = {
    "sparse_prefill_sq4096_skv32768_h128_topk2048": dict(seed=7, s_q=4096, s_kv=32768, heads=128, topk=2048),
}

SM_SCALE_DEFAULT = 1.0 / math.sqrt(192.0)

# MODEL1 record decode at the shape of the 128-head decode (the pool holds
# exactly the live pages, shuffled)
MODEL1_CONFIGS = {
    "decode_model1_b64_h128": dict(seed=12, batch=64, heads=128, page_size=64, kv_lens=("uniform", 512, 4096),
                                   pool_factor=1),
}


@dataclasses.dataclass
class Workload:
    name: str
    kind: str                      # "decode" | "prefill"
    kv_format: str                 # "bf16" | "fp8"
    batch: int
    num_heads: int
    page_size: int
    num_pages: int
    kv_len: torch.Tensor           # int32 [B], CPU
    kv_indptr: torch.Tensor        # int32 [B+1], CPU
    kv_indices: torch.Tensor       # int32 [nnz], CPU
    qo_indptr: Optional[torch.Tensor]  # int32 [B+1], CPU (prefill)
    q_nope: torch.Tensor           # bf16 [rows, H, 512]
    q_pe: torch.Tensor             # bf16 [rows, H, 64]
    ckv: Optional[torch.Tensor]    # bf16 [P, ps, 512]
    kpe: Optional[torch.Tensor]    # bf16 [P, ps, 64]
    kv_fp8: Optional[torch.Tensor]  # uint8 [P, ps, 656]
    sm_scale: float
    out_dtype: torch.dtype
    causal: bool
    seed: int

    @property
    def rows(self) -> int:
        return self.q_nope.shape[0]

    @property
    def device(self) -> torch.device:
        return self.q_nope.device

    def q_lens(self) -> torch.Tensor:
        if self.qo_indptr is None:
            return torch.ones(self.batch, dtype=torch.int32)
        return (self.qo_indptr[1:] - self.qo_indptr[:-1]).to(torch.int32)


def _draw_lens(spec, batch: int, g: torch.Generator) -> torch.Tensor:
    if isinstance(spec, (list, tuple)) and spec and spec[0] == "uniform":
        _, lo, hi = spec
        return torch.randint(lo, hi + 1, (batch,), generator=g, dtype=torch.int64).to(torch.int32)
    if isinstance(spec, (list, tuple)) and spec and spec[0] == "skew":
        _, base, big, n_big = spec
        lens = torch.full((batch,), base, dtype=torch.int32)
        pick = torch.randperm(batch, generator=g)[:n_big]
        lens[pick] = big
        return lens
    return torch.as_tensor(list(spec), dtype=torch.int32)


def _randn_bf16(shape, g: torch.Generator, device, chunk_rows: int = 1024) -> torch.Tensor:
    """N(0,1) fp32 rounded to bf16, generated in fixed chunks of the first dim."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    for i in range(0, shape[0], chunk_rows):
        n = min(chunk_rows, shape[0] - i)
        out[i:i + n] = torch.randn((n,) + tuple(shape[1:]), generator=g, device=device,
                                   dtype=torch.float32).to(torch.bfloat16)
    return out


def quantize_fp8_records(src: torch.Tensor, chunk_pages: int = 2048) -> torch.Tensor:
    """bf16 [P, ps, 576] -> uint8 [P, ps, 656] records (input preparation)."""
    P, ps, D = src.shape
    assert D == HEAD_DIM_CKV + HEAD_DIM_KPE
    out = torch.empty((P, ps, FP8_RECORD_BYTES), dtype=torch.uint8, device=src.device)
    for i in range(0, P, chunk_pages):
        x = src[i:i + chunk_pages]
        n = x.shape[0]
        nope = x[..., :HEAD_DIM_CKV].to(torch.float32).reshape(n, ps, 4, 128)
        amax = nope.abs().amax(dim=-1)
        scale = amax / 448.0
        q = nope / scale.unsqueeze(-1)
        q = torch.where(scale.unsqueeze(-1) == 0, torch.zeros_like(q), q)
        codes = q.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).reshape(n, ps, 512)
        out[i:i + n, :, :512] = codes
        out[i:i + n, :, 512:528] = scale.contiguous().view(torch.uint8).reshape(n, ps, 16)
        out[i:i + n, :, 528:] = x[..., HEAD_DIM_CKV:].contiguous().view(torch.uint8).reshape(n, ps, 128)
    return out


def make_workload(name: Optional[str] = None, *, device: Union[str, torch.device] = "cpu",
                  poison: bool = True, seed: Optional[int] = None, kind: str = "decode",
                  kv_format: str = "bf16", batch: Optional[int] = None, heads: int = 16,
                  page_size: int = 64, kv_lens=None, q_lens=None, pool_pages: Optional[int] = None,
                  pool_factor: int = 2, sm_scale: float = SM_SCALE_DEFAULT,
                  out_dtype: torch.dtype = torch.bfloat16, causal: bool = True) -> Workload:
    """Build one workload: a named one from CONFIGS, or a custom one."""
    if name is not None:
        spec = dict(CONFIGS[name])
        seed = spec.pop("seed") if seed is None else seed
        kind = spec.pop("kind", "decode")
        kv_format = spec.pop("kv_format", "bf16")
        batch = spec.pop("batch")
        heads = spec.pop("heads")
        page_size = spec.pop("page_size")
        kv_lens = spec.pop("kv_lens")
        q_lens = spec.pop("q_lens", None)
        pool_pages = spec.pop("pool_pages", None)
        pool_factor = spec.pop("pool_factor", 2)
        out_dtype = spec.pop("out_dtype", torch.bfloat16)
        causal = spec.pop("causal", True)
    else:
        name = "custom"
        seed = 0 if seed is None else seed
        if batch is None:
            batch = len(kv_lens)
    device = torch.device(device)
    g = torch.Generator().manual_seed(seed)

    if kind == "prefill":
        ql = _draw_lens(q_lens if q_lens is not None else [1] * batch, batch, g)
        qo_indptr = torch.zeros(batch + 1, dtype=torch.int32)
        qo_indptr[1:] = torch.cumsum(ql, 0).to(torch.int32)
    else:
        ql = torch.ones(batch, dtype=torch.int32)
        qo_indptr = None
    lens = _draw_lens(kv_lens, batch, g)
    pages_per = (lens.to(torch.int64) + page_size - 1) // page_size
    needed = int(pages_per.sum())
    if pool_pages is None:
        pool_pages = max(1, pool_factor * needed)
    if pool_pages < needed:
        raise ValueError(f"pool of {pool_pages} pages cannot hold the {needed} needed")
    perm = torch.randperm(pool_pages, generator=g).to(torch.int32)
    kv_indices = perm[:needed].clone()
    kv_indptr = torch.zeros(batch + 1, dtype=torch.int32)
    kv_indptr[1:] = torch.cumsum(pages_per, 0).to(torch.int32)

    gv = g if device.type == "cpu" else torch.Generator(device=device).manual_seed(seed)
    rows = int(ql.sum())
    q_nope = _randn_bf16((rows, heads, HEAD_DIM_CKV), gv, device)
    q_pe = _randn_bf16((rows, heads, HEAD_DIM_KPE), gv, device)
    ckv = kpe = kv_fp8 = None
    if kv_format == "bf16":
        ckv = _randn_bf16((pool_pages, page_size, HEAD_DIM_CKV), gv, device,
                          chunk_rows=max(1, 65536 // page_size))
        kpe = _randn_bf16((pool_pages, page_size, HEAD_DIM_KPE), gv, device,
                          chunk_rows=max(1, 65536 // page_size))
    elif kv_format == "fp8":
        src = _randn_bf16((pool_pages, page_size, HEAD_DIM_CKV + HEAD_DIM_KPE), gv, device,
                          chunk_rows=max(1, 65536 // page_size))
        kv_fp8 = quantize_fp8_records(src)
        del src
    else:
        raise ValueError(kv_format)

    if poison:
        live = torch.zeros(pool_pages * page_size, dtype=torch.bool)
        for b in range(batch):
            L = int(lens[b])
            pg = kv_indices[int(kv_indptr[b]):int(kv_indptr[b + 1])].to(torch.int64)
            slots = (pg[:, None] * page_size + torch.arange(page_size)[None, :]).reshape(-1)[:L]
            live[slots] = True
        dead = (~live).nonzero().reshape(-1).to(device)
        if kv_format == "bf16":
            ckv.view(-1, HEAD_DIM_CKV)[dead] = float("nan")
            kpe.view(-1, HEAD_DIM_KPE)[dead] = float("nan")
        else:
            kv_fp8.view(-1, FP8_RECORD_BYTES)[dead] = 0xFF

    return Workload(name=name, kind=kind, kv_format=kv_format, batch=batch, num_heads=heads,
                    page_size=page_size, num_pages=pool_pages, kv_len=lens, kv_indptr=kv_indptr,
                    kv_indices=kv_indices, qo_indptr=qo_indptr, q_nope=q_nope, q_pe=q_pe,
                    ckv=ckv, kpe=kpe, kv_fp8=kv_fp8, sm_scale=sm_scale, out_dtype=out_dtype,
                    causal=causal, seed=seed)


@dataclasses.dataclass
class SparseWorkload:
    name: str
    batch: int
    s_q: int
    num_heads: int
    topk: int
    page_size: int
    num_pages: int
    kv_len: torch.Tensor                 # int32 [B], CPU
    kv_indptr: torch.Tensor              # int32 [B+1], CPU (page lists the indices were drawn through)
    kv_indices: torch.Tensor             # int32 [nnz], CPU
    q: torch.Tensor                      # bf16 [T, H, 576], T = B * s_q (latent, then rope)
    kv_fp8: torch.Tensor                 # uint8 [P, ps, 656]
    indices: torch.Tensor                # int32 [T, topk] flat slots, -1 / >= P*ps invalid (CPU)
    topk_length: Optional[torch.Tensor]  # int32 [T] (CPU) or None
    attn_sink: Optional[torch.Tensor]    # fp32 [H] (CPU) or None
    sm_scale: float
    out_dtype: torch.dtype
    seed: int

    @property
    def tokens(self) -> int:
        return self.q.shape[0]

    @property
    def num_slots(self) -> int:
        return self.num_pages * self.page_size


def make_sparse_workload(name: Optional[str] = None, *, device: Union[str, torch.device] = "cpu",
                         poison: bool = True, seed: Optional[int] = None, batch: Optional[int] = None,
                         s_q: int = 2, heads: int = 128, topk: int = 2048, page_size: int = 64, kv_lens=None,
                         pool_factor: int = 2, invalid_frac: float = 0.0, topk_min: Optional[int] = None,
                         sink: bool = False, sm_scale: float = SM_SCALE_DEFAULT,
                         out_dtype: torch.dtype = torch.bfloat16) -> SparseWorkload:
    """Build one token-sparse fp8 workload: a named one from SPARSE_CONFIGS, or a custom one."""
    if name is not None:
        spec = dict(SPARSE_CONFIGS[name])
        seed = spec.pop("seed") if seed is None else seed
        batch, s_q, heads, topk = spec.pop("batch"), spec.pop("s_q"), spec.pop("heads"), spec.pop("topk")
        page_size, kv_lens, pool_factor = spec.pop("page_size"), spec.pop("kv_lens"), spec.pop("pool_factor")
    else:
        name = "custom_sparse"
        seed = 0 if seed is None else seed
        if batch is None:
            batch = len(kv_lens)
    base = make_workload(device=device, poison=poison, seed=seed, kind="decode", kv_format="fp8", batch=batch,
                         heads=1, page_size=page_size, kv_lens=kv_lens, pool_factor=pool_factor)
    g = torch.Generator().manual_seed(seed + 1)
    num_slots = base.num_pages * page_size
    T = batch * s_q
    indices = torch.full((T, topk), -1, dtype=torch.int32)
    for b in range(batch):
        L = int(base.kv_len[b])
        pages = base.kv_indices[int(base.kv_indptr[b]):int(base.kv_indptr[b + 1])].to(torch.int64)
        for i in range(s_q):
            n = min(topk, L)
            pos = torch.randperm(L, generator=g)[:n]
            slots = pages[pos // page_size] * page_size + pos % page_size
            indices[b * s_q + i, :n] = slots.to(torch.int32)
    if invalid_frac > 0:
        hit = torch.rand((T, topk), generator=g) < invalid_frac
        past = torch.randint(num_slots, num_slots + 1000, (T, topk), generator=g, dtype=torch.int32)
        kind = torch.rand((T, topk), generator=g) < 0.5
        indices = torch.where(hit, torch.where(kind, torch.full_like(indices, -1), past), indices)
    topk_length = None
    if topk_min is not None:
        topk_length = torch.randint(topk_min, topk + 1, (T,), generator=g, dtype=torch.int64).to(torch.int32)
    attn_sink = (math.log(topk) + 1.5 + 2.0 * torch.randn(heads, generator=g)).to(torch.float32) if sink else None
    dev = torch.device(device)
    gv = torch.Generator().manual_seed(seed + 1) if dev.type == "cpu" else \
        torch.Generator(device=dev).manual_seed(seed + 1)
    q = _randn_bf16((T, heads, HEAD_DIM_CKV + HEAD_DIM_KPE), gv, dev)
    return SparseWorkload(name=name, batch=batch, s_q=s_q, num_heads=heads, topk=topk, page_size=page_size,
                          num_pages=base.num_pages, kv_len=base.kv_len, kv_indptr=base.kv_indptr,
                          kv_indices=base.kv_indices, q=q, kv_fp8=base.kv_fp8, indices=indices,
                          topk_length=topk_length, attn_sink=attn_sink, sm_scale=sm_scale, out_dtype=out_dtype,
                          seed=seed)


@dataclasses.dataclass
class SparsePrefillWorkload:
    name: str
    num_heads: int
    topk: int
    q: torch.Tensor                      # bf16 [s_q, H, 576]
    kv: torch.Tensor                     # bf16 [s_kv, 576]
    indices: torch.Tensor                # int32 [s_q, topk] (CPU), -1 / >= s_kv invalid
    topk_length: Optional[torch.Tensor]  # int32 [s_q] (CPU) or None
    attn_sink: Optional[torch.Tensor]    # fp32 [H] (CPU) or None
    sm_scale: float
    out_dtype: torch.dtype
    seed: int

    @property
    def tokens(self) -> int:
        return self.q.shape[0]

    @property
    def num_slots(self) -> int:
        return self.kv.shape[0]


def make_sparse_prefill_workload(name: Optional[str] = None, *, device: Union[str, torch.device] = "cpu",
                                 seed: Optional[int] = None, s_q: int = 4, s_kv: int = 256, heads: int = 128,
                                 topk: int = 128, invalid_frac: float = 0.0, topk_min: Optional[int] = None,
                                 sink: bool = False, sm_scale: float = SM_SCALE_DEFAULT,
                                 out_dtype: torch.dtype = torch.bfloat16) -> SparsePrefillWorkload:
    """Build one token-sparse prefill workload: named (SPARSE_PREFILL_CONFIGS) or custom."""
    if name is not None:
        spec = dict(SPARSE_PREFILL_CONFIGS[name])
        seed = spec.pop("seed") if seed is None else seed
        s_q, s_kv, heads, topk = spec.pop("s_q"), spec.pop("s_kv"), spec.pop("heads"), spec.pop("topk")
    else:
        name = "custom_sparse_prefill"
        seed = 0 if seed is None else seed
    g = torch.Generator().manual_seed(seed)
    indices = torch.randint(0, s_kv, (s_q, topk), generator=g, dtype=torch.int64).to(torch.int32)
    if invalid_frac > 0:
        hit = torch.rand((s_q, topk), generator=g) < invalid_frac
        past = torch.randint(s_kv, s_kv + 1000, (s_q, topk), generator=g, dtype=torch.int32)
        kind = torch.rand((s_q, topk), generator=g) < 0.5
        indices = torch.where(hit, torch.where(kind, torch.full_like(indices, -1), past), indices)
    topk_length = None
    if topk_min is not None:
        topk_length = torch.randint(topk_min, topk + 1, (s_q,), generator=g, dtype=torch.int64).to(torch.int32)
    attn_sink = (math.log(topk) + 1.5 + 2.0 * torch.randn(heads, generator=g)).to(torch.float32) if sink else None
    dev = torch.device(device)
    gv = g if dev.type == "cpu" else torch.Generator(device=dev).manual_seed(seed)
    q = _randn_bf16((s_q, heads, HEAD_DIM_CKV + HEAD_DIM_KPE), gv, dev)
    kv = _randn_bf16((s_kv, HEAD_DIM_CKV + HEAD_DIM_KPE), gv, dev, chunk_rows=65536)
    return SparsePrefillWorkload(name=name, num_heads=heads, topk=topk, q=q, kv=kv, indices=indices,
                                 topk_length=topk_length, attn_sink=attn_sink, sm_scale=sm_scale,
                                 out_dtype=out_dtype, seed=seed)


def quantize_q_e4m3(q_nope: torch.Tensor, q_pe: torch.Tensor) -> torch.Tensor:
    """[rows, H, 512] + [rows, H, 64] bf16 -> [rows, H, 576] uint8 e4m3 codes of
    the concatenated query (clamp to +-448, then torch's float8_e4m3fn cast,
    round to nearest even; no scale).  Input preparation for the fp8-query
    decode."""
    q = torch.cat([q_nope, q_pe], dim=-1).to(torch.float32).clamp(-448.0, 448.0)
    return q.to(torch.float8_e4m3fn).view(torch.uint8).contiguous()


# MODEL1 records (FlashMLA FP8 section, MODEL1_FP8Sparse: 448 NoPE dims in 7
# tiles of 64, 64 RoPE dims; byte order as the printed 656-byte layout):
# [448 e4m3 codes][7 x fp32 scale][64 x bf16 RoPE] = 604 bytes per token.
MODEL1_NOPE = 448
MODEL1_RECORD_BYTES = 604


def quantize_model1_records(src: torch.Tensor) -> torch.Tensor:
    """bf16 [..., 512] (448 NoPE + 64 RoPE) -> uint8 [..., 604] records (input
    preparation): per 64-dim tile scale = amax / 448 in fp32, codes = the
    float8_e4m3fn cast of x / scale after a clamp to +-448 (round to nearest
    even); a zero tile has scale 0 and codes 0."""
    lead = src.shape[:-1]
    x = src.reshape(-1, MODEL1_NOPE + HEAD_DIM_KPE)
    n = x.shape[0]
    nope = x[:, :MODEL1_NOPE].to(torch.float32).reshape(n, 7, 64)
    scale = nope.abs().amax(dim=-1) / 448.0
    q = nope / scale.unsqueeze(-1)
    q = torch.where(scale.unsqueeze(-1) == 0, torch.zeros_like(q), q)
    out = torch.empty((n, MODEL1_RECORD_BYTES), dtype=torch.uint8, device=src.device)
    out[:, :MODEL1_NOPE] = q.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).reshape(n, MODEL1_NOPE)
    out[:, MODEL1_NOPE:MODEL1_NOPE + 28] = scale.contiguous().view(torch.uint8).reshape(n, 28)
    out[:, MODEL1_NOPE + 28:] = x[:, MODEL1_NOPE:].contiguous().view(torch.uint8).reshape(n, 128)
    return out.reshape(*lead, MODEL1_RECORD_BYTES)


@dataclasses.dataclass
class Model1Workload:
    name: str
    batch: int
    num_heads: int
    page_size: int
    num_pages: int
    q: torch.Tensor           # [B, H, 512] bf16
    records: torch.Tensor     # [num_pages, page_size, 604] uint8
    kv_indptr: torch.Tensor   # [B + 1] int32
    kv_indices: torch.Tensor  # int32
    kv_len: torch.Tensor      # [B] int32
    sm_scale: float
    seed: int


def make_model1_workload(kv_lens=None, *, batch: Optional[int] = None, heads: int = 16, page_size: int = 64, seed: int = 0,
                         device: Union[str, torch.device] = "cpu", pool_factor: int = 2,
                         sm_scale: float = SM_SCALE_DEFAULT, name: str = "custom_model1",
                         poison: bool = True) -> Model1Workload:
    """Decode over MODEL1 records: lengths -> page permutation -> q -> source
    pool (bf16 N(0,1), 512 dims per token) -> records, in that draw order.
    With ``poison`` every record no request reads (unused pages, tail slots)
    is all 0xFF bytes: NaN codes, NaN scales and NaN RoPE values."""
    if kv_lens is None:
        spec = dict(MODEL1_CONFIGS[name])
        seed, batch, heads = spec["seed"], spec["batch"], spec["heads"]
        page_size, kv_lens, pool_factor = spec["page_size"], spec["kv_lens"], spec["pool_factor"]
    if batch is None:
        batch = len(kv_lens)
    g = torch.Generator().manual_seed(seed)
    lens = _draw_lens(kv_lens, batch, g)
    pages_per = (lens.to(torch.int64) + page_size - 1) // page_size
    needed = int(pages_per.sum())
    pool_pages = max(1, pool_factor * needed)
    perm = torch.randperm(pool_pages, generator=g).to(torch.int32)
    kv_indptr = torch.zeros(batch + 1, dtype=torch.int32)
    kv_indptr[1:] = torch.cumsum(pages_per, 0).to(torch.int32)
    device = torch.device(device)
    gv = g if device.type == "cpu" else torch.Generator(device=device).manual_seed(seed)
    q = _randn_bf16((batch, heads, MODEL1_NOPE + HEAD_DIM_KPE), gv, device)
    src = _randn_bf16((pool_pages, page_size, MODEL1_NOPE + HEAD_DIM_KPE), gv, device,
                      chunk_rows=max(1, 65536 // page_size))
    records = quantize_model1_records(src)
    del src
    kv_indices = perm[:needed].clone()
    if poison:
        live = torch.zeros(pool_pages * page_size, dtype=torch.bool)
        for b in range(batch):
            L = int(lens[b])
            pg = kv_indices[int(kv_indptr[b]):int(kv_indptr[b + 1])].to(torch.int64)
            slots = (pg[:, None] * page_size + torch.arange(page_size)[None, :]).reshape(-1)[:L]
            live[slots] = True
        dead = (~live).nonzero().reshape(-1).to(device)
        records.view(-1, MODEL1_RECORD_BYTES)[dead] = 0xFF
    return Model1Workload(name=name, batch=batch, num_heads=heads, page_size=page_size, num_pages=pool_pages,
                          q=q, records=records, kv_indptr=kv_indptr, kv_indices=kv_indices,
                          kv_len=lens.to(torch.int32), sm_scale=sm_scale, seed=seed)
