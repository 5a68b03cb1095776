"""ctypes binding of libmla.so (argument marshalling only)."""

from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))

MLA_OK = 0
MLA_KIND_DECODE = 0
MLA_KIND_PREFILL = 1
MLA_KIND_SPARSE_DECODE = 2
MLA_KV_BF16 = 0
MLA_KV_FP8_E4M3_T128 = 1
MLA_KV_FP8_MODEL1 = 2
MLA_DTYPE_BF16 = 0
MLA_DTYPE_FP32 = 1
MLA_TILE_AUTO = 0
MLA_TILE_WIDE = 1
MLA_TILE_NARROW = 2
MLA_TILE_QUAD = 3
MLA_LSE_ROWS = 0
MLA_LSE_HEADS_FIRST = 1
MLA_ERR_INVALID_ARGUMENT = -1

_DIM_CKV = 512
_DIM_KPE = 64
_FP8_RECORD = 656


class MLAError(RuntimeError):
    """A status other than MLA_OK from the library (or a missing library)."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status}")


class _Desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "kind", "batch", "num_qo_heads", "head_dim_ckv", "head_dim_kpe", "page_size", "num_pages",
        "kv_format", "causal", "num_cus", "max_splits", "force_splits", "tile_mode", "validate", "lse_layout",
        "max_kv_len", "max_seq_len_q")]


_lib = None
_lock = threading.Lock()


def lib_path() -> str:
    return os.environ.get("MLA_LIBRARY", os.path.join(_HERE, "libmla.so"))


def load_library():
    """Load libmla.so once; raise MLAError if it is not there."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = lib_path()
        if not os.path.exists(path):
            raise MLAError(-5, f"libmla.so not built ({path}); run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
        pi32 = ctypes.POINTER(ctypes.c_int32)
        L.mla_plan_create.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(_Desc), pi32, pi32, pi32]
        L.mla_plan_create.restype = i32
        L.mla_plan_destroy.argtypes = [vp]
        L.mla_plan_destroy.restype = None
        L.mla_plan_workspace_bytes.argtypes = [vp]
        L.mla_plan_workspace_bytes.restype = sz
        L.mla_plan_num_work_items.argtypes = [vp]
        L.mla_plan_num_work_items.restype = i32
        L.mla_plan_num_split_groups.argtypes = [vp]
        L.mla_plan_num_split_groups.restype = i32
        L.mla_plan_get_work_items.argtypes = [vp, pi32, sz]
        L.mla_plan_get_work_items.restype = i32
        L.mla_plan_num_workgroups.argtypes = [vp]
        L.mla_plan_num_workgroups.restype = i32
        L.mla_plan_group_size.argtypes = [vp]
        L.mla_plan_group_size.restype = i32
        L.mla_plan_get_workgroup_ptr.argtypes = [vp, pi32, sz]
        L.mla_plan_get_workgroup_ptr.restype = i32
        L.mla_plan_upload.argtypes = [vp, vp, sz, vp]
        L.mla_plan_upload.restype = i32
        L.mla_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, f32, vp, i32, vp, vp, sz, vp]
        L.mla_decode.restype = i32
        L.mla_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, i32, vp, vp, sz, vp]
        L.mla_prefill.restype = i32
        L.mla_decode_live.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, i32, vp, vp, sz, vp]
        L.mla_decode_live.restype = i32
        L.mla_prefill_live.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, i32, vp, vp, sz, vp]
        L.mla_prefill_live.restype = i32
        L.mla_decode_fp8.argtypes = [vp, vp, vp, vp, vp, vp, f32, vp, i32, vp, vp, sz, vp]
        L.mla_decode_fp8.restype = i32
        L.mla_decode_fp8_q8.argtypes = [vp, vp, vp, vp, vp, f32, vp, i32, vp, vp, sz, vp]
        L.mla_decode_fp8_q8.restype = i32
        L.mla_decode_packed.argtypes = [vp, vp, vp, vp, vp, f32, f32, vp, i32, vp, vp, sz, vp]
        L.mla_decode_packed.restype = i32
        L.mla_prefill_packed.argtypes = [vp, vp, vp, vp, vp, vp, f32, f32, vp, i32, vp, vp, sz, vp]
        L.mla_prefill_packed.restype = i32
        L.mla_block_table_to_indices.argtypes = [vp, vp, i32, vp, vp, vp]
        L.mla_block_table_to_indices.restype = i32
        L.mla_sparse_plan_create.argtypes = [ctypes.POINTER(vp), i32, i32, i32, i32, i32, i32, i32]
        L.mla_sparse_plan_create.restype = i32
        L.mla_sparse_decode_fp8.argtypes = [vp, vp, vp, vp, vp, vp, f32, vp, i32, vp, vp, vp, sz, vp]
        L.mla_sparse_decode_fp8.restype = i32
        L.mla_sparse_prefill.argtypes = [vp, vp, vp, vp, vp, vp, f32, vp, i32, vp, vp, vp, sz, vp]
        L.mla_decode_model1.argtypes = [vp, vp, vp, vp, vp, f32, vp, i32, vp, vp, sz, vp]
        L.mla_decode_model1.restype = i32
        L.mla_sparse_decode_model1.argtypes = [vp, vp, vp, vp, vp, vp, f32, vp, i32, vp, vp, vp, sz, vp]
        L.mla_sparse_decode_model1.restype = i32
        L.mla_sparse_prefill.restype = i32
        L.mla_model1_expand_records.argtypes = [vp, ctypes.c_int64, vp, vp]
        L.mla_model1_expand_records.restype = i32
        L.mla_model1_expand_q.argtypes = [vp, ctypes.c_int64, vp, vp]
        L.mla_model1_expand_q.restype = i32
        L.mla_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, f32, vp, i32, vp, vp]
        L.mla_decode_noalloc.restype = i32
        L.mla_record_attention_events.argtypes = [vp, vp]
        L.mla_record_attention_events.restype = i32
        L.mla_status_str.argtypes = [i32]
        L.mla_status_str.restype = ctypes.c_char_p
        _lib = L
        return L


def _check(status: int, what: str):
    if status != MLA_OK:
        msg = load_library().mla_status_str(status).decode()
        raise MLAError(status, f"{what} failed ({msg})")


def _host_i32(x, n: Optional[int] = None):
    if x is None:
        return None, None
    t = torch.as_tensor(x).detach().to("cpu", torch.int32).contiguous()
    if n is not None and t.numel() != n:
        raise ValueError(f"expected {n} int32 values, got {t.numel()}")
    return t, t.data_ptr()


class Plan:
    """A host plan (split-KV schedule) plus its device workspace."""

    s_q = 1  # query tokens per request (prefill plans: set at creation)

    def __init__(self, handle, desc: _Desc, kv_len, kv_indptr, qo_indptr):
        self._h = handle
        self.desc = desc
        self.kv_len = kv_len
        self.kv_indptr = kv_indptr
        self.qo_indptr = qo_indptr
        self._ws = {}

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.mla_plan_destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    @property
    def kind(self) -> int:
        return self.desc.kind

    @property
    def num_heads(self) -> int:
        return self.desc.num_qo_heads

    @property
    def workspace_bytes(self) -> int:
        return int(load_library().mla_plan_workspace_bytes(self._h))

    @property
    def num_work_items(self) -> int:
        return int(load_library().mla_plan_num_work_items(self._h))

    @property
    def num_split_groups(self) -> int:
        return int(load_library().mla_plan_num_split_groups(self._h))

    def work_items(self) -> torch.Tensor:
        n = self.num_work_items
        buf = torch.zeros((max(n, 1), 8), dtype=torch.int32)
        _check(load_library().mla_plan_get_work_items(
            self._h, ctypes.cast(buf.data_ptr(), ctypes.POINTER(ctypes.c_int32)), n), "mla_plan_get_work_items")
        return buf[:n]

    @property
    def group_size(self) -> int:
        return int(load_library().mla_plan_group_size(self._h))

    def workgroup_ptr(self) -> torch.Tensor:
        n = int(load_library().mla_plan_num_workgroups(self._h))
        buf = torch.zeros(n + 1, dtype=torch.int32)
        _check(load_library().mla_plan_get_workgroup_ptr(
            self._h, ctypes.cast(buf.data_ptr(), ctypes.POINTER(ctypes.c_int32)), n + 1),
            "mla_plan_get_workgroup_ptr")
        return buf

    def workspace(self, device: torch.device) -> torch.Tensor:
        """The device workspace of this plan, allocated and uploaded once per device."""
        device = torch.device(device)
        key = (device.type, device.index if device.index is not None else torch.cuda.current_device())
        ws = self._ws.get(key)
        if ws is None:
            nbytes = max(self.workspace_bytes, 256)
            ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
            off = (-ws.data_ptr()) % 256
            ws = ws[off:off + nbytes]
            stream = torch.cuda.current_stream(device)
            _check(load_library().mla_plan_upload(self._h, ws.data_ptr(), nbytes, stream.cuda_stream),
                   "mla_plan_upload")
            self._ws[key] = ws
        return ws


def mla_plan_create(kind: int, batch: int, num_heads: int, page_size: int, num_pages: int, kv_len,
                    kv_indptr, qo_indptr=None, kv_format: int = MLA_KV_BF16, causal: bool = True,
                    num_cus: int = 0, max_splits: int = 0, force_splits: int = 0,
                    tile_mode: int = MLA_TILE_AUTO, validate: bool = False, lse_layout: int = MLA_LSE_ROWS,
                    max_kv_len: int = 0, max_seq_len_q: int = 0) -> Plan:
    """Host plan for one set of request lengths, or (max_kv_len > 0) a
    capacity plan for any live lengths within the bounds (see include/mla.h)."""
    L = load_library()
    d = _Desc(kind=kind, batch=batch, num_qo_heads=num_heads, head_dim_ckv=_DIM_CKV,
              head_dim_kpe=_DIM_KPE, page_size=page_size, num_pages=num_pages, kv_format=kv_format,
              causal=int(bool(causal)), num_cus=num_cus, max_splits=max_splits,
              force_splits=force_splits, tile_mode=tile_mode, validate=int(validate),
              lse_layout=lse_layout, max_kv_len=max_kv_len, max_seq_len_q=max_seq_len_q)
    kl, kl_p = _host_i32(kv_len, batch) if kv_len is not None else (None, None)
    ki, ki_p = _host_i32(kv_indptr, batch + 1) if kv_indptr is not None else (None, None)
    qo, qo_p = _host_i32(qo_indptr, batch + 1) if qo_indptr is not None else (None, None)
    h = ctypes.c_void_p()
    P = ctypes.POINTER(ctypes.c_int32)
    cast = lambda p: ctypes.cast(p, P) if p is not None else None
    _check(L.mla_plan_create(ctypes.byref(h), ctypes.byref(d), cast(kl_p), cast(ki_p), cast(qo_p)),
           "mla_plan_create")
    plan = Plan(h, d, kl, ki, qo)
    # query tokens per request: the lse layout [batch, H, s_q] is sized by it
    if kind == MLA_KIND_PREFILL:
        if max_kv_len > 0 and max_seq_len_q > 0:
            plan.s_q = max_seq_len_q
        else:
            deltas = (qo[1:] - qo[:-1]) if qo is not None and batch > 0 else torch.ones(1, dtype=torch.int32)
            plan.s_q = int(deltas.max()) if deltas.numel() else 1
    return plan


def mla_sparse_plan_create(num_tokens: int, num_heads: int, num_slots: int, topk: int,
                           kv_format: int = MLA_KV_FP8_E4M3_T128, num_cus: int = 0, force_splits: int = 0) -> Plan:
    """Host plan of the token-sparse attention: num_tokens query tokens, each
    with a list of topk entries into num_slots key rows (fp8 records for
    mla_sparse_decode_fp8, bf16 rows for mla_sparse_prefill; see include/mla.h)."""
    L = load_library()
    h = ctypes.c_void_p()
    _check(L.mla_sparse_plan_create(ctypes.byref(h), num_tokens, num_heads, num_slots, topk, kv_format, num_cus,
                                    force_splits), "mla_sparse_plan_create")
    d = _Desc(kind=MLA_KIND_SPARSE_DECODE, batch=num_tokens, num_qo_heads=num_heads, head_dim_ckv=_DIM_CKV,
              head_dim_kpe=_DIM_KPE, page_size=1, num_pages=num_slots, kv_format=kv_format, causal=0,
              num_cus=num_cus, max_splits=0, force_splits=force_splits, tile_mode=MLA_TILE_WIDE)
    plan = Plan(h, d, None, None, None)
    plan.topk = topk
    return plan


def mla_sparse_decode_fp8(plan: Plan, q, kv_cache, indices, sm_scale: float, topk_length=None, attn_sink=None,
                          out=None, lse=None, max_logits=None, out_dtype=torch.bfloat16, workspace=None):
    """Token-sparse decode over 656-byte fp8 records: q [T, H, 576] bf16,
    kv_cache [..., 656] uint8 (num_slots records), indices [T, topk] int32 flat
    slots (-1 / out of range: skipped), optional topk_length [T] int32 and
    attn_sink [H] fp32.  Returns (out [T, H, 512], lse [T, H], max_logits [T, H])."""
    L = load_library()
    if plan.desc.kv_format != MLA_KV_FP8_E4M3_T128:
        raise ValueError("mla_sparse_decode_fp8 needs a plan made with kv_format=MLA_KV_FP8_E4M3_T128")
    if not isinstance(kv_cache, torch.Tensor) or kv_cache.shape[-1] != _FP8_RECORD or \
            kv_cache.numel() // _FP8_RECORD != plan.desc.num_pages:
        raise ValueError(f"kv_cache must hold {plan.desc.num_pages} records of {_FP8_RECORD} bytes")
    kv = _dev(kv_cache, "kv_cache", torch.uint8)
    qq, ix, tl, sk, out, lse, code, max_logits, mx = _sparse_extras(plan, q, indices, topk_length, attn_sink, out,
                                                                     lse, max_logits, out_dtype)
    ws = plan.workspace(q.device) if workspace is None else workspace
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(L.mla_sparse_decode_fp8(plan.handle, qq, kv, ix, tl, sk, float(sm_scale), out.data_ptr(), code,
                                   lse.data_ptr(), mx, ws.data_ptr(), ws.numel(), stream), "mla_sparse_decode_fp8")
    return out, lse, max_logits


def _sparse_extras(plan, q, indices, topk_length, attn_sink, out, lse, max_logits, out_dtype, q_dims=_DIM_CKV + _DIM_KPE):
    T, H, topk = plan.desc.batch, plan.desc.num_qo_heads, plan.topk
    qq = _dev(q, "q", torch.bfloat16, (T, H, q_dims))
    ix = _dev(indices, "indices", torch.int32, (T, topk))
    tl = _dev(topk_length, "topk_length", torch.int32, (T,)) if topk_length is not None else None
    sk = _dev(attn_sink, "attn_sink", torch.float32, (H,)) if attn_sink is not None else None
    out, lse, code = _packed_outputs(q, out, lse, out_dtype, plan)
    if max_logits is None:
        max_logits = torch.empty((T, H), dtype=torch.float32, device=q.device)
    mx = _dev(max_logits, "max_logits", torch.float32, (T, H))
    return qq, ix, tl, sk, out, lse, code, max_logits, mx


def mla_sparse_prefill(plan: Plan, q, kv, indices, sm_scale: float, topk_length=None, attn_sink=None, out=None,
                       lse=None, max_logits=None, out_dtype=torch.bfloat16, workspace=None):
    """Token-sparse attention over bf16 KV rows (FlashMLA's sparse prefill):
    q [s_q, H, 576] bf16, kv [s_kv, 576] (or [s_kv, 1, 576]) bf16, indices
    [s_q, topk] int32 (-1 / out of range: skipped), optional topk_length [s_q]
    and attn_sink [H].  Returns (out [s_q, H, 512], lse [s_q, H], max_logits [s_q, H])."""
    L = load_library()
    if plan.desc.kv_format != MLA_KV_BF16:
        raise ValueError("mla_sparse_prefill needs a plan made with kv_format=MLA_KV_BF16")
    width = _DIM_CKV + _DIM_KPE
    if not isinstance(kv, torch.Tensor) or kv.shape[-1] != width or kv.numel() // width != plan.desc.num_pages:
        raise ValueError(f"kv must hold {plan.desc.num_pages} rows of {width} bf16 values")
    k = _dev(kv, "kv", torch.bfloat16)
    qq, ix, tl, sk, out, lse, code, max_logits, mx = _sparse_extras(plan, q, indices, topk_length, attn_sink, out,
                                                                     lse, max_logits, out_dtype)
    ws = plan.workspace(q.device) if workspace is None else workspace
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(L.mla_sparse_prefill(plan.handle, qq, k, ix, tl, sk, float(sm_scale), out.data_ptr(), code,
                                lse.data_ptr(), mx, ws.data_ptr(), ws.numel(), stream), "mla_sparse_prefill")
    return out, lse, max_logits


def mla_record_attention_events(before, after):
    """Record two caller-owned hipEvent_t handles around the attention kernel
    of the next run call on this thread (timing diagnostics)."""
    _check(load_library().mla_record_attention_events(before, after), "mla_record_attention_events")


def _dev(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _lse_shape(plan, rows: int, H: int):
    if plan is not None and plan.desc.lse_layout == MLA_LSE_HEADS_FIRST:
        return (plan.desc.batch, H, plan.s_q)
    return (rows, H)


def _outputs(q_nope: torch.Tensor, out, lse, out_dtype, plan=None):
    rows, H = q_nope.shape[0], q_nope.shape[1]
    if out is None:
        out = torch.empty((rows, H, _DIM_CKV), dtype=out_dtype, device=q_nope.device)
    if lse is None:
        lse = torch.empty(_lse_shape(plan, rows, H), dtype=torch.float32, device=q_nope.device)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out must be bf16 or fp32")
    _dev(out, "out", out.dtype, (rows, H, _DIM_CKV))
    _dev(lse, "lse", torch.float32, _lse_shape(plan, rows, H))
    code = MLA_DTYPE_BF16 if out.dtype == torch.bfloat16 else MLA_DTYPE_FP32
    return out, lse, code


def _q(plan: Plan, q_nope, q_pe, rows: int):
    H = plan.num_heads
    return (_dev(q_nope, "q_nope", torch.bfloat16, (rows, H, _DIM_CKV)),
            _dev(q_pe, "q_pe", torch.bfloat16, (rows, H, _DIM_KPE)))


def _nonempty(t: torch.Tensor) -> torch.Tensor:
    """An empty index tensor has no storage (a null pointer, which the C ABI
    refuses): hand over one padding entry instead; it is never read."""
    return t if t.numel() > 0 else torch.zeros(1, dtype=t.dtype, device=t.device)


def _paging(plan: Plan, kv_indptr, kv_indices):
    kv_indices = _nonempty(kv_indices)
    a = _dev(kv_indptr, "kv_indptr", torch.int32, (plan.desc.batch + 1,))
    b = _dev(kv_indices, "kv_indices", torch.int32)
    if plan.desc.batch > 0 and plan.kv_indptr is not None and kv_indices.numel() < int(plan.kv_indptr[-1]):
        raise ValueError("kv_indices is shorter than kv_indptr[-1]")
    return a, b


def mla_decode(plan: Plan, q_nope, q_pe, ckv_cache, kpe_cache, kv_indptr, kv_indices, sm_scale: float,
               out=None, lse=None, out_dtype=torch.bfloat16, workspace=None):
    """Paged MLA decode; returns (out [B, H, 512], lse [B, H] fp32, natural log)."""
    L = load_library()
    B, P, ps = plan.desc.batch, plan.desc.num_pages, plan.desc.page_size
    qn, qp = _q(plan, q_nope, q_pe, B)
    c = _dev(ckv_cache, "ckv_cache", torch.bfloat16, (P, ps, _DIM_CKV))
    k = _dev(kpe_cache, "kpe_cache", torch.bfloat16, (P, ps, _DIM_KPE))
    ip, ix = _paging(plan, kv_indptr, kv_indices)
    out, lse, code = _outputs(q_nope, out, lse, out_dtype, plan)
    ws = plan.workspace(q_nope.device) if workspace is None else workspace
    stream = torch.cuda.current_stream(q_nope.device).cuda_stream
    _check(L.mla_decode(plan.handle, qn, qp, c, k, ip, ix, float(sm_scale), out.data_ptr(), code,
                        lse.data_ptr(), ws.data_ptr(), ws.numel(), stream), "mla_decode")
    return out, lse


NOALLOC_SCRATCH_BYTES = 64 << 20


def mla_decode_noalloc(plan: Plan, q_nope, q_pe, ckv_cache, kpe_cache, kv_indptr, kv_indices, sm_scale: float,
                       out=None, lse=None, out_dtype=torch.bfloat16):
    """mla_decode with the library's fixed device scratch array as its
    workspace (no device allocation by the library; see include/mla.h).
    Calls on one GPU share the array and must not overlap in time."""
    L = load_library()
    B, P, ps = plan.desc.batch, plan.desc.num_pages, plan.desc.page_size
    qn, qp = _q(plan, q_nope, q_pe, B)
    c = _dev(ckv_cache, "ckv_cache", torch.bfloat16, (P, ps, _DIM_CKV))
    k = _dev(kpe_cache, "kpe_cache", torch.bfloat16, (P, ps, _DIM_KPE))
    ip, ix = _paging(plan, kv_indptr, kv_indices)
    out, lse, code = _outputs(q_nope, out, lse, out_dtype, plan)
    stream = torch.cuda.current_stream(q_nope.device).cuda_stream
    _check(L.mla_decode_noalloc(plan.handle, qn, qp, c, k, ip, ix, float(sm_scale), out.data_ptr(), code,
                                lse.data_ptr(), stream), "mla_decode_noalloc")
    return out, lse


def mla_prefill(plan: Plan, q_nope, q_pe, ckv_cache, kpe_cache, qo_indptr, kv_indptr, kv_indices,
                sm_scale: float, out=None, lse=None, out_dtype=torch.bfloat16, workspace=None):
    """Paged MLA prefill over packed queries; returns (out [total_q, H, 512], lse [total_q, H])."""
    L = load_library()
    B, P, ps = plan.desc.batch, plan.desc.num_pages, plan.desc.page_size
    total_q = int(plan.qo_indptr[-1]) if plan.qo_indptr is not None else 0
    qn, qp = _q(plan, q_nope, q_pe, total_q)
    c = _dev(ckv_cache, "ckv_cache", torch.bfloat16, (P, ps, _DIM_CKV))
    k = _dev(kpe_cache, "kpe_cache", torch.bfloat16, (P, ps, _DIM_KPE))
    qo = _dev(qo_indptr, "qo_indptr", torch.int32, (B + 1,))
    ip, ix = _paging(plan, kv_indptr, kv_indices)
    out, lse, code = _outputs(q_nope, out, lse, out_dtype, plan)
    ws = plan.workspace(q_nope.device) if workspace is None else workspace
    stream = torch.cuda.current_stream(q_nope.device).cuda_stream
    _check(L.mla_prefill(plan.handle, qn, qp, c, k, qo, ip, ix, float(sm_scale), out.data_ptr(), code,
                         lse.data_ptr(), ws.data_ptr(), ws.numel(), stream), "mla_prefill")
    return out, lse


def mla_decode_live(plan: Plan, q_nope, q_pe, ckv_cache, kpe_cache, kv_len, kv_indptr, kv_indices, sm_scale: float,
                    out=None, lse=None, out_dtype=torch.bfloat16, workspace=None):
    """Decode with a capacity plan: kv_len [B] int32 on the device holds this
    call's live key counts (each <= the plan's max_kv_len)."""
    L = load_library()
    B, P, ps = plan.desc.batch, plan.desc.num_pages, plan.desc.page_size
    qn, qp = _q(plan, q_nope, q_pe, B)
    c = _dev(ckv_cache, "ckv_cache", torch.bfloat16, (P, ps, _DIM_CKV))
    k = _dev(kpe_cache, "kpe_cache", torch.bfloat16, (P, ps, _DIM_KPE))
    kl = _dev(kv_len, "kv_len", torch.int32, (B,))
    ip = _dev(kv_indptr, "kv_indptr", torch.int32, (B + 1,))
    kv_indices = _nonempty(kv_indices)
    ix = _dev(kv_indices, "kv_indices", torch.int32)
    out, lse, code = _outputs(q_nope, out, lse, out_dtype, plan)
    ws = plan.workspace(q_nope.device) if workspace is None else workspace
    stream = torch.cuda.current_stream(q_nope.device).cuda_stream
    _check(L.mla_decode_live(plan.handle, qn, qp, c, k, kl, ip, ix, float(sm_scale), out.data_ptr(), code,
                             lse.data_ptr(), ws.data_ptr(), ws.numel(), stream), "mla_decode_live")
    return out, lse


def mla_prefill_live(plan: Plan, q_nope, q_pe, ckv_cache, kpe_cache, qo_indptr, kv_len, kv_indptr, kv_indices,
                     sm_scale: float, out=None, lse=None, out_dtype=torch.bfloat16, workspace=None):
    """Prefill with a capacity plan: qo_indptr [B+1], kv_len [B] and kv_indptr
    [B+1] on the device hold this call's live query offsets, key counts and
    page offsets.  q_nope / q_pe hold qo_indptr[B] query tokens (rows)."""
    L = load_library()
    B, P, ps = plan.desc.batch, plan.desc.num_pages, plan.desc.page_size
    rows = q_nope.shape[0]
    qn, qp = _q(plan, q_nope, q_pe, rows)
    c = _dev(ckv_cache, "ckv_cache", torch.bfloat16, (P, ps, _DIM_CKV))
    k = _dev(kpe_cache, "kpe_cache", torch.bfloat16, (P, ps, _DIM_KPE))
    qo = _dev(qo_indptr, "qo_indptr", torch.int32, (B + 1,))
    kl = _dev(kv_len, "kv_len", torch.int32, (B,))
    ip = _dev(kv_indptr, "kv_indptr", torch.int32, (B + 1,))
    kv_indices = _nonempty(kv_indices)
    ix = _dev(kv_indices, "kv_indices", torch.int32)
    out, lse, code = _outputs(q_nope, out, lse, out_dtype, plan)
    ws = plan.workspace(q_nope.device) if workspace is None else workspace
    stream = torch.cuda.current_stream(q_nope.device).cuda_stream
    _check(L.mla_prefill_live(plan.handle, qn, qp, c, k, qo, kl, ip, ix, float(sm_scale), out.data_ptr(), code,
                              lse.data_ptr(), ws.data_ptr(), ws.numel(), stream), "mla_prefill_live")
    return out, lse


def mla_decode_fp8(plan: Plan, q_nope, q_pe, kv_cache, kv_indptr, kv_indices, sm_scale: float,
                   out=None, lse=None, out_dtype=torch.bfloat16, workspace=None):
    """Paged MLA decode over 656-byte fp8 token records."""
    L = load_library()
    B, P, ps = plan.desc.batch, plan.desc.num_pages, plan.desc.page_size
    qn, qp = _q(plan, q_nope, q_pe, B)
    kv = _dev(kv_cache, "kv_cache", torch.uint8, (P, ps, _FP8_RECORD))
    ip, ix = _paging(plan, kv_indptr, kv_indices)
    out, lse, code = _outputs(q_nope, out, lse, out_dtype, plan)
    ws = plan.workspace(q_nope.device) if workspace is None else workspace
    stream = torch.cuda.current_stream(q_nope.device).cuda_stream
    _check(L.mla_decode_fp8(plan.handle, qn, qp, kv, ip, ix, float(sm_scale), out.data_ptr(), code,
                            lse.data_ptr(), ws.data_ptr(), ws.numel(), stream), "mla_decode_fp8")
    return out, lse


def _packed_q(plan: Plan, q, rows: int):
    return _dev(q, "q", torch.bfloat16, (rows, plan.num_heads, _DIM_CKV + _DIM_KPE))


def _packed_outputs(q: torch.Tensor, out, lse, out_dtype, plan=None):
    rows, H = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty((rows, H, _DIM_CKV), dtype=out_dtype, device=q.device)
    return _outputs(out, out, lse, out.dtype, plan)


def mla_decode_fp8_q8(plan: Plan, q, kv_cache, kv_indptr, kv_indices, sm_scale: float, out=None, lse=None,
                      out_dtype=torch.bfloat16, workspace=None):
    """Decode over 656-byte fp8 records with an e4m3 query: q [B, H, 576]
    uint8 codes (latent then rope dims).  Returns (out [B, H, 512], lse [B, H])."""
    L = load_library()
    B, P, ps = plan.desc.batch, plan.desc.num_pages, plan.desc.page_size
    qq = _dev(q, "q", torch.uint8, (B, plan.num_heads, _DIM_CKV + _DIM_KPE))
    kv = _dev(kv_cache, "kv_cache", torch.uint8, (P, ps, _FP8_RECORD))
    ip, ix = _paging(plan, kv_indptr, kv_indices)
    out, lse, code = _packed_outputs(q, out, lse, out_dtype, plan)
    ws = plan.workspace(q.device) if workspace is None else workspace
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(L.mla_decode_fp8_q8(plan.handle, qq, kv, ip, ix, float(sm_scale), out.data_ptr(), code, lse.data_ptr(),
                               ws.data_ptr(), ws.numel(), stream), "mla_decode_fp8_q8")
    return out, lse


def mla_decode_packed(plan: Plan, q, kv_cache, kv_indptr, kv_indices, sm_scale: float, out_scale: float = 1.0,
                      out=None, lse=None, out_dtype=torch.bfloat16, workspace=None):
    """Paged MLA decode over the concatenated layout: q [B, H, 576], kv_cache
    [num_pages, page_size, 576] (latent dims, then rope dims); out is scaled
    by out_scale.  Returns (out [B, H, 512], lse [B, H])."""
    L = load_library()
    B, P, ps = plan.desc.batch, plan.desc.num_pages, plan.desc.page_size
    qq = _packed_q(plan, q, B)
    kv = _dev(kv_cache, "kv_cache", torch.bfloat16, (P, ps, _DIM_CKV + _DIM_KPE))
    ip, ix = _paging(plan, kv_indptr, kv_indices)
    out, lse, code = _packed_outputs(q, out, lse, out_dtype, plan)
    ws = plan.workspace(q.device) if workspace is None else workspace
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(L.mla_decode_packed(plan.handle, qq, kv, ip, ix, float(sm_scale), float(out_scale), out.data_ptr(), code,
                               lse.data_ptr(), ws.data_ptr(), ws.numel(), stream), "mla_decode_packed")
    return out, lse


def mla_prefill_packed(plan: Plan, q, kv_cache, qo_indptr, kv_indptr, kv_indices, sm_scale: float,
                       out_scale: float = 1.0, out=None, lse=None, out_dtype=torch.bfloat16, workspace=None):
    """Paged MLA prefill over packed queries in the concatenated layout:
    q [total_q, H, 576], kv_cache [num_pages, page_size, 576]."""
    L = load_library()
    B, P, ps = plan.desc.batch, plan.desc.num_pages, plan.desc.page_size
    total_q = int(plan.qo_indptr[-1]) if plan.qo_indptr is not None else 0
    qq = _packed_q(plan, q, total_q)
    kv = _dev(kv_cache, "kv_cache", torch.bfloat16, (P, ps, _DIM_CKV + _DIM_KPE))
    qo = _dev(qo_indptr, "qo_indptr", torch.int32, (B + 1,))
    ip, ix = _paging(plan, kv_indptr, kv_indices)
    out, lse, code = _packed_outputs(q, out, lse, out_dtype, plan)
    ws = plan.workspace(q.device) if workspace is None else workspace
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(L.mla_prefill_packed(plan.handle, qq, kv, qo, ip, ix, float(sm_scale), float(out_scale), out.data_ptr(),
                                code, lse.data_ptr(), ws.data_ptr(), ws.numel(), stream), "mla_prefill_packed")
    return out, lse


def mla_block_table_to_indices(plan: Plan, block_table, kv_indptr, kv_indices=None):
    """kv_indices (int32 device) from a dense block table [batch, max_blocks]:
    the first kv_indptr[b+1] - kv_indptr[b] entries of each row, in order."""
    L = load_library()
    B = plan.desc.batch
    bt = _dev(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [batch={B}, max_blocks]")
    ip = _dev(kv_indptr, "kv_indptr", torch.int32, (B + 1,))
    n = int(plan.kv_indptr[-1]) if B > 0 else 0
    if kv_indices is None:
        kv_indices = torch.empty((max(n, 1),), dtype=torch.int32, device=block_table.device)
    ix = _dev(kv_indices, "kv_indices", torch.int32)
    if kv_indices.numel() < n:
        raise ValueError("kv_indices is shorter than kv_indptr[-1]")
    stream = torch.cuda.current_stream(block_table.device).cuda_stream
    _check(L.mla_block_table_to_indices(plan.handle, bt, int(block_table.shape[1]), ip, ix, stream),
           "mla_block_table_to_indices")
    return kv_indices


MODEL1_RECORD = 604
MODEL1_NOPE = 448


def mla_model1_expand_records(records, rows=None):
    """MODEL1 records [..., 604] (uint8, device) -> bf16 rows [..., 576] in the
    concatenated layout (dims 448..511 zero); see mla_model1_expand_records in mla.h."""
    L = load_library()
    if records.dtype != torch.uint8 or records.shape[-1] != MODEL1_RECORD or not records.is_contiguous():
        raise ValueError("records must be contiguous uint8 [..., 604]")
    n = records.numel() // MODEL1_RECORD
    if rows is None:
        rows = torch.empty(tuple(records.shape[:-1]) + (_DIM_CKV + _DIM_KPE,), dtype=torch.bfloat16,
                           device=records.device)
    if rows.dtype != torch.bfloat16 or rows.numel() != n * (_DIM_CKV + _DIM_KPE) or not rows.is_contiguous():
        raise ValueError("rows must be contiguous bf16 with 576 values per record")
    stream = torch.cuda.current_stream(records.device).cuda_stream
    _check(L.mla_model1_expand_records(records.data_ptr(), n, rows.data_ptr(), stream), "mla_model1_expand_records")
    return rows


def mla_model1_expand_q(q, q576=None):
    """Query rows [..., 512] (bf16: 448 NoPE + 64 RoPE) -> [..., 576] with zeros in dims 448..511."""
    L = load_library()
    if q.dtype != torch.bfloat16 or q.shape[-1] != MODEL1_NOPE + _DIM_KPE or not q.is_contiguous():
        raise ValueError("q must be contiguous bf16 [..., 512]")
    n = q.numel() // (MODEL1_NOPE + _DIM_KPE)
    if q576 is None:
        q576 = torch.empty(tuple(q.shape[:-1]) + (_DIM_CKV + _DIM_KPE,), dtype=torch.bfloat16, device=q.device)
    if q576.dtype != torch.bfloat16 or q576.numel() != n * (_DIM_CKV + _DIM_KPE) or not q576.is_contiguous():
        raise ValueError("q576 must be contiguous bf16 with 576 values per row")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(L.mla_model1_expand_q(q.data_ptr(), n, q576.data_ptr(), stream), "mla_model1_expand_q")
    return q576


def mla_decode_model1(plan: Plan, q, kv_cache, kv_indptr, kv_indices, sm_scale: float, out=None, lse=None,
                      out_dtype=torch.bfloat16, workspace=None):
    """Paged decode over MODEL1 records, dequantised in the kernel: q [B, H, 512]
    bf16 (448 NoPE + 64 RoPE), kv_cache [num_pages, page_size, 604] uint8.
    Returns (out [B, H, 512] with dims 448..511 zero, lse [B, H])."""
    L = load_library()
    if plan.desc.kv_format != MLA_KV_FP8_MODEL1:
        raise ValueError("mla_decode_model1 needs a plan made with kv_format=MLA_KV_FP8_MODEL1")
    B, P, ps = plan.desc.batch, plan.desc.num_pages, plan.desc.page_size
    qq = _dev(q, "q", torch.bfloat16, (B, plan.num_heads, MODEL1_NOPE + _DIM_KPE))
    kv = _dev(kv_cache, "kv_cache", torch.uint8, (P, ps, MODEL1_RECORD))
    ip, ix = _paging(plan, kv_indptr, kv_indices)
    if out is None:
        out = torch.empty((B, plan.num_heads, _DIM_CKV), dtype=out_dtype, device=q.device)
    out, lse, code = _outputs(out, out, lse, out.dtype, plan)
    ws = plan.workspace(q.device) if workspace is None else workspace
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(L.mla_decode_model1(plan.handle, qq, kv, ip, ix, float(sm_scale), out.data_ptr(), code, lse.data_ptr(),
                               ws.data_ptr(), ws.numel(), stream), "mla_decode_model1")
    return out, lse


def mla_sparse_decode_model1(plan: Plan, q, kv_cache, indices, sm_scale: float, topk_length=None, attn_sink=None,
                             out=None, lse=None, max_logits=None, out_dtype=torch.bfloat16, workspace=None):
    """Token-sparse decode over MODEL1 records: q [T, H, 512] bf16, kv_cache
    [..., 604] uint8 (num_slots records), indices [T, topk] int32 flat slots.
    Returns (out [T, H, 512] with dims 448..511 zero, lse [T, H], max_logits [T, H])."""
    L = load_library()
    if plan.desc.kv_format != MLA_KV_FP8_MODEL1:
        raise ValueError("mla_sparse_decode_model1 needs a plan made with kv_format=MLA_KV_FP8_MODEL1")
    if not isinstance(kv_cache, torch.Tensor) or kv_cache.shape[-1] != MODEL1_RECORD or \
            kv_cache.numel() // MODEL1_RECORD != plan.desc.num_pages:
        raise ValueError(f"kv_cache must hold {plan.desc.num_pages} records of {MODEL1_RECORD} bytes")
    kv = _dev(kv_cache, "kv_cache", torch.uint8)
    if out is None:
        out = torch.empty((plan.desc.batch, plan.num_heads, _DIM_CKV), dtype=out_dtype, device=q.device)
    qq, ix, tl, sk, out, lse, code, max_logits, mx = _sparse_extras(plan, q, indices, topk_length, attn_sink, out,
                                                                     lse, max_logits, out_dtype,
                                                                     q_dims=MODEL1_NOPE + _DIM_KPE)
    ws = plan.workspace(q.device) if workspace is None else workspace
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(L.mla_sparse_decode_model1(plan.handle, qq, kv, ix, tl, sk, float(sm_scale), out.data_ptr(), code,
                                      lse.data_ptr(), mx, ws.data_ptr(), ws.numel(), stream),
           "mla_sparse_decode_model1")
    return out, lse, max_logits
