"""Host-side tests of libmla.so: it loads, exports every declared symbol, the
planner's schedule is a correct and balanced cover, and argument errors are
reported as statuses.  No kernel is launched."""

import ctypes
import os
import re

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def mla():
    import paged_mla_decode_05_amd as m

    if not os.path.exists(m.lib_path()):
        import __graft_entry__

        __graft_entry__.build()
    m.load_library()
    return m


def test_library_exports_every_declared_function(mla):
    header = open(os.path.join(ROOT, "include", "mla.h")).read()
    names = set(re.findall(r"^\s*(?:mla_status|void|size_t|int32_t|const char\*)\s+(mla_\w+)\s*\(", header, re.M))
    assert {"mla_plan_create", "mla_decode", "mla_prefill", "mla_decode_fp8", "mla_decode_packed",
            "mla_prefill_packed", "mla_block_table_to_indices"} <= names
    lib = mla.load_library()
    for n in sorted(names):
        assert hasattr(lib, n), n


def _items(plan):
    it = plan.work_items().numpy()
    return [dict(b=r[0], row0=r[1], nrows=r[2], t0=r[3], t1=r[4], L=r[5], n=r[6], slot=r[7]) for r in it]


def _visible(L, n, H, row0, nrows, causal):
    if not causal:
        return L
    last_q = (row0 + nrows - 1) // H
    return L - n + last_q + 1


def _check_cover(plan, kv_len, q_len, H, causal=False, prefill=False):
    items = _items(plan)
    # every (request, row) lies in exactly one row block, and each block's
    # visible keys are covered exactly once by its items
    blocks = {}
    for it in items:
        assert it["t0"] % 64 == 0
        assert 0 <= it["t0"] <= it["t1"]
        blocks.setdefault((it["b"], it["row0"], it["nrows"]), []).append((it["t0"], it["t1"], it["slot"]))
    for b, (L, n) in enumerate(zip(kv_len, q_len)):
        rows = n * H
        covered = np.zeros(rows, dtype=int)
        for (bb, r0, nr), pieces in blocks.items():
            if bb != b:
                continue
            covered[r0:r0 + nr] += 1
            vis = _visible(L, n, H, r0, nr, causal and prefill)
            pieces.sort()
            assert pieces[0][0] == 0 and pieces[-1][1] == vis
            for (a0, a1, _), (c0, c1, _) in zip(pieces[:-1], pieces[1:]):
                assert a1 == c0  # contiguous, no overlap
            slots = [s for _, _, s in pieces]
            if len(pieces) == 1:
                assert slots == [-1]
            else:
                assert slots == list(range(slots[0], slots[0] + len(slots)))
        assert np.all(covered == 1), f"request {b} rows covered {covered}"
    # workgroup ranges partition the item list
    ptr = plan.workgroup_ptr().numpy()
    assert ptr[0] == 0 and ptr[-1] == len(items) and np.all(np.diff(ptr) >= 1)
    return items, ptr


@pytest.mark.parametrize("tile_mode", [0, 1, 2, 3])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_schedule_covers_every_key_once(mla, tile_mode, seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    lens = rng.integers(0, 5000, B)
    lens[0] = 0
    ps = int(rng.choice([1, 16, 64, 128]))
    pages = -(-lens // ps)
    indptr = np.concatenate([[0], np.cumsum(pages)])
    H = int(rng.choice([16, 128, 40]))
    plan = mla.mla_plan_create(0, B, H, ps, int(max(1, indptr[-1])), lens, indptr, num_cus=int(rng.integers(1, 300)),
                               tile_mode=tile_mode)
    _check_cover(plan, lens, [1] * B, H)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_schedule_covers_visible_keys(mla, causal):
    rng = np.random.default_rng(7)
    B = 20
    qlens = rng.integers(0, 9, B)
    lens = rng.integers(8, 3000, B)
    qo = np.concatenate([[0], np.cumsum(qlens)])
    indptr = np.concatenate([[0], np.cumsum(-(-lens // 64))])
    plan = mla.mla_plan_create(1, B, 128, 64, int(indptr[-1]), lens, indptr, qo_indptr=qo, causal=causal,
                               num_cus=256)
    _check_cover(plan, lens, qlens, 128, causal=causal, prefill=True)


def test_prefill_gangs_walk_keys_together(mla):
    """The query tokens of a prefill request (one 128-row block each) get the
    same key pieces, at the same position of neighbouring lists (in sub-gangs
    of up to 8 tokens)."""
    rng = np.random.default_rng(11)
    B = 32
    qlens = rng.integers(1, 9, B)
    lens = rng.integers(1024, 4097, B)
    qo = np.concatenate([[0], np.cumsum(qlens)])
    indptr = np.concatenate([[0], np.cumsum(-(-lens // 64))])
    plan = mla.mla_plan_create(1, B, 128, 64, int(indptr[-1]), lens, indptr, qo_indptr=qo, causal=True,
                               num_cus=256)
    items, ptr = _check_cover(plan, lens, qlens, 128, causal=True, prefill=True)
    where = {}  # (b, row0) -> [(list, position, t0)]
    for w in range(len(ptr) - 1):
        for pos, it in enumerate(items[ptr[w]:ptr[w + 1]]):
            where.setdefault((it["b"], it["row0"]), []).append((w, pos, it["t0"]))
    # consecutive tokens either walk in step (same pieces, next list) or
    # start a new sub-gang; most of them walk in step
    ganged = 0
    for b in range(B):
        seqs = [sorted(where[(b, 128 * j)]) for j in range(qlens[b])]
        for j in range(1, qlens[b]):
            same = [(pos, t0) for _, pos, t0 in seqs[j]] == [(pos, t0) for _, pos, t0 in seqs[j - 1]]
            if same and [w for w, _, _ in seqs[j]] == [w + 1 for w, _, _ in seqs[j - 1]]:
                ganged += 1
    assert ganged >= 0.6 * int(np.sum(qlens - 1))


@pytest.mark.parametrize("seed", range(6))
def test_prefill_schedules_cover_random_shapes(mla, seed):
    """Random prefill shapes (every tile mode, causal or not, CU counts from 1
    to 300): whichever packing the planner keeps (greedy, one item per list,
    gangs), every visible key of every row block is covered exactly once."""
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 24))
    H = int(rng.choice([16, 40, 64, 128, 256]))
    qlens = rng.integers(0, 17, B)
    lens = qlens + rng.integers(0, 3000, B)
    qo = np.concatenate([[0], np.cumsum(qlens)])
    ps = int(rng.choice([1, 16, 64]))
    indptr = np.concatenate([[0], np.cumsum(-(-lens // ps))])
    causal = bool(rng.integers(0, 2))
    plan = mla.mla_plan_create(1, B, H, ps, int(max(1, indptr[-1])), lens, indptr, qo_indptr=qo, causal=causal,
                               num_cus=int(rng.integers(1, 301)), tile_mode=int(rng.integers(0, 4)))
    _check_cover(plan, lens, qlens, H, causal=causal, prefill=True)


@pytest.mark.timeout(60)
@pytest.mark.parametrize("num_cus", [1, 3, 7, 8, 9])
def test_prefill_gangs_wider_than_the_machine(mla, num_cus):
    """Requests with more query tokens (gang width) than there are lists: the
    gang search gives up and the greedy plan is kept (this once looped)."""
    qlens = np.array([16, 9, 1, 12])
    lens = qlens + np.array([3000, 500, 70, 1200])
    qo = np.concatenate([[0], np.cumsum(qlens)])
    indptr = np.concatenate([[0], np.cumsum(-(-lens // 64))])
    plan = mla.mla_plan_create(1, 4, 128, 64, int(indptr[-1]), lens, indptr, qo_indptr=qo, causal=True,
                               num_cus=num_cus, tile_mode=1)
    _, ptr = _check_cover(plan, lens, qlens, 128, causal=True, prefill=True)
    assert len(ptr) - 1 <= num_cus


def test_forced_splits(mla):
    lens = np.array([1, 37, 64, 200, 1000])
    indptr = np.concatenate([[0], np.cumsum(-(-lens // 64))])
    plan = mla.mla_plan_create(0, 5, 16, 64, int(indptr[-1]), lens, indptr, num_cus=8, force_splits=3)
    items, _ = _check_cover(plan, lens, [1] * 5, 16)
    per_req = {}
    for it in items:
        per_req[it["b"]] = per_req.get(it["b"], 0) + 1
    # a request is cut into min(3, ceil(L/64)) chunks
    assert per_req == {0: 1, 1: 1, 2: 1, 3: 3, 4: 3}
    assert plan.num_split_groups == 2


def test_schedule_balances_skewed_lengths(mla):
    # 120 requests of 8192 keys and 8 of 32768 (16 heads): every workgroup
    # gets close to the mean number of keys
    lens = np.full(128, 8192)
    lens[np.random.default_rng(3).permutation(128)[:8]] = 32768
    indptr = np.concatenate([[0], np.cumsum(lens // 64)])
    plan = mla.mla_plan_create(0, 128, 16, 64, int(indptr[-1]), lens, indptr, num_cus=256)
    items, ptr = _check_cover(plan, lens, [1] * 128, 16)
    cost = np.array([sum(items[i]["t1"] - items[i]["t0"] + 64 for i in range(ptr[w], ptr[w + 1]))
                     for w in range(len(ptr) - 1)])
    assert len(ptr) - 1 <= 256
    assert cost.max() <= 1.1 * cost.mean() + 192


def test_decode_128_heads_balance(mla):
    rng = np.random.default_rng(2)
    lens = rng.integers(512, 4097, 64)
    indptr = np.concatenate([[0], np.cumsum(-(-lens // 64))])
    plan = mla.mla_plan_create(0, 64, 128, 64, int(indptr[-1]), lens, indptr, num_cus=256)
    items, ptr = _check_cover(plan, lens, [1] * 64, 128)
    cost = np.array([sum(items[i]["t1"] - items[i]["t0"] + 64 for i in range(ptr[w], ptr[w + 1]))
                     for w in range(len(ptr) - 1)])
    assert cost.max() <= 1.1 * cost.mean() + 192


def _status(mla, **kw):
    try:
        mla.mla_plan_create(**kw)
    except mla.MLAError as e:
        return e.status
    return 0


def test_plan_argument_errors(mla):
    ok = dict(kind=0, batch=2, num_heads=16, page_size=64, num_pages=4, kv_len=[10, 70], kv_indptr=[0, 1, 3],
              num_cus=4)
    assert _status(mla, **ok) == 0
    assert _status(mla, **{**ok, "page_size": 48}) == -2                 # not a power of two
    assert _status(mla, **{**ok, "kv_indptr": [0, 1, 2]}) == -1          # 70 keys need 2 pages
    assert _status(mla, **{**ok, "kv_indptr": [1, 2, 4]}) == -1          # indptr[0] != 0
    assert _status(mla, **{**ok, "kv_len": [10, -1]}) == -1
    assert _status(mla, **{**ok, "num_heads": 0}) == -1
    assert _status(mla, **{**ok, "kind": 0, "qo_indptr": [0, 1, 2]}) == -1   # decode takes no qo_indptr
    pre = dict(ok, kind=1, qo_indptr=[0, 3, 4])
    assert _status(mla, **pre) == 0
    assert _status(mla, **{**pre, "qo_indptr": [0, 11, 12]}) == -1      # causal: 11 queries > 10 keys
    assert _status(mla, **{**pre, "qo_indptr": [0, 11, 12], "causal": False}) == 0
    assert _status(mla, **{**pre, "qo_indptr": [0, 3, 2]}) == -1        # decreasing
    assert _status(mla, **{**pre, "kv_format": 1}) == -2                # fp8 prefill
    assert _status(mla, **{**ok, "batch": 0, "kv_len": [], "kv_indptr": [0]}) == 0
    assert _status(mla, **{**ok, "tile_mode": 4}) == -1
    assert _status(mla, **{**ok, "kv_format": 1}) == 0                  # fp8 decode
    assert _status(mla, **{**ok, "kv_format": 1, "tile_mode": 3}) == -2  # fp8 has no quad tile


def test_header_dims_are_enforced(mla):
    lib = mla.load_library()
    from paged_mla_decode_05_amd._binding import _Desc

    d = _Desc(kind=0, batch=1, num_qo_heads=16, head_dim_ckv=256, head_dim_kpe=64, page_size=64, num_pages=1,
              kv_format=0, causal=0, num_cus=4, max_splits=0, force_splits=0, tile_mode=0)
    h = ctypes.c_void_p()
    kl = (ctypes.c_int32 * 1)(5)
    ip = (ctypes.c_int32 * 2)(0, 1)
    assert lib.mla_plan_create(ctypes.byref(h), ctypes.byref(d), kl, ip, None) == -2
    assert lib.mla_plan_create(None, ctypes.byref(d), kl, ip, None) == -1
    assert lib.mla_plan_create(ctypes.byref(h), None, kl, ip, None) == -1


def test_run_call_errors_before_any_launch(mla):
    # These calls fail validation on the host and never touch a device.
    lib = mla.load_library()
    dec = mla.mla_plan_create(0, 2, 16, 64, 4, [10, 70], [0, 1, 3], num_cus=4)
    pre = mla.mla_plan_create(1, 2, 16, 64, 4, [10, 70], [0, 1, 3], qo_indptr=[0, 1, 2], num_cus=4)
    fake = ctypes.c_void_p(0x1000)
    args = [fake] * 6
    # prefill plan passed to decode -> plan mismatch
    assert lib.mla_decode(pre.handle, *args, 0.1, fake, 0, fake, fake, 1 << 20, None) == -4
    # decode plan passed to the fp8 entry -> plan mismatch
    assert lib.mla_decode_fp8(dec.handle, *[fake] * 5, 0.1, fake, 0, fake, fake, 1 << 20, None) == -4
    # non-finite scale, bad dtype, null pointer, small workspace
    assert lib.mla_decode(dec.handle, *args, float("nan"), fake, 0, fake, fake, 1 << 20, None) == -1
    assert lib.mla_decode(dec.handle, *args, 0.1, fake, 7, fake, fake, 1 << 20, None) == -1
    assert lib.mla_decode(dec.handle, None, *args[1:], 0.1, fake, 0, fake, fake, 1 << 20, None) == -1
    assert lib.mla_decode(dec.handle, *args, 0.1, fake, 0, fake, fake, 16, None) == -3
    assert lib.mla_decode(None, *args, 0.1, fake, 0, fake, fake, 1 << 20, None) == -1
    assert lib.mla_status_str(-4).decode().startswith("plan")


def test_packed_layout_and_block_table_errors(mla):
    lib = mla.load_library()
    dec = mla.mla_plan_create(0, 2, 16, 64, 4, [10, 70], [0, 1, 3], num_cus=4)
    pre = mla.mla_plan_create(1, 2, 16, 64, 4, [10, 70], [0, 1, 3], qo_indptr=[0, 1, 2], num_cus=4)
    fake = ctypes.c_void_p(0x1000)
    tail = (fake, 0, fake, fake, 1 << 20, None)
    # wrong plan kind, non-finite output scale, missing q or cache
    assert lib.mla_decode_packed(pre.handle, fake, fake, fake, fake, 0.1, 1.0, *tail) == -4
    assert lib.mla_prefill_packed(dec.handle, fake, fake, fake, fake, fake, 0.1, 1.0, *tail) == -4
    assert lib.mla_decode_packed(dec.handle, fake, fake, fake, fake, 0.1, float("inf"), *tail) == -1
    assert lib.mla_decode_packed(dec.handle, None, fake, fake, fake, 0.1, 1.0, *tail) == -1
    assert lib.mla_decode_packed(dec.handle, fake, None, fake, fake, 0.1, 1.0, *tail) == -1
    assert lib.mla_prefill_packed(pre.handle, fake, fake, None, fake, fake, 0.1, 1.0, *tail) == -1
    # block table: a request with more pages than the table has columns, null table, null plan
    assert lib.mla_block_table_to_indices(dec.handle, fake, 1, fake, fake, None) == -1
    assert lib.mla_block_table_to_indices(dec.handle, None, 2, fake, fake, None) == -1
    assert lib.mla_block_table_to_indices(dec.handle, fake, -1, fake, fake, None) == -1
    assert lib.mla_block_table_to_indices(None, fake, 2, fake, fake, None) == -1
    empty = mla.mla_plan_create(0, 0, 16, 64, 1, [], [0], num_cus=4)
    assert lib.mla_block_table_to_indices(empty.handle, None, 0, None, None, None) == 0


def test_workspace_grows_with_splits(mla):
    lens = [4096] * 4
    indptr = np.concatenate([[0], np.cumsum(np.array(lens) // 64)])
    p1 = mla.mla_plan_create(0, 4, 128, 64, int(indptr[-1]), lens, indptr, num_cus=4)
    p8 = mla.mla_plan_create(0, 4, 128, 64, int(indptr[-1]), lens, indptr, num_cus=4, force_splits=8)
    assert p1.num_split_groups == 0
    assert p8.num_split_groups == 4
    assert p8.workspace_bytes >= 4 * 8 * 128 * (512 * 2 + 4)  # bf16 partial rows + fp32 lse


def test_auto_mode_choice(mla):
    # automatic tile: 128-row tile from 64 rows per request, else 16-row tile
    lens = np.array([300, 700])
    indptr = np.concatenate([[0], np.cumsum(-(-lens // 64))])
    for heads, group in ((128, 1), (64, 1), (16, 1)):
        plan = mla.mla_plan_create(0, 2, heads, 64, int(indptr[-1]), lens, indptr, num_cus=8)
        assert plan.group_size == group
        items, _ = _check_cover(plan, lens, [1, 1], heads)
        want = 128 if heads >= 64 else 16
        assert max(it["nrows"] for it in items) == min(want, heads)


def test_quad_mode_groups_siblings(mla):
    # 128 heads -> four 32-row sibling workgroups per row group, work lists
    # are a multiple of 8 so that siblings share blockIdx.x mod 8
    rng = np.random.default_rng(2)
    lens = rng.integers(512, 4097, 64)
    indptr = np.concatenate([[0], np.cumsum(-(-lens // 64))])
    plan = mla.mla_plan_create(0, 64, 128, 64, int(indptr[-1]), lens, indptr, num_cus=256,
                               tile_mode=mla.MLA_TILE_QUAD)
    assert plan.group_size == 4
    items, ptr = _check_cover(plan, lens, [1] * 64, 128)
    assert len(ptr) - 1 <= 64
    assert all(it["nrows"] == 128 for it in items)
    # a request mostly fits one work list: few split groups
    assert plan.num_split_groups <= 48


@pytest.mark.parametrize("L,splits", [(6400, 100), (4096, 64), (32768, 512), (64, 1)])
def test_quad_mode_lists_fit_the_grid(mla, L, splits):
    # forced splits add a per-piece overhead the first budget does not count;
    # the budget search must still end with no more lists than the quad grid
    # runs (num_cus / (8 G) * 8 of them, siblings sharing an XCD)
    B, H, cus = 64, 128, 256
    lens = np.full(B, L)
    indptr = np.concatenate([[0], np.cumsum(-(-lens // 64))])
    plan = mla.mla_plan_create(0, B, H, 64, int(indptr[-1]), lens, indptr, num_cus=cus,
                               tile_mode=mla.MLA_TILE_QUAD, force_splits=splits)
    G = plan.group_size
    lists = (cus // (8 * G)) * 8
    ptr = plan.workgroup_ptr()
    assert len(ptr) - 1 <= lists
    _check_cover(plan, lens, [1] * B, H)


def test_sparse_plan_and_call_errors(mla):
    lib = mla.load_library()
    sp = mla.mla_sparse_plan_create(6, 128, 1000, 300, num_cus=4)
    items = sp.work_items().numpy()
    # every query token's topk entries are covered once, in stage-aligned pieces
    for t in range(6):
        mine = sorted((int(r[3]), int(r[4])) for r in items if r[0] == t)
        assert mine[0][0] == 0 and mine[-1][1] == 300
        assert all(a[1] == b[0] for a, b in zip(mine, mine[1:]))
        assert all(a % 64 == 0 for a, _ in mine)
    assert sp.workspace_bytes >= 6 * 300 * 4
    dec = mla.mla_plan_create(0, 2, 16, 64, 4, [10, 70], [0, 1, 3], num_cus=4, kv_format=1)
    fake = ctypes.c_void_p(0x1000)
    tail = (0.1, fake, 0, fake, fake, fake, 1 << 24, None)
    assert lib.mla_sparse_decode_fp8(dec.handle, fake, fake, fake, None, None, *tail) == -4
    assert lib.mla_decode_fp8(sp.handle, *[fake] * 5, 0.1, fake, 0, fake, fake, 1 << 24, None) == -4
    assert lib.mla_sparse_decode_fp8(sp.handle, fake, fake, None, None, None, *tail) == -1
    assert lib.mla_sparse_decode_fp8(sp.handle, None, fake, fake, None, None, *tail) == -1
    assert lib.mla_sparse_decode_fp8(sp.handle, fake, fake, fake, None, None, 0.1, fake, 0, fake, fake, fake, 64,
                                     None) == -3
    h = ctypes.c_void_p()
    for args in ((-1, 128, 10, 8), (4, 0, 10, 8), (4, 128, 0, 8), (4, 128, 10, 0)):
        assert lib.mla_sparse_plan_create(ctypes.byref(h), *args, 1, 4, 0) == -1
    assert lib.mla_sparse_plan_create(ctypes.byref(h), 1 << 20, 128, 10, 1 << 12, 1, 4, 0) == -1
    assert lib.mla_sparse_plan_create(ctypes.byref(h), 4, 128, 10, 8, 7, 4, 0) == -2
    # a bf16 sparse plan is not an fp8 one, and the other way round
    spb = mla.mla_sparse_plan_create(6, 128, 1000, 300, kv_format=0, num_cus=4)
    assert lib.mla_sparse_decode_fp8(spb.handle, fake, fake, fake, None, None, *tail) == -4
    assert lib.mla_sparse_prefill(sp.handle, fake, fake, fake, None, None, *tail) == -4
    assert lib.mla_sparse_prefill(spb.handle, fake, None, fake, None, None, *tail) == -1


def test_model1_expand_argument_checks(mla):
    """Rejected before any launch: negative counts, null or misaligned
    pointers with a non-zero count; a zero count is a no-op."""
    L = mla.load_library()
    ok, bad = 0, -1
    assert L.mla_model1_expand_records(None, 0, None, None) == ok
    assert L.mla_model1_expand_records(None, -1, None, None) == bad
    assert L.mla_model1_expand_records(None, 5, None, None) == bad
    assert L.mla_model1_expand_records(2, 5, 16, None) == bad     # records not 4-byte aligned
    assert L.mla_model1_expand_records(4, 5, 8, None) == bad      # rows not 16-byte aligned
    assert L.mla_model1_expand_q(None, 0, None, None) == ok
    assert L.mla_model1_expand_q(None, -3, None, None) == bad
    assert L.mla_model1_expand_q(16, 3, 8, None) == bad


def test_boundary_option_errors(mla):
    ip = [0, 2, 3]
    kw = dict(kind=0, batch=2, num_heads=16, page_size=64, num_pages=8, kv_len=[100, 30], kv_indptr=ip, num_cus=4)
    for bad in (dict(validate=2), dict(lse_layout=2), dict(max_kv_len=-1), dict(max_seq_len_q=3),
                dict(max_kv_len=100, max_seq_len_q=2)):
        with pytest.raises(mla.MLAError) as e:
            mla.mla_plan_create(**kw, **bad)
        assert e.value.status == -1, bad
    with pytest.raises(mla.MLAError) as e:  # capacity plans are bf16 only
        mla.mla_plan_create(**dict(kw, kv_len=None, kv_indptr=None), kv_format=1, max_kv_len=100)
    assert e.value.status == -2
    qo = [0, 2, 5]
    with pytest.raises(mla.MLAError) as e:  # [batch, H, s_q] needs one query count for all requests
        mla.mla_plan_create(1, 2, 16, 64, 8, [100, 30], ip, qo_indptr=qo, lse_layout=1, num_cus=4)
    assert e.value.status == -1
    with pytest.raises(mla.MLAError) as e:  # causal capacity: more queries than keys
        mla.mla_plan_create(1, 2, 16, 64, 8, None, None, max_kv_len=4, max_seq_len_q=5, num_cus=4)
    assert e.value.status == -1
    mla.mla_plan_create(1, 2, 16, 64, 8, [100, 30], ip, qo_indptr=[0, 3, 6], lse_layout=1, num_cus=4)


@pytest.mark.parametrize("kind,mode", [(0, 1), (0, 2), (1, 1), (1, 3)])
def test_capacity_plan_covers_the_bound(mla, kind, mode):
    # every request planned at max_kv_len keys (and max_seq_len_q queries),
    # with no causal trimming: the kernels clip to the live counts
    B, H, max_kv, max_q = 5, 32, 1000, (3 if kind == 1 else 1)
    plan = mla.mla_plan_create(kind, B, H, 16, 500, None, None, tile_mode=mode, max_kv_len=max_kv,
                               max_seq_len_q=max_q if kind == 1 else 0, num_cus=64)
    _check_cover(plan, [max_kv] * B, [max_q] * B, H)
    assert all(it["t1"] <= max_kv for it in _items(plan))
