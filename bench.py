#!/usr/bin/env python3
"""Paged MLA decode benchmark on one MI355X; prints one JSON line.

A step is one mla_decode (or mla_prefill / mla_decode_fp8) call over the
whole workload: the attention kernel plus the split combine.  Inputs are
resident in HBM before the timed region.  To keep repeated steps from being
served by the 256 MB Infinity Cache, the key/value pool is replicated and
consecutive steps read different replicas (at least ~1 GB apart).

value        = algorithmic FLOP/s of the step (TFLOP/s): 2*(512+64) + 2*512
               flops per visible (row, key), masked keys excluded
kv_gb_per_s  = live latent-cache bytes / step time (each live key once)
roofline     = the attention kernel alone, timed with HIP events recorded
               around it inside the timed region, against MI355X's
               published peaks (HBM 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s)
cpu_baseline = the float64 oracle on this host's cores, timed on repeated
               passes over the same workload (bounded to ~10-30 s)
"""

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode TFLOP/s + KV GB/s (% of roofline), B=64 H=128 d=512+64"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
FLOPS_PER_ROW_KEY = 2 * (512 + 64) + 2 * 512
KV_BYTES = {"bf16": (512 + 64) * 2, "fp8": 656}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def workload_counts(w):
    """Exact algorithmic flops and bytes of a workload."""
    import numpy as np

    H = w.num_heads
    L = w.kv_len.numpy().astype(np.int64)
    n = w.q_lens().numpy().astype(np.int64)
    rows_keys = 0
    for b in range(w.batch):
        if w.kind == "prefill" and w.causal:
            vis = L[b] - n[b] + np.arange(n[b]) + 1
            rows_keys += int(vis.sum()) * H
        else:
            rows_keys += int(n[b] * L[b]) * H
    flops = rows_keys * FLOPS_PER_ROW_KEY
    live_kv = int(L.sum()) * KV_BYTES[w.kv_format]
    rows = int(n.sum())
    out_bytes = 4 if str(w.out_dtype).endswith("float32") else 2
    bytes_alg = (live_kv + rows * H * (512 + 64) * 2 + rows * H * 512 * out_bytes + rows * H * 4
                 + int(w.kv_indices.numel()) * 4)
    return flops, live_kv, bytes_alg


class HipEvents:
    """hipEvent_t handles from the HIP runtime (for the per-kernel timing)."""

    def __init__(self):
        import paged_mla_decode_05_amd as mla

        mla.load_library()
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def elapsed_ms(self, a, b):
        self.hip.hipEventSynchronize(b)
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value


def read_counters(config_name, kernel_sha):
    """HBM traffic per attention launch from committed rocprofv3 counter runs,
    if they were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"attention_{config_name}_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_sha:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _pmc_values(csv_dir, name_filter):
    """Per-dispatch values of the one counter in a rocprofv3 --pmc csv run,
    for dispatches whose kernel name contains name_filter."""
    import csv
    import glob

    vals = []
    for f in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if name_filter in r.get("Kernel_Name", ""):
                vals.append(float(r["Counter_Value"]))
    return vals


def write_counters(config_name, pmc_dir, copy_bytes, commands):
    """Summarise FETCH_SIZE / WRITE_SIZE runs of the attention kernel into
    profiles/attention_<config>_counters.txt, scaled by the same counters
    read on a plain copy kernel of known size (copy_bytes read + written).

    Layout under pmc_dir: fetch/, write/ (bench runs of the workload) and
    copy_fetch/, copy_write/ (bench --copy-calibration runs)."""
    import statistics

    cf = statistics.median(_pmc_values(os.path.join(pmc_dir, "copy_fetch"), "copy"))
    cw = statistics.median(_pmc_values(os.path.join(pmc_dir, "copy_write"), "copy"))
    kib = copy_bytes / 1024.0
    f_fetch, f_write = kib / cf, kib / cw
    fv = _pmc_values(os.path.join(pmc_dir, "fetch"), "mla_attn")
    wv = _pmc_values(os.path.join(pmc_dir, "write"), "mla_attn")
    fetch_b = statistics.median(fv) * 1024 * f_fetch
    write_b = statistics.median(wv) * 1024 * f_write
    activity = _activity_lines(os.path.join(pmc_dir, "sq"))
    path = os.path.join(ROOT, "profiles", f"attention_{config_name}_counters.txt")
    with open(path, "w") as fo:
        fo.write(f"# HBM traffic and matrix-core / LDS activity of the attention kernel, workload {config_name}\n")
        fo.write("# rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per dispatch), median over dispatches,\n")
        fo.write(f"# scaled by the same counters on a plain copy kernel of {copy_bytes} bytes read + written\n")
        for c in commands:
            fo.write(f"# command: {c}\n")
        fo.write(f"kernel_source_sha256: {kernel_sha()}\n")
        fo.write(f"copy_fetch_kib: {cf:.1f}\ncopy_write_kib: {cw:.1f}\n")
        fo.write(f"fetch_scale: {f_fetch:.4f}\nwrite_scale: {f_write:.4f}\n")
        fo.write(f"attention_fetch_kib_median: {statistics.median(fv):.1f}  (n={len(fv)})\n")
        fo.write(f"attention_write_kib_median: {statistics.median(wv):.1f}  (n={len(wv)})\n")
        fo.write(f"hbm_fetch_bytes_per_launch: {fetch_b:.0f}\n")
        fo.write(f"hbm_write_bytes_per_launch: {write_b:.0f}\n")
        fo.write(f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}\n")
        for line in activity:
            fo.write(line + "\n")
    return path


def _activity_lines(sq_dir):
    """Matrix-core and LDS activity of the attention kernel from one
    rocprofv3 --pmc run of SQ counters (medians over dispatches):
    SQ_VALU_MFMA_BUSY_CYCLES (cycles, summed over SIMDs), SQ_WAVE_CYCLES
    (quad-cycles, summed over waves; one wave per SIMD here, so 4x it is the
    SIMD-cycles the waves were resident), SQ_LDS_IDX_ACTIVE and
    SQ_LDS_BANK_CONFLICT (LDS cycles, summed over CUs), instruction counts.
    Empty when the run is absent."""
    import csv
    import glob
    import statistics

    per = {}
    for f in glob.glob(os.path.join(sq_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if "mla_attn" not in r.get("Kernel_Name", ""):
                continue
            key = (r["Dispatch_Id"], r["Counter_Name"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        return []
    names = sorted({k[1] for k in per})
    med = {n: statistics.median([v for (d, c), v in per.items() if c == n]) for n in names}
    out = ["# activity: rocprofv3 --pmc SQ counters of the same kernel (median per dispatch)"]
    out += [f"{n}: {med[n]:.0f}" for n in names]
    busy, waves = med.get("SQ_VALU_MFMA_BUSY_CYCLES"), med.get("SQ_WAVE_CYCLES")
    if busy is not None and waves:
        out.append(f"mfma_busy_per_resident_simd_cycle: {busy / (4.0 * waves):.4f}")
    conf, act = med.get("SQ_LDS_BANK_CONFLICT"), med.get("SQ_LDS_IDX_ACTIVE")
    if conf is not None and act:
        out.append(f"lds_bank_conflict_share_of_lds_active_cycles: {conf / act:.4f}")
    if act is not None and waves:
        out.append(f"lds_active_cycles_per_resident_cu_cycle: {act / waves:.4f}")
    vi, mi = med.get("SQ_INSTS_VALU"), med.get("SQ_INSTS_MFMA")
    if vi is not None and mi:
        out.append(f"valu_instructions_per_mfma: {(vi - mi) / mi:.2f}")
    return out


def copy_calibration(nbytes):
    """A plain device copy of nbytes (read nbytes, write nbytes), five times."""
    import torch

    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4, "repeats": 5}), flush=True)


def kernel_sha():
    import hashlib

    h = hashlib.sha256()
    for f in ("mla_attn.hip", "mla_internal.h"):
        h.update(open(os.path.join(ROOT, "paged_mla_decode_05_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def host_description():
    """CPU model (lscpu), usable cores and the thread environment of the oracle run."""
    import subprocess

    model = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except Exception:  # pragma: no cover
        pass
    if model is None:
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        except OSError:  # pragma: no cover
            pass
    env = {k: os.environ[k] for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS",
                                      "NUMEXPR_NUM_THREADS") if k in os.environ}
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)), "thread_env": env}


def cpu_baseline(w, flops_total, min_seconds):
    """Time the oracle on repeated passes over the workload's requests."""
    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    # host copies once, outside the timed region
    if w.kind == "prefill":
        args = (w.q_nope.cpu(), w.q_pe.cpu(), w.ckv.cpu(), w.kpe.cpu(), w.qo_indptr, w.kv_indptr,
                w.kv_indices, w.kv_len, w.sm_scale)
        fn = lambda reqs: oracle.mla_prefill_ref(*args, causal=w.causal, requests=reqs)
    elif w.kv_format == "fp8":
        args = (w.q_nope.cpu(), w.q_pe.cpu(), w.kv_fp8.cpu(), w.kv_indptr, w.kv_indices, w.kv_len, w.sm_scale)
        fn = lambda reqs: oracle.mla_decode_fp8_ref(*args, requests=reqs)
    else:
        args = (w.q_nope.cpu(), w.q_pe.cpu(), w.ckv.cpu(), w.kpe.cpu(), w.kv_indptr, w.kv_indices, w.kv_len,
                w.sm_scale)
        fn = lambda reqs: oracle.mla_decode_ref(*args, requests=reqs)
    import numpy as np

    L = w.kv_len.numpy().astype(np.int64)
    n = w.q_lens().numpy().astype(np.int64)
    per_req = []
    for b in range(w.batch):
        if w.kind == "prefill" and w.causal:
            keys = int((L[b] - n[b] + np.arange(n[b]) + 1).sum())
        else:
            keys = int(n[b] * L[b])
        per_req.append(keys * w.num_heads * FLOPS_PER_ROW_KEY)
    done_flops = 0.0
    reqs_done = 0
    t0 = time.perf_counter()
    stop = False
    while not stop:
        for b in range(w.batch):
            fn([b])
            reqs_done += 1
            done_flops += per_req[b]
            if time.perf_counter() - t0 >= 30.0:
                stop = True
                break
        if time.perf_counter() - t0 >= min_seconds:
            stop = True
    dt = time.perf_counter() - t0
    return {"value": done_flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{reqs_done} request evaluations ({reqs_done / w.batch:.2f} passes over all "
                      f"{w.batch} requests of {w.name}), {dt:.1f} s wall, float64 NumPy",
}


def setup_dense(args, mla, dev):
    """Plan, inputs and step of a paged dense workload (decode, prefill, fp8 decode)."""
    import torch

    from workloads import make_workload

    log(f"bench: generating {args.config} on {dev}")
    w = make_workload(args.config, device=dev, poison=False)
    flops, live_kv, bytes_alg = workload_counts(w)
    fmt = mla.MLA_KV_FP8_E4M3_T128 if w.kv_format == "fp8" else mla.MLA_KV_BF16
    kind = mla.MLA_KIND_PREFILL if w.kind == "prefill" else mla.MLA_KIND_DECODE
    t_plan = time.perf_counter()
    plan = mla.mla_plan_create(kind, w.batch, w.num_heads, w.page_size, w.num_pages, w.kv_len, w.kv_indptr,
                               qo_indptr=w.qo_indptr if w.kind == "prefill" else None, kv_format=fmt,
                               causal=w.causal, tile_mode=args.tile_mode)
    plan_ms = (time.perf_counter() - t_plan) * 1e3
    kv_indptr = w.kv_indptr.to(dev)
    kv_indices = w.kv_indices.to(dev)
    qo_indptr = w.qo_indptr.to(dev) if w.qo_indptr is not None else None
    pool_bytes = (w.kv_fp8.numel() if fmt else (w.ckv.numel() + w.kpe.numel()) * 2)
    reps = max(1, min(16, math.ceil(args.rotate_bytes / max(live_kv, 1))))
    pools = [(w.ckv, w.kpe, w.kv_fp8)]
    for _ in range(reps - 1):
        pools.append((w.ckv.clone() if w.ckv is not None else None, w.kpe.clone() if w.kpe is not None else None,
                      w.kv_fp8.clone() if w.kv_fp8 is not None else None))
    if args.q_fp8 and not fmt:
        raise SystemExit("--q-fp8 applies to the fp8 cache only")
    q8 = None
    if args.q_fp8:
        from workloads import quantize_q_e4m3

        q8 = quantize_q_e4m3(w.q_nope, w.q_pe)
        bytes_alg -= w.rows * w.num_heads * 576  # one byte per query dim instead of two
    packed = args.layout == "packed"
    if packed:
        if fmt:
            raise SystemExit("--layout packed applies to the bf16 cache only")
        q_cat = torch.cat([w.q_nope, w.q_pe], dim=-1).contiguous()
        pools = [(torch.cat([c, k], dim=-1).contiguous(), None, None) for c, k, _ in pools]
        torch.cuda.empty_cache()
    out = torch.empty((w.rows, w.num_heads, 512), dtype=w.out_dtype, device=dev)
    lse = torch.empty((w.rows, w.num_heads), dtype=torch.float32, device=dev)
    ws = plan.workspace(dev)
    log(f"bench: {plan.num_work_items} work items on {plan.workgroup_ptr().numel() - 1} workgroups, "
        f"{plan.num_split_groups} split groups, workspace {plan.workspace_bytes / 1e6:.1f} MB, "
        f"{reps} pool replicas of {pool_bytes / 1e6:.0f} MB")

    def step(i):
        ckv, kpe, kv8 = pools[i % reps]
        if q8 is not None:
            mla.mla_decode_fp8_q8(plan, q8, kv8, kv_indptr, kv_indices, w.sm_scale, out=out, lse=lse, workspace=ws)
        elif fmt:
            mla.mla_decode_fp8(plan, w.q_nope, w.q_pe, kv8, kv_indptr, kv_indices, w.sm_scale, out=out, lse=lse,
                               workspace=ws)
        elif packed and kind == mla.MLA_KIND_PREFILL:
            mla.mla_prefill_packed(plan, q_cat, ckv, qo_indptr, kv_indptr, kv_indices, w.sm_scale, out=out, lse=lse,
                                   workspace=ws)
        elif packed:
            mla.mla_decode_packed(plan, q_cat, ckv, kv_indptr, kv_indices, w.sm_scale, out=out, lse=lse, workspace=ws)
        elif kind == mla.MLA_KIND_PREFILL:
            mla.mla_prefill(plan, w.q_nope, w.q_pe, ckv, kpe, qo_indptr, kv_indptr, kv_indices, w.sm_scale,
                            out=out, lse=lse, workspace=ws)
        else:
            mla.mla_decode(plan, w.q_nope, w.q_pe, ckv, kpe, kv_indptr, kv_indices, w.sm_scale, out=out,
                           lse=lse, workspace=ws)

    config = {"workload": w.name, "batch": w.batch, "num_qo_heads": w.num_heads, "head_dim_ckv": 512,
              "head_dim_kpe": 64, "page_size": w.page_size, "kv_format": w.kv_format,
              "kv_len_total": int(w.kv_len.sum()), "rows": w.rows, "parallelism": "single GPU",
              "layout": args.layout, "q_dtype": "fp8-e4m3" if q8 is not None else "bf16"}
    dtype = "bf16" if w.kv_format == "bf16" else "fp8-e4m3 cache, bf16 math"
    if q8 is not None:
        dtype = "fp8-e4m3 q and cache: fp8 x fp8 MFMA for the latent q.k, bf16 P.V"
    # the e4m3-query kernel runs the latent q.k (2 * 512 of the 2176 flops per
    # row and key) on the fp8 matrix cores and the rest on bf16 ones: its
    # peak is the time-weighted blend of the two
    peak = BF16_PEAK_TFLOPS
    if q8 is not None:
        f8, f16 = 2 * 512, FLOPS_PER_ROW_KEY - 2 * 512
        peak = FLOPS_PER_ROW_KEY / (f8 / FP8_PEAK_TFLOPS + f16 / BF16_PEAK_TFLOPS)
    return {"step": step, "flops": flops, "live_kv": live_kv, "bytes_alg": bytes_alg, "plan_ms": plan_ms,
            "config": config, "kernel": "mla_attn_kernel", "mfma_peak": peak,
            "dtype": dtype,
            "cpu_baseline": lambda secs: cpu_baseline(w, flops, secs)}


def setup_model1(args, mla, dev):
    """Decode over MODEL1 records (448 NoPE dims in 7 tiles of 64 + 64 RoPE
    dims, 604 bytes per token), dequantised in the attention kernel
    (mla_decode_model1): one step is that call.

    Algorithmic units of the MODEL1 attention: 2*512 + 2*448 = 1920 flops per
    visible (row, key); bytes = live records (604 B per token) + q (1024 B per
    row) + out (896 B per row, 448 bf16 dims) + lse + page indices."""
    import numpy as np
    import torch

    from workloads import make_model1_workload

    log(f"bench: generating {args.config} on {dev}")
    w = make_model1_workload(name=args.config, device=dev, poison=False)
    L = w.kv_len.numpy().astype(np.int64)
    H = w.num_heads
    flops = int(L.sum()) * H * (2 * 512 + 2 * 448)
    live = int(L.sum()) * 604
    bytes_alg = live + w.batch * H * (1024 + 896 + 4) + int(w.kv_indptr[-1]) * 4
    t_plan = time.perf_counter()
    plan = mla.mla_plan_create(mla.MLA_KIND_DECODE, w.batch, H, w.page_size, w.num_pages, w.kv_len, w.kv_indptr,
                               kv_format=mla.MLA_KV_FP8_MODEL1, tile_mode=args.tile_mode)
    plan_ms = (time.perf_counter() - t_plan) * 1e3
    kv_indptr = w.kv_indptr.to(dev)
    kv_indices = w.kv_indices.to(dev)
    reps = max(1, min(16, math.ceil(args.rotate_bytes / max(w.records.numel(), 1))))
    pools = [w.records] + [w.records.clone() for _ in range(reps - 1)]
    out = torch.empty((w.batch, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, H), dtype=torch.float32, device=dev)
    ws = plan.workspace(dev)
    log(f"bench: {plan.num_work_items} work items on {plan.workgroup_ptr().numel() - 1} workgroups, "
        f"{plan.num_split_groups} split groups, {reps} record pool replicas of {w.records.numel() / 1e6:.0f} MB")

    def step(i):
        mla.mla_decode_model1(plan, w.q, pools[i % reps], kv_indptr, kv_indices, w.sm_scale, out=out, lse=lse,
                              workspace=ws)

    def cpu(secs):
        import oracle

        args_ = (w.q.cpu(), w.records.cpu(), w.kv_indptr, w.kv_indices, w.kv_len, w.sm_scale)
        done = 0.0
        n = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < secs:
            b = n % w.batch
            oracle.mla_decode_model1_ref(*args_, requests=[b])
            done += int(L[b]) * H * 1920
            n += 1
        dt = time.perf_counter() - t0
        return {"value": done / dt / 1e12, "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
                "sample": f"{n} request evaluations of {w.name}, {dt:.1f} s wall, float64 NumPy"}

    config = {"workload": w.name, "batch": w.batch, "num_qo_heads": H, "head_dim_nope": 448, "head_dim_kpe": 64,
              "page_size": w.page_size, "kv_format": "MODEL1 fp8 records (604 B)", "kv_len_total": int(L.sum()),
              "rows": w.batch, "parallelism": "single GPU"}
    return {"step": step, "flops": flops, "live_kv": live, "bytes_alg": bytes_alg, "plan_ms": plan_ms,
            "config": config, "kernel": "mla_attn_kernel",
            "dtype": "MODEL1 e4m3 records read in the kernel, bf16 math", "cpu_baseline": cpu}


def setup_sparse(args, mla, dev):
    """Plan, inputs and step of a token-sparse workload (fp8 records, or bf16
    KV rows for the sparse prefill form).

    Algorithmic units: each valid (query token, list entry) costs 2176 flops
    per head; bytes are the distinct key rows the lists name (656 B per fp8
    record, 1152 B per bf16 row: a row named by several lists is needed once
    per launch), the lists (4 B per entry), q (1152 B per row), out, lse and
    max_logits."""
    import numpy as np
    import torch

    from workloads import SPARSE_PREFILL_CONFIGS, make_sparse_prefill_workload, make_sparse_workload

    log(f"bench: generating {args.config} on {dev}")
    bf16_rows = args.config in SPARSE_PREFILL_CONFIGS
    if bf16_rows:
        w = make_sparse_prefill_workload(args.config, device=dev)
        cache, row_bytes, fmt = w.kv, KV_BYTES["bf16"], mla.MLA_KV_BF16
    else:
        w = make_sparse_workload(args.config, device=dev, poison=False)
        cache, row_bytes, fmt = w.kv_fp8, KV_BYTES["fp8"], mla.MLA_KV_FP8_E4M3_T128
    idx = w.indices.numpy().astype(np.int64)
    lim = idx.shape[1] if w.topk_length is None else w.topk_length.numpy()[:, None]
    valid = (idx >= 0) & (idx < w.num_slots) & (np.arange(idx.shape[1])[None, :] < lim)
    n_valid = valid.sum(axis=1)
    H, T = w.num_heads, w.tokens
    flops = int(n_valid.sum()) * H * FLOPS_PER_ROW_KEY
    live_kv = int(np.unique(idx[valid]).size) * row_bytes
    out_bytes = 4 if str(w.out_dtype).endswith("float32") else 2
    bytes_alg = live_kv + T * H * (576 * 2 + 512 * out_bytes + 4 + 4) + idx.size * 4
    t_plan = time.perf_counter()
    plan = mla.mla_sparse_plan_create(T, H, w.num_slots, w.topk, kv_format=fmt)
    plan_ms = (time.perf_counter() - t_plan) * 1e3
    indices = w.indices.to(dev)
    reps = max(1, min(16, math.ceil(args.rotate_bytes / max(live_kv, 1))))
    pools = [cache] + [cache.clone() for _ in range(reps - 1)]
    out = torch.empty((T, H, 512), dtype=w.out_dtype, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    mx = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = plan.workspace(dev)
    log(f"bench: {plan.num_work_items} work items on {plan.workgroup_ptr().numel() - 1} workgroups, "
        f"{plan.num_split_groups} split groups, workspace {plan.workspace_bytes / 1e6:.1f} MB, "
        f"{reps} pool replicas of {cache.numel() * cache.element_size() / 1e6:.0f} MB, "
        f"{int(n_valid.sum())} valid entries")
    run = mla.mla_sparse_prefill if bf16_rows else mla.mla_sparse_decode_fp8

    def step(i):
        run(plan, w.q, pools[i % reps], indices, w.sm_scale, out=out, lse=lse, max_logits=mx, workspace=ws)

    def cpu(secs):
        import oracle

        try:
            from threadpoolctl import threadpool_info

            threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        except Exception:  # pragma: no cover
            threads = os.cpu_count()
        q_host, kv_host = w.q.cpu(), cache.cpu()
        ref = oracle.mla_sparse_prefill_ref if bf16_rows else oracle.mla_sparse_decode_fp8_ref
        done, n = 0.0, 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < secs:
            t = n % T
            ref(q_host, kv_host, w.indices, w.sm_scale, tokens=[t])
            done += int(n_valid[t]) * H * FLOPS_PER_ROW_KEY
            n += 1
        dt = time.perf_counter() - t0
        return {"value": done / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
                "sample": f"{n} query-token evaluations of {w.name} ({n / T:.2f} passes over its {T} tokens), "
                          f"{dt:.1f} s wall, float64 NumPy"}

    if bf16_rows:
        config = {"workload": w.name, "s_q": T, "s_kv": w.num_slots, "num_qo_heads": H, "topk": w.topk,
                  "head_dim_ckv": 512, "head_dim_kpe": 64, "kv_format": "bf16"}
    else:
        config = {"workload": w.name, "batch": w.batch, "s_q": w.s_q, "num_qo_heads": H, "topk": w.topk,
                  "head_dim_ckv": 512, "head_dim_kpe": 64, "kv_format": "fp8", "page_size": w.page_size}
    config.update({"valid_entries": int(n_valid.sum()), "distinct_key_rows": live_kv // row_bytes, "rows": T,
                   "parallelism": "single GPU"})
    return {"step": step, "flops": flops, "live_kv": live_kv, "bytes_alg": bytes_alg, "plan_ms": plan_ms,
            "config": config, "kernel": "mla_attn_kernel (token-sparse " + ("bf16)" if bf16_rows else "fp8)"),
            "dtype": "bf16" if bf16_rows else "fp8-e4m3 cache, bf16 math", "cpu_baseline": cpu}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="decode_b64_h128")
    ap.add_argument("--rotate-bytes", type=float, default=1.5e9,
                    help="replicate the cache pool until consecutive steps are this many bytes apart")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tile-mode", type=int, default=0,
                    help="0 = planner's choice; 1 wide, 2 narrow, 3 quad")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES (counter calibration) and exit")
    ap.add_argument("--write-counters", metavar="PMC_DIR",
                    help="summarise rocprofv3 FETCH_SIZE/WRITE_SIZE runs under PMC_DIR into profiles/ and exit")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--layout", choices=("split", "packed"), default="split",
                    help="bf16 q / cache as separate latent and rope tensors, or one 576-wide row per token")
    ap.add_argument("--q-fp8", action="store_true",
                    help="fp8 cache workloads: an e4m3 query (fp8 x fp8 matrix cores for the latent q.k)")
    ap.add_argument("--command", action="append", default=[], help="command lines recorded with --write-counters")
    args = ap.parse_args()

    if args.write_counters:
        print(write_counters(args.config, args.write_counters, args.copy_bytes, args.command))
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(one MI355X share of the workload is what it measures).", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_mla_decode_05_amd as mla
    from workloads import MODEL1_CONFIGS, SPARSE_CONFIGS, SPARSE_PREFILL_CONFIGS

    if not os.path.exists(mla.lib_path()):
        import __graft_entry__

        __graft_entry__.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.config in MODEL1_CONFIGS:
        setup = setup_model1
    elif args.config in SPARSE_CONFIGS or args.config in SPARSE_PREFILL_CONFIGS:
        setup = setup_sparse
    else:
        setup = setup_dense
    S = setup(args, mla, dev)
    step, flops, live_kv, bytes_alg, plan_ms = S["step"], S["flops"], S["live_kv"], S["bytes_alg"], S["plan_ms"]

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"bench: warmup {args.warmup} done; timing {args.steps} steps")

    # Inside the timed region every EVENT_EVERY-th step has the attention
    # kernel's dispatch record its own start / end events (its launch
    # duration); a step that records them runs 5-7 us longer (the kernel
    # trace shows the gaps), so they are taken on one step in ten.
    EVENT_EVERY = 10
    sampled = list(range(0, args.steps, EVENT_EVERY))
    ev = HipEvents()
    kb = {i: ev.create() for i in sampled}
    ke = {i: ev.create() for i in sampled}
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        if i in kb:
            mla.mla_record_attention_events(kb[i], ke[i])
        step(args.warmup + i)
    t_end.record()
    issued = time.perf_counter() - wall0
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    attn_ms = sorted(ev.elapsed_ms(kb[i], ke[i]) for i in sampled)
    attn_avg = sum(attn_ms) / len(attn_ms)
    # host time to issue a step: when it approaches the step time, the
    # launches (not the GPU) set the pace
    log(f"bench: host issue {issued / args.steps * 1e6:.1f} us/step")
    log(f"bench: {ms_step * 1e3:.1f} us/step (wall {wall / args.steps * 1e6:.1f} us), attention kernel avg "
        f"{attn_avg * 1e3:.1f} us (p10 {attn_ms[len(attn_ms) // 10] * 1e3:.1f}, "
        f"p90 {attn_ms[(9 * len(attn_ms)) // 10] * 1e3:.1f})")

    mfma_peak = S.get("mfma_peak", BF16_PEAK_TFLOPS)
    ai = flops / bytes_alg
    ridge = mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    hbm_bound = ai < ridge
    t_s = ms_step * 1e-3
    ta_s = attn_avg * 1e-3
    tflops = flops / t_s / 1e12
    kv_gbs = live_kv / t_s / 1e9
    pct = 100.0 * max((bytes_alg / (HBM_PEAK_GBS * 1e9)), flops / (mfma_peak * 1e12)) / t_s
    sha = kernel_sha()
    # counters are per kernel variant: the e4m3-query and packed-layout runs
    # launch other instantiations than the default run they share a workload with
    variant = args.config + ("_q8" if args.q_fp8 else "") + ("_packed" if args.layout == "packed" else "")
    traffic = read_counters(variant, sha)
    if traffic is not None:
        log(f"bench: HBM traffic per attention launch {traffic / 1e6:.1f} MB "
            f"({traffic / bytes_alg:.2f}x the algorithmic {bytes_alg / 1e6:.1f} MB)")
    if hbm_bound:
        achieved = bytes_alg / ta_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": (round(traffic / ta_s / 1e9, 1) if traffic is not None else None)}
    else:
        achieved = flops / ta_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": round(mfma_peak, 1), "unit": "TFLOP/s",
                "frac": round(achieved / mfma_peak, 4),
                "traffic": (round(traffic / ta_s / 1e9, 1) if traffic is not None else None)}
    roof["kernel"] = S["kernel"]
    roof["kernel_avg_us"] = round(attn_avg * 1e3, 2)
    roof["algorithmic_bytes_per_launch"] = bytes_alg
    roof["algorithmic_flops_per_launch"] = flops
    if traffic is not None:
        roof["traffic_bytes_per_launch"] = round(traffic)
        roof["traffic_note"] = ("GB/s: HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-kernel "
                                "scaled) / average launch time")
    result_steps = {"p10_us": round(attn_ms[len(attn_ms) // 10] * 1e3, 2),
                    "p90_us": round(attn_ms[(9 * len(attn_ms)) // 10] * 1e3, 2),
                    "median_us": round(attn_ms[len(attn_ms) // 2] * 1e3, 2)}
    roof["kernel_time"] = result_steps

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": S["dtype"],
        "data": "synthetic (seeded N(0,1) bf16 inputs shaped like the workload)",
        "config": S["config"],
        "kv_gb_per_s": round(kv_gbs, 1),
        "pct_of_roofline": round(pct, 2),
        "plan_ms": round(plan_ms, 3),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle")
        result["cpu_baseline"] = S["cpu_baseline"](args.cpu_seconds)
        result["cpu_baseline"]["host"] = host_description()
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
