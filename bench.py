"""Benchmark of the hot path on one MI355X: top-k KV-tile selection + block-sparse attention.

One step = nsa_select (pool, score, top-k, CSR) + nsa_block_sparse_attn over one
batch of the long-context workload (B 1, Hq 64, Hkv 8, S 131072, D 128, bf16,
causal, block_q 128 / block_kv 64, budget 0.05, sink tile pinned, 1% of
non-diagonal tiles dropped), inputs resident in HBM.

value = attention FLOPs over kept tiles (tiles entirely in the causal future
excluded, full tile area otherwise: 4 * D * |Q_i| * |K_j| per kept tile and
query head) divided by the wall time of a whole step.

Prints ONE JSON line (see the keys below). Usage:
  python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
import top_kv_tile_amd as tkt  # noqa: E402

METRIC = "block-sparse attn TFLOP/s over kept tiles (+% MFMA peak); select GB/s"
WORKLOAD = "long_causal_gqa_bf16_s128k"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
ATTN_KERNEL_SRC = os.path.join(ROOT, "top_kv_tile_amd", "csrc", "attn_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", f"attn_fwd_{WORKLOAD}_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kept_tile_flops(sel: tkt.Selection, w: synth.Workload):
    """(full-tile FLOPs, visible-pair FLOPs, kept tiles visited) over all query heads."""
    row_ptr = sel.row_ptr.cpu().numpy().astype(np.int64)
    col = sel.col_idx.cpu().numpy().astype(np.int64)
    B, H, NQ, NK = sel.keep.shape
    rows = np.arange(B * H * NQ)
    counts = np.diff(row_ptr)
    row_of = np.repeat(rows, counts)
    ti = row_of % NQ
    q_lo = ti * w.block_q
    q_hi = np.minimum(q_lo + w.block_q, w.S)          # exclusive
    k_lo = col * w.block_kv
    k_hi = np.minimum(k_lo + w.block_kv, w.S)
    if w.causal:
        live = k_lo <= q_hi - 1
    else:
        live = np.ones_like(k_lo, bool)
    area = (q_hi - q_lo) * (k_hi - k_lo)
    if w.causal:
        # visible pairs of a tile: sum over queries t in [q_lo, q_hi) of
        # clip(t - k_lo + 1, 0, n), n = k_hi - k_lo (a ramp, then n per query)
        n = k_hi - k_lo
        t_flat = k_lo + n - 1
        r_lo, r_hi = np.maximum(q_lo, k_lo), np.minimum(q_hi - 1, t_flat - 1)
        m = np.clip(r_hi - r_lo + 1, 0, None)
        first = r_lo - k_lo + 1
        vis = m * first + m * (m - 1) // 2
        vis = vis + np.clip(q_hi - 1 - np.maximum(q_lo, t_flat) + 1, 0, None) * n
    else:
        vis = area
    heads_per_row = (w.Hq // H)
    D = w.D
    full = float(4 * D * (area * live).sum() * heads_per_row)
    visible = float(4 * D * vis.sum() * heads_per_row)
    return full, visible, int(live.sum()) * heads_per_row


def read_traffic():
    """Counter-based HBM traffic per attention launch from the committed profile, or None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                a, b = line.split(":", 1)
                kv[a.strip()] = b.strip()
    try:
        src_hash = hashlib.sha256(open(ATTN_KERNEL_SRC, "rb").read()).hexdigest()
        if kv.get("kernel_source_sha256") != src_hash:
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _oracle_attention_threaded(inp, w: synth.Workload, keep, rows, threads: int) -> float:
    """Wall time of oracle.attention over `rows` (b, h, i), one query head's slice
    per call (q[b, h], its kv head, its selection plane), `threads` calls at a
    time with BLAS held to one thread each, so the per-row work occupies the
    cores the way one large BLAS call would."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from threadpoolctl import threadpool_limits

    group = w.Hq // w.Hkv
    by_head = {}
    for b, h, i in rows:
        by_head.setdefault((b, h), []).append(i)
    jobs = [(b, h, t) for (b, h), t in sorted(by_head.items())]

    def run(job):
        b, h, tiles = job
        g = h // group
        kb = b if keep.shape[0] == w.B else 0
        hs = h if keep.shape[1] == w.Hq else 0
        oracle.attention(inp.q[b:b + 1, h:h + 1], inp.k[b:b + 1, g:g + 1], inp.v[b:b + 1, g:g + 1],
                         keep[kb:kb + 1, hs:hs + 1], w.block_q, w.block_kv, w.causal,
                         rows=[(0, 0, i) for i in tiles])

    nthr = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        with threadpool_limits(1), ThreadPoolExecutor(threads) as ex:
            list(ex.map(run, jobs))
        return time.perf_counter() - t0
    finally:
        torch.set_num_threads(nthr)


def cpu_baseline(inp, w: synth.Workload, full_flops: float, heads_per_index: int = 4):
    """The oracle, untuned, on the host cores: oracle.select_blocks on the whole
    workload, and oracle.attention (fp64) on a seeded 1/16 of the (b, h, q-tile)
    rows (heads_per_index heads for every query-tile index), extrapolated
    linearly to all rows. value = the step's kept-tile FLOPs / that time."""
    import oracle

    threads = max(1, min(16, os.cpu_count() or 1))
    t0 = time.perf_counter()
    ref = oracle.select_blocks(inp.q, inp.k, w.budget, w.block_q, w.block_kv, w.head_shared, False,
                               inp.pins, inp.drops)
    t_sel = time.perf_counter() - t0
    rng = np.random.default_rng(11)
    rows = []
    for i in range(w.nq):
        for p in rng.choice(w.B * w.Hq, size=min(heads_per_index, w.B * w.Hq), replace=False):
            rows.append((int(p) // w.Hq, int(p) % w.Hq, i))
    total_rows = w.B * w.Hq * w.nq
    t_att = _oracle_attention_threaded(inp, w, ref["keep"], rows, threads)
    frac = len(rows) / total_rows
    t_step = t_sel + t_att / frac
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": full_flops / t_step / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "host_cpus": os.cpu_count(), "cpu_model": cpu_model,
        "select_s": round(t_sel, 2), "attn_sample_s": round(t_att, 2), "attn_sample_rows": len(rows),
        "attn_sample_frac": frac, "step_s_extrapolated": round(t_step, 2),
        "sample": (f"oracle.select_blocks on the whole workload ({w.B * (1 if w.head_shared else w.Hq) * w.nq} "
                   f"rows, {t_sel:.1f} s, torch/numpy on {torch.get_num_threads()} threads) + oracle.attention "
                   f"(fp64) on a seeded 1/{round(1 / frac)} of the query rows ({len(rows)} rows: "
                   f"{heads_per_index} heads per query-tile index, {t_att:.1f} s on {threads} threads, one "
                   f"head slice per call), extrapolated linearly to all rows; value = the step's kept-tile "
                   f"FLOPs over select + extrapolated attention time"),
    }


def backward_timing(q, k, v, out, lse, sel, w: synth.Workload, fwd_flops: float, steps: int):
    """Times nsa_block_sparse_attn_bwd on the step's selection, outside the step.

    Kept-tile FLOPs of the gradients are 2.5x the forward's (five products per
    tile: S, dP, dQ, dK, dV against the forward's two); the kernels compute S and
    dP twice (once per kernel), 3.5x in all, which is not counted."""
    dev = q.device
    g = torch.Generator(device=dev).manual_seed(2024)
    dout = torch.randn(q.shape, generator=g, device=dev, dtype=torch.float32).to(q.dtype)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(1, tkt.nsa_attn_bwd_workspace_size(q, k, sel)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def call():
        tkt.nsa_block_sparse_attn_bwd(q, k, v, out, lse, dout, sel, w.causal, workspace=ws, dq=dq, dk=dk, dv=dv)

    log("[bench] backward warmup")
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    log(f"[bench] backward timing {steps} calls")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e in ev:
        e[0].record(stream)
        call()
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    flops = 2.5 * fwd_flops
    tflops = flops / (ms * 1e-3) / 1e12
    # Per-kernel device time from the library's stage events (3 more calls):
    # delta, the kv-major index, dQ (S, dP and dQ products: 1.5x the forward's
    # kept-tile FLOPs executed) and dK/dV (S, dP, dV and dK: 2x).
    tkt.nsa_stage_timing_begin()
    for _ in range(3):
        call()
    recs = tkt.nsa_stage_timing_end()
    per = {}
    for name, t in recs:
        per.setdefault(name, []).append(t)
    kernels = {}
    for name, xs in per.items():
        kms = float(np.median(xs))
        d = {"ms": round(kms, 3)}
        mult = {"dq": 1.5, "dkdv": 2.0}.get(name)
        if mult:
            d["executed_TFLOPs"] = round(mult * fwd_flops / (kms * 1e-3) / 1e12, 2)
            d["executed_frac_bf16_peak"] = round(d["executed_TFLOPs"] / PEAK_BF16_TFLOPS, 4)
        kernels[name] = d
    return {"ms": round(ms, 3), "kept_tile_flops_per_call": flops, "TFLOPs": round(tflops, 2),
            "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4), "kernels": kernels,
            "kernel_names": "delta_kernel, kv-major index (colcount, colscan x3, colfill), "
                            "bwd_dq_mfma_kernel<128,4>, bwd_dkdv_mfma_kernel<128>"}


def _event_ms(fn, calls: int, stream, queued: bool = False) -> float:
    """Mean duration of fn() in ms, HIP events around each call on `stream`.

    queued=True puts a GPU spin of a few ms on the stream before each batch of
    8 calls, so the host enqueues the batch before the device reaches it: the
    events then time the device work of a call (its kernels and the gaps
    between them), not the host-side argument handling of a Python caller.
    (Batches of 8: the library's pinned upload ring has 8 slots, and a ninth
    queued upload would wait for the first.)"""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    batch = 8 if queued else calls
    for b0 in range(0, calls, batch):
        if queued:
            torch.cuda._sleep(int(5e6))
        for e in ev[b0:b0 + batch]:
            e[0].record(stream)
            fn()
            e[1].record(stream)
        torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def measured_peaks(reps: int = 10) -> dict:
    """Rates this box reaches on two plain references, timed with events:
    a contiguous 8192^3 bf16 GEMM through torch (the vendor GEMM library) and
    a 2 GiB device-to-device copy (2 GiB read + 2 GiB written per call)."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(0)
    n = 8192
    a = torch.randn(n, n, generator=g, device=dev).to(torch.bfloat16)
    b = torch.randn(n, n, generator=g, device=dev).to(torch.bfloat16)
    c = torch.empty(n, n, dtype=torch.bfloat16, device=dev)
    x = torch.empty(1 << 29, dtype=torch.float32, device=dev)  # 2 GiB
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        torch.matmul(a, b, out=c)
        y.copy_(x)
    gemm_ms = _event_ms(lambda: torch.matmul(a, b, out=c), reps, stream)
    copy_ms = _event_ms(lambda: y.copy_(x), reps, stream)
    del a, b, c, x, y
    return {"bf16_gemm_TFLOPs": round(2 * n ** 3 / (gemm_ms * 1e-3) / 1e12, 1),
            "torch_copy_GBps": round(2 * (1 << 31) / (copy_ms * 1e-3) / 1e9, 1),
            "how": "8192^3 bf16 torch.matmul and a 2 GiB torch tensor copy on the same GPU, events, "
                   f"mean of {reps} calls; torch's copy streams slower than this library's own "
                   "pooling and permutation kernels, so HBM fractions use the published 8 TB/s"}


PEAK_FP32_TFLOPS = 157.3     # MI355X dense fp32 (matrix and vector)


def stage_timing(plan, plan_dev, q, k, ws, sel: tkt.Selection, w: synth.Workload, spec: tkt.SparseSpec,
                 calls: int = 20) -> dict:
    """Device time of every selection stage, from the library's stage events,
    over `calls` planned selections (run after the timed steps, same inputs),
    with each stage's algorithmic bytes (and FLOPs for the score product):
      pool_q / pool_k: read q / k once, write the pooled fp32 means;
      scores_c (head chunk c): 2 * B * nh * NQ * NK * D FLOP, writes the chunk's fp32 scores
        (with more than 64 query tiles per head the library runs them as six bf16 matrix
        products per fp32 one, on split operands: that executed rate is reported too);
      topk_c: reads the chunk's scores, writes its keep bytes, CSR entries and row offsets.
    Reports p10 / p50 / p90 in ms, GB/s and fractions at the published peaks."""
    stream = torch.cuda.current_stream()
    for _ in range(2):
        tkt.nsa_select_planned(plan, q, k, workspace=ws, plan_dev=plan_dev)
    torch.cuda.synchronize()
    tkt.nsa_stage_timing_begin()
    for _ in range(calls):
        tkt.nsa_select_planned(plan, q, k, workspace=ws, plan_dev=plan_dev)
    recs = tkt.nsa_stage_timing_end()
    per_call = len(recs) // calls
    if per_call * calls != len(recs):
        raise RuntimeError(f"stage timing: {len(recs)} records for {calls} calls")
    names, seen = [], {}
    for name, _ in recs[:per_call]:
        n = seen.get(name, 0)
        seen[name] = n + 1
        names.append(f"{name}_{n}" if name in ("scores", "topk") else name)
    times = {nm: [recs[c * per_call + x][1] for c in range(calls)] for x, nm in enumerate(names)}

    H = sel.keep.shape[1]
    NQ, NK, D, B = w.nq, w.nk, w.D, w.B
    esz = q.element_size()
    chunk = max(1, min(H, spec.score_chunk_bytes // (NQ * NK * 4)))
    row_ptr = sel.row_ptr.cpu().numpy().astype(np.int64)
    out = {}
    for nm, xs in times.items():
        ms = float(np.median(xs))
        d = {"p10_ms": round(float(np.percentile(xs, 10)), 4), "p50_ms": round(ms, 4),
             "p90_ms": round(float(np.percentile(xs, 90)), 4)}
        flops = None
        if nm == "pool_q":
            nbytes = B * w.Hq * w.S * D * esz + B * w.Hq * NQ * D * 4
        elif nm == "pool_k":
            nbytes = B * w.Hkv * w.S * D * esz + B * w.Hkv * NK * D * 4
        elif nm == "head_mean":
            nbytes = B * (w.Hq * NQ + w.Hkv * NK + NQ + NK) * D * 4
        else:
            c = int(nm.rsplit("_", 1)[1])
            h0 = c * chunk
            nh = min(chunk, H - h0)
            cells = B * nh * NQ * NK
            if nm.startswith("scores"):
                flops = 2.0 * cells * D
                nbytes = cells * 4
            else:
                nnz = sum(int(row_ptr[(b * H + h0 + nh) * NQ] - row_ptr[(b * H + h0) * NQ]) for b in range(B))
                nbytes = cells * 4 + cells + 4 * nnz + 4 * B * nh * NQ
        gbs = nbytes / (ms * 1e-3) / 1e9
        d.update({"bytes": float(nbytes), "GBps": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)})
        if flops is not None:
            tf = flops / (ms * 1e-3) / 1e12
            d.update({"flops": flops, "TFLOPs": round(tf, 2)})
            if NQ > 64:  # split-operand bf16 products
                d.update({"executed_bf16_TFLOPs": round(6 * tf, 2),
                          "executed_frac_bf16_peak": round(6 * tf / PEAK_BF16_TFLOPS, 4)})
            else:
                d["frac_fp32_peak"] = round(tf / PEAK_FP32_TFLOPS, 4)
        out[nm] = d
    out["how"] = (f"HIP events the library records on the selection stream between its launches "
                  f"(nsa_stage_timing_begin/_end), {calls} planned selections after the timed steps; "
                  f"fractions against 8 TB/s HBM, 2.5 PFLOP/s bf16 and 157.3 TFLOP/s fp32")
    return out


def _host_us(fn, calls: int) -> float:
    """Mean host (wall) time of one call in us, with the device idle at the start."""
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(calls):
        fn()
    host = (time.perf_counter() - t) / calls * 1e6
    torch.cuda.synchronize()
    return host


def decode_timing(q, k, v, w: synth.Workload, calls: int = 20):
    """One decoding step over the workload's keys and values as a KV cache: the
    last token attends to the first S - 1 cached tokens plus itself.

    * pool update: the pooled key of the cache's last (partial) tile;
    * select: scores of the new token's query against every pooled key tile,
      per query head, with the sink tile pinned, and the top-k;
    * attention: over the kept tiles (split over workgroups, partials merged).
    Also the dense attention over the whole cache (query heads of a GQA group
    packed, so every K/V byte is read once). HBM bytes: the K and V tiles read
    (each kept tile of each query head, or the whole cache once)."""
    dev = q.device
    stream = torch.cuda.current_stream()
    L = w.S
    q1 = q[:, :, L - 1:L].contiguous()
    nk = -(-L // w.block_kv)
    pooled = torch.zeros(w.B, w.Hkv, nk, w.D, dtype=torch.float32, device=dev)
    tkt.nsa_decode_pool_update(k, 0, L - 1, w.block_kv, pooled)
    spec = tkt.SparseSpec(budget=w.budget, block_q=32, block_kv=w.block_kv, head_shared=w.head_shared)
    pins = np.zeros((1, 1, 1, nk), np.int8)
    pins[..., 0] = 1
    sws = torch.empty(1 << 24, dtype=torch.uint8, device=dev)
    aws = torch.empty(1 << 24, dtype=torch.uint8, device=dev)
    out = torch.empty_like(q1)
    lse = torch.empty(q1.shape[:3], dtype=torch.float32, device=dev)
    box = {}

    def upd():
        tkt.nsa_decode_pool_update(k, L - 1, L, w.block_kv, pooled)

    def sel():
        box["sel"] = tkt.nsa_decode_select(q1, pooled, L, L - 1, spec, pins=pins, workspace=sws)

    def att():
        tkt.nsa_decode_attn(q1, k, v, L, L - 1, box["sel"], out=out, lse=lse, workspace=aws)

    def dense():
        tkt.nsa_decode_attn(q1, k, v, L, L - 1, None, out=out, lse=lse, workspace=aws)

    log("[bench] decode step")
    for fn in (upd, sel, att, dense):
        fn()
    torch.cuda.synchronize()
    up_ms, sel_ms, att_ms, dense_ms = (_event_ms(fn, calls, stream, queued=True) for fn in (upd, sel, att, dense))
    host_us = {name: round(_host_us(fn, calls), 1) for name, fn in (("pool_update", upd), ("select", sel),
                                                                    ("attn", att))}
    nnz = int(box["sel"].nnz)
    heads_per_row = w.Hq if w.head_shared else 1
    tile_bytes = 2 * w.block_kv * w.D * q.element_size()
    att_bytes = float(nnz * heads_per_row * tile_bytes)
    dense_bytes = float(2 * w.B * w.Hkv * L * w.D * q.element_size())
    return {"cache_tokens": L, "new_tokens": 1, "kept_tiles": nnz,
            "pool_update_us": round(up_ms * 1e3, 1), "select_us": round(sel_ms * 1e3, 1),
            "attn_us": round(att_ms * 1e3, 1), "step_us": round((up_ms + sel_ms + att_ms) * 1e3, 1),
            "attn_bytes": att_bytes, "attn_GBps": round(att_bytes / (att_ms * 1e-3) / 1e9, 1),
            "attn_frac_hbm": round(att_bytes / (att_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "dense_attn_us": round(dense_ms * 1e3, 1), "dense_bytes": dense_bytes,
            "dense_GBps": round(dense_bytes / (dense_ms * 1e-3) / 1e9, 1),
            "dense_frac_hbm": round(dense_bytes / (dense_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "timing": "device time per call (calls queued behind a GPU spin); host_us: wall time per "
                      "call of the Python binding",
            "host_us": host_us,
            "kernels": "pool_kernel (tile range), score_rows_kernel, topk_rows_kernel, attn_decode_kernel<128> + "
                       "attn_combine_kernel"}


def reorder_timing(q, w: synth.Workload, calls: int = 10):
    """Hilbert order of a 256 x 512 token grid (host), then the row gather of q
    along it and the scatter back on the GPU; HBM bytes = one read and one write of q."""
    dev = q.device
    stream = torch.cuda.current_stream()
    rows = 256
    cols = w.S // rows
    t0 = time.perf_counter()
    perm = torch.from_numpy(tkt.nsa_curve_order(tkt.NSA_CURVE_HILBERT, (rows, cols))).to(dev)
    host_ms = (time.perf_counter() - t0) * 1e3
    y = torch.empty_like(q)
    z = torch.empty_like(q)
    tkt.nsa_permute_tokens(q, perm, out=y)
    tkt.nsa_permute_tokens(y, perm, inverse=True, out=z)
    torch.cuda.synchronize()
    if not torch.equal(z, q):
        raise RuntimeError("token reordering did not round-trip")
    g_ms = _event_ms(lambda: tkt.nsa_permute_tokens(q, perm, out=y), calls, stream)
    s_ms = _event_ms(lambda: tkt.nsa_permute_tokens(y, perm, inverse=True, out=z), calls, stream)
    nbytes = float(2 * q.numel() * q.element_size())
    return {"grid": [rows, cols], "curve": "hilbert", "order_host_ms": round(host_ms, 2),
            "gather_us": round(g_ms * 1e3, 1), "scatter_us": round(s_ms * 1e3, 1), "bytes": nbytes,
            "gather_GBps": round(nbytes / (g_ms * 1e-3) / 1e9, 1),
            "gather_frac_hbm": round(nbytes / (g_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "scatter_GBps": round(nbytes / (s_ms * 1e-3) / 1e9, 1), "kernel": "permute_rows_kernel<16>"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the separate timing of the attention gradients")
    ap.add_argument("--backward-steps", type=int, default=5)
    ap.add_argument("--no-decode", action="store_true", help="skip the decoding-step timing")
    ap.add_argument("--no-reorder", action="store_true", help="skip the token-reordering timing")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured reference rates (a large bf16 GEMM and a device copy)")
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB read + 1 GiB write elementwise kernel 3 times "
                         "(reference for HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        x = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")  # 1 GiB
        y = torch.empty_like(x)
        for _ in range(3):
            torch.neg(x, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": x.numel() * 4, "bytes_written": y.numel() * 4}))
        return

    w = synth.workload(args.workload)
    log(f"[bench] generating {w.name}")
    t0 = time.perf_counter()
    inp = synth.make_inputs(w)
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s; uploading")
    dev = torch.device("cuda:0")
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    spec = tkt.SparseSpec(budget=w.budget, block_q=w.block_q, block_kv=w.block_kv, head_shared=w.head_shared)
    # The plan depends on geometry, spec and masks only: built once and kept on
    # the device, as the selection page caches it across the steps of a run.
    plan = tkt.nsa_plan_create(q, k, spec, inp.pins, inp.drops)
    plan_dev = plan.upload(dev)
    sizes = plan.sizes()
    ws = torch.empty(sizes.workspace_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        sel = tkt.nsa_select_planned(plan, q, k, workspace=ws, plan_dev=plan_dev)
        if ev is not None:
            ev[1].record(stream)
        tkt.nsa_block_sparse_attn(q, k, v, sel, w.causal, out=out, lse=lse)
        if ev is not None:
            ev[2].record(stream)
        return sel

    log("[bench] warmup")
    for _ in range(args.warmup):
        sel = step()
    torch.cuda.synchronize()
    full_flops, vis_flops, tiles = kept_tile_flops(sel, w)

    log(f"[bench] timing {args.steps} steps")
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    sel_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    attn_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    pct = lambda xs: {f"p{p}": round(float(np.percentile(xs, p)), 4) for p in (10, 50, 90)}  # noqa: E731
    step_pct = pct([e[0].elapsed_time(e[2]) for e in events])
    attn_pct = pct([e[1].elapsed_time(e[2]) for e in events])

    value = full_flops / (ms_step * 1e-3) / 1e12
    kv_bytes = float(tiles * 2 * w.block_kv * w.D * 2 + 2 * q.numel() * q.element_size())
    attn_tflops = full_flops / (attn_ms * 1e-3) / 1e12
    select_bytes = (q.numel() + k.numel()) * q.element_size() + sel.keep.numel() + 4 * (sel.nnz + sel.row_ptr.numel())
    select_bytes += (2 * w.nq * ((w.nk + 63) // 64) * 8)  # bit-packed pins + drops
    select_gbs = select_bytes / (sel_ms * 1e-3) / 1e9
    traffic = read_traffic()

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "S": w.S, "D": w.D,
                   "block_q": w.block_q, "block_kv": w.block_kv, "budget": w.budget, "causal": w.causal,
                   "head_shared": w.head_shared, "sink_pin": w.sink_pin, "drop_frac": w.drop_frac,
                   "nnz_tiles": sel.nnz, "kept_tiles_visited": tiles},
        "roofline": {"bound": "mfma", "kernel": "attn_mfma_kernel<128,4>",
                     "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "flops_per_launch": full_flops, "visible_pair_flops_per_launch": vis_flops,
                     "avg_launch_ms": round(attn_ms, 4),
                     # K/V supply: every kept, live tile visit reads one 64-key K tile and
                     # one V tile (32 KiB at D = 128) unless L2 still holds it; plus Q read
                     # and O written once.
                     "kv_visit_bytes_per_launch": kv_bytes,
                     "kv_visit_GBps": round(kv_bytes / (attn_ms * 1e-3) / 1e9, 1),
                     "kv_visit_frac_hbm": round(kv_bytes / (attn_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "stages": {"select_ms": round(sel_ms, 4), "select_GBps": round(select_gbs, 1),
                   "select_frac_hbm": round(select_gbs / PEAK_HBM_GBS, 4),
                   "select_algorithmic_bytes": select_bytes, "attn_ms": round(attn_ms, 4),
                   "attn_TFLOPs": round(attn_tflops, 2),
                   "step_ms_events": step_pct, "attn_ms_events": attn_pct},
    }
    log("[bench] per-stage selection timing")
    res["stages"]["select_stages"] = stage_timing(plan, plan_dev, q, k, ws, sel, w, spec)
    if not args.no_peaks:
        peaks = measured_peaks()
        res["measured_peaks"] = peaks
        res["roofline"]["frac_of_measured_gemm"] = round(attn_tflops / peaks["bf16_gemm_TFLOPs"], 4)
    if not args.no_backward:
        res["backward"] = backward_timing(q, k, v, out, lse, sel, w, full_flops, args.backward_steps)
    if not args.no_decode:
        res["decode"] = decode_timing(q, k, v, w)
    if not args.no_reorder:
        log("[bench] token reordering")
        res["reorder"] = reorder_timing(q, w)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on a bounded sample)")
        res["cpu_baseline"] = cpu_baseline(inp, w, full_flops)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
