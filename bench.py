#!/usr/bin/env python3
"""Benchmark: MLA decode over a latent cache on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--split-tokens T | --units N] [--fused]

A step is one pass of the whole decode hot path over one batch of synthetic
DeepSeek-V3-shaped input already resident in HBM:
    mla_absorb_query -> mla_decode_partial_balanced -> mla_combine_balanced -> mla_out_proj
by default (work-balanced split over the compute units), or with --split-tokens T
the fixed-chunk pair mla_decode_partial -> mla_combine.  --fused runs the split-K merge and
the value projection as one call (mla_combine_out_proj_balanced / mla_combine_out_proj).
W untimed warm-up steps, then exactly K timed steps bracketed by device
synchronisation.  Prints one JSON line.

value = cache GB/s = (sum over sequences of cached tokens x 1,152 B) / time per step.
The roofline object covers the dominant kernel (the split-K decode): its
algorithmic bytes per launch over its average duration, timed with HIP events
on the stream it runs on.  cpu_baseline times the fp64 oracle on a bounded
sample of the same workload on the host cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
DEFAULT_WORKLOAD = "v3_b64_ragged_paged"
DECODE_SOURCES = ("mla_latent_kv_31_amd/csrc/decode_mfma.hip", "mla_latent_kv_31_amd/csrc/schedule.h",
                  "mla_latent_kv_31_amd/csrc/common.h")


def _kernel_sha() -> str:
    """Hash of the decode kernel's sources with comments and blank space removed, so that stored
    counter results stay tied to the code they measured and nothing else."""
    import re

    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        p = os.path.join(ROOT, rel)
        if os.path.exists(p):
            text = open(p, encoding="utf-8").read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            text = re.sub(r"//[^\n]*", "", text)
            h.update(re.sub(r"\s+", " ", text).strip().encode())
    return h.hexdigest()[:16]


def _traffic(workload: str, sha: str):
    """HBM bytes per decode launch from committed rocprofv3 counter runs, if they match the source."""
    p = os.path.join(ROOT, "profiles", f"decode_traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:  # noqa: BLE001 - informational only
        pass
    return len(os.sched_getaffinity(0))


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo", encoding="utf-8"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measured_copy_gbs(dev, mib: int = 1024, min_ms: float = 150.0) -> dict:
    """HBM bandwidth of a plain device-to-device copy (bytes read + bytes written per second), the
    achievable denominator beside the published peak; the buffers exceed the 256 MB Infinity Cache
    several times over.  Copies run back to back for at least `min_ms` of GPU time and the median
    copy is reported.  From idle the board needs a few tens of milliseconds of load before its
    clocks reach their sustained level, so this probe also leaves them settled for whatever runs
    next."""
    import statistics

    import torch

    src = torch.ones(mib << 18, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    times, total = [], 0.0
    while total < min_ms and len(times) < 4000:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(32)]
        for a, b in ev:
            a.record(stream)
            dst.copy_(src)
            b.record(stream)
        torch.cuda.synchronize()
        t = [a.elapsed_time(b) for a, b in ev]
        times += t
        total += sum(t)
    del src, dst
    ms = statistics.median(times)
    return {"gbs": round(2 * (mib << 20) / (ms * 1e-3) / 1e9, 1), "copies": len(times), "gpu_ms": round(total, 1)}


def cpu_baseline(inp: dict, seconds: float) -> dict:
    """The fp64 oracle, as it stands, on whole sequences of the same workload until `seconds` pass."""
    import numpy as np

    import oracle.mla_oracle as O
    from mla_workloads import gen

    w = inp["workload"]
    dt = inp["dtype"]
    w_uk = gen.as_f64(inp["w_uk"], dt)
    w_uv = gen.as_f64(inp["w_uv"], dt)
    toks, n = 0, 0
    t0 = time.perf_counter()
    for b in range(w.batch):
        L = int(inp["lens"][b])
        cache = gen.as_f64(O.gather_rows(inp["pool"], inp["page_table"], b, L), dt)
        O.attention(gen.as_f64(inp["q_c"][b], dt), gen.as_f64(inp["q_r"][b], dt), L - 1, cache, w_uk, w_uv,
                    w.d_c, base=w.rope_base)
        toks += L
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    row_bytes = (w.d_c + w.d_r) * (2 if dt == "bf16" else 4)
    return {"value": round(toks * row_bytes / el / 1e9, 6), "unit": "GB/s", "cores": _blas_threads(),
            "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": f"first {n} of {w.batch} sequences ({toks} cached tokens, all {w.n_heads} heads, "
                      f"unabsorbed fp64 NumPy) in {el:.1f} s"}


def cpu_baseline_prefill(inp: dict, seconds: float, unabsorbed: bool = False) -> dict:
    """The fp64 oracle on prefill rows of the same workload until `seconds` pass (algorithmic flops/s:
    2,176 per visible (query head, key) pair for the absorbed path, 640 for the unabsorbed one)."""
    import oracle.mla_oracle as O
    from mla_workloads import gen

    w = inp["workload"]
    dt = inp["dtype"]
    w_uk = gen.as_f64(inp["w_uk"], dt)
    w_uv = gen.as_f64(inp["w_uv"], dt)
    flops, n = 0, 0
    t0 = time.perf_counter()
    b = 0
    cache = gen.as_f64(O.gather_rows(inp["pool"], inp["page_table"], b, int(inp["lens"][b])), dt)
    for i in range(w.q_len):
        p = int(inp["q_start"][b]) + i
        O.attention(gen.as_f64(inp["q_c"][b, i], dt), gen.as_f64(inp["q_r"][b, i], dt), p, cache[:p + 1], w_uk, w_uv,
                    w.d_c, base=w.rope_base)
        per_pair = 2 * (w.d_k + w.d_r) + 2 * w.d_v if unabsorbed else 2 * (w.d_c + w.d_r) + 2 * w.d_c
        flops += (p + 1) * w.n_heads * per_pair
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    return {"value": round(flops / el / 1e12, 9), "unit": "TFLOP/s", "cores": _blas_threads(), "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"first {n} of {w.q_len} query rows of sequence 0 (all {w.n_heads} heads, unabsorbed fp64 "
                      f"NumPy; algorithmic {'unabsorbed attention' if unabsorbed else 'absorbed'} flops counted) "
                      f"in {el:.1f} s"}


def cpu_baseline_fp8(inp: dict, seconds: float) -> dict:
    """The fp64 oracle on the FP8 cache of the same batch, whole sequences until `seconds` pass:
    its own E4M3 quantisation of each sequence's latents, their dequantisation, then attention
    (GB/s of 656-byte FP8 rows)."""
    import numpy as np

    import oracle.mla_oracle as O
    from mla_workloads import gen

    w = inp["workload"]
    dt = inp["dtype"]
    w_uk = gen.as_f64(inp["w_uk"], dt)
    w_uv = gen.as_f64(inp["w_uv"], dt)
    toks, n = 0, 0
    t0 = time.perf_counter()
    for b in range(w.batch):
        L = int(inp["lens"][b])
        rows = O.gather_rows(inp["pool"], inp["page_table"], b, L)
        codes, scale = O.quantize_latents_fp8(gen.as_f64(rows[:, :w.d_c], dt))
        cache = np.concatenate([O.dequantize_latents_fp8(codes, scale), gen.as_f64(rows[:, w.d_c:], dt)], axis=1)
        O.attention(gen.as_f64(inp["q_c"][b], dt), gen.as_f64(inp["q_r"][b], dt), L - 1, cache, w_uk, w_uv,
                    w.d_c, base=w.rope_base)
        toks += L
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    return {"value": round(toks * O.FP8_ROW_BYTES / el / 1e9, 6), "unit": "GB/s", "cores": _blas_threads(),
            "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": f"first {n} of {w.batch} sequences ({toks} cached tokens as {O.FP8_ROW_BYTES}-byte FP8 rows, "
                      f"quantised and dequantised by the oracle, all {w.n_heads} heads, unabsorbed fp64 NumPy) "
                      f"in {el:.1f} s"}


def cpu_baseline_verify(inp: dict, seconds: float) -> dict:
    """The fp64 oracle on the draft rows of the same verify batch until `seconds` pass: row (b, i)
    attends over keys t <= q_start[b] + i, t < len[b] (draft tokens per second)."""
    import oracle.mla_oracle as O
    from mla_workloads import gen

    w = inp["workload"]
    dt = inp["dtype"]
    w_uk = gen.as_f64(inp["w_uk"], dt)
    w_uv = gen.as_f64(inp["w_uv"], dt)
    n = 0
    t0 = time.perf_counter()
    done = False
    for b in range(w.batch):
        L = int(inp["lens"][b])
        cache = gen.as_f64(O.gather_rows(inp["pool"], inp["page_table"], b, L), dt)
        for i in range(w.q_len):
            p = int(inp["q_start"][b]) + i
            keys = min(p + 1, L)
            if keys > 0:
                O.attention(gen.as_f64(inp["q_c"][b, i], dt), gen.as_f64(inp["q_r"][b, i], dt), p, cache[:keys],
                            w_uk, w_uv, w.d_c, base=w.rope_base)
            n += 1
            if time.perf_counter() - t0 >= seconds:
                done = True
                break
        if done:
            break
    el = time.perf_counter() - t0
    return {"value": round(n / el, 4), "unit": "tokens/s", "cores": _blas_threads(), "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"first {n} of {w.batch * w.q_len} draft rows (all {w.n_heads} heads, unabsorbed fp64 NumPy) "
                      f"in {el:.1f} s"}


def cpu_baseline_precomposed(inp: dict, seconds: float) -> dict:
    """The fp64 oracle's two per-step precomposed products on a sample of the same rows, scaled to
    all rows (ms per step).  The precomposition itself, an offline step, is done first and not
    timed."""
    import oracle.mla_oracle as O
    from mla_workloads import gen

    w = inp["workload"]
    dt = w.dtype
    R = int(inp["c_q"].shape[0])
    wa = O.precompose_query_weights(gen.as_f64(inp["w_uq"], dt), gen.as_f64(inp["w_uk"], dt))
    w_uvo = O.precompose_out_weights(gen.as_f64(inp["w_uv"], dt), gen.as_f64(inp["w_o"], dt))
    w_qr = gen.as_f64(inp["w_qr"], dt)
    nq = 0
    t0 = time.perf_counter()
    while nq < R:
        O.absorbed_query_precomposed(gen.as_f64(inp["c_q"][nq], dt), wa, w_qr, int(inp["pos"][nq]), base=w.rope_base)
        nq += 1
        if time.perf_counter() - t0 >= seconds / 2:
            break
    tq = (time.perf_counter() - t0) / nq
    no = 0
    t0 = time.perf_counter()
    while no < R:
        O.out_proj_fused(inp["z"][no:no + 1].astype("float64"), w_uvo)
        no += 1
        if time.perf_counter() - t0 >= seconds / 2:
            break
    to = (time.perf_counter() - t0) / no
    return {"value": round((tq + to) * R * 1e3, 3), "unit": "ms", "cores": _blas_threads(), "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"fused query on {nq} and fused output on {no} of {R} rows (fp64 NumPy, precomposition "
                      f"untimed), scaled to {R} rows"}


def bench_prefill_unabsorbed(args, w) -> dict:
    """Chunked prefill the unabsorbed way: mla_decompress_kv -> mla_prefill_unabsorbed per step.
    Same inputs and outputs as bench_prefill; its own algorithmic flops (decompression of every
    cached latent per head, then 2 * (d_k + d_r) + 2 * d_v per visible pair)."""
    import numpy as np
    import torch

    from mla_latent_kv_31_amd import runner
    from mla_workloads import gen

    inp = gen.make_prefill_inputs(w)
    dev = torch.device("cuda:0")
    st = runner.PrefillUnabsorbedStep(inp, dev)
    if not st.supported():
        raise SystemExit(f"the unabsorbed prefill does not support workload {w.name}")
    pairs = int(sum(min(int(inp["lens"][b]), int(inp["q_start"][b]) + i + 1)
                    for b in range(w.batch) for i in range(w.q_len)))
    flops_attn = pairs * w.n_heads * (2 * (w.d_k + w.d_r) + 2 * w.d_v)
    flops_dec = int(np.sum(inp["lens"])) * w.n_heads * 2 * w.d_c * (w.d_k + w.d_v)
    for _ in range(args.warmup):
        st.run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        st.decompress()
        ev[i][0].record(stream)
        st.attend()
        ev[i][1].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    ms_attn = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    tf_attn = flops_attn / (ms_attn * 1e-3) / 1e12
    return {
        "metric": "MLA chunked-prefill TFLOP/s, unabsorbed path (V3 shape, 1 GPU)",
        "value": round((flops_attn + flops_dec) / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "prior_tokens": w.ctx, "chunk": w.q_len,
                   "heads": w.n_heads, "d_c": w.d_c, "d_r": w.d_r, "causal_pairs": pairs, "seed": w.seed,
                   "path": "unabsorbed (decompress + attend)"},
        "query_tokens_per_s": round(w.batch * w.q_len / (ms_step * 1e-3), 1),
        "roofline": {"bound": "mfma", "kernel": "mla_prefill_unabsorbed", "achieved": round(tf_attn, 3),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf_attn / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "ms_per_launch": round(ms_attn, 6), "algorithmic_flops_per_launch": flops_attn},
        "decompress": {"ms_per_launch": round(ms_step - ms_attn, 6), "algorithmic_flops_per_launch": flops_dec,
                       "tflops": round(flops_dec / ((ms_step - ms_attn) * 1e-3) / 1e12, 3)},
    } | ({} if args.no_cpu_baseline else {"cpu_baseline": cpu_baseline_prefill(inp, args.cpu_seconds, True)})


def bench_prefill(args, w) -> dict:
    """Chunked prefill: absorb -> mla_prefill_chunk -> out_proj per step; MFMA-bound."""
    import numpy as np
    import torch

    from mla_latent_kv_31_amd import runner
    from mla_workloads import gen

    inp = gen.make_prefill_inputs(w)
    dev = torch.device("cuda:0")
    st = runner.PrefillStep(inp, dev)
    pairs = int(sum(min(int(inp["lens"][b]), int(inp["q_start"][b]) + i + 1)
                    for b in range(w.batch) for i in range(w.q_len)))
    flops_attn = pairs * w.n_heads * (2 * (w.d_c + w.d_r) + 2 * w.d_c)
    flops_proj = w.batch * w.q_len * 2 * w.n_heads * w.d_c * (w.d_k + w.d_v)
    for _ in range(args.warmup):
        st.run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        st.absorb()
        ev[i][0].record(stream)
        st.attend()
        ev[i][1].record(stream)
        st.out_proj()
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    ms_attn = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    tf_attn = flops_attn / (ms_attn * 1e-3) / 1e12
    rec = {
        "metric": "MLA chunked-prefill TFLOP/s (V3 shape, 1 GPU)",
        "value": round((flops_attn + flops_proj) / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "prior_tokens": w.ctx, "chunk": w.q_len,
                   "heads": w.n_heads, "d_c": w.d_c, "d_r": w.d_r, "causal_pairs": pairs, "seed": w.seed,
                   "prefill_kernel": "mfma" if st.uses_mfma() else "generic"},
        "query_tokens_per_s": round(w.batch * w.q_len / (ms_step * 1e-3), 1),
        "roofline": {"bound": "mfma", "kernel": "mla_prefill_chunk", "achieved": round(tf_attn, 3),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf_attn / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "ms_per_launch": round(ms_attn, 6), "algorithmic_flops_per_launch": flops_attn},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_prefill(inp, args.cpu_seconds)
    return rec


def bench_verify(args, w) -> dict:
    """Multi-token verify: q_len draft tokens per sequence of a ragged decode batch, each a decode
    row over its own prefix.  Step: mla_verify_rows -> absorb -> balanced decode with the draft
    rows of a sequence as one row group (mla_decode_partial_grouped) -> combine -> out_proj.  The
    same rows on the plain balanced split, and the same inputs through mla_prefill_chunk (one
    workgroup per query row), are timed beside it for comparison."""
    import numpy as np
    import torch

    from mla_latent_kv_31_amd import runner
    from mla_workloads import gen

    inp = gen.make_prefill_inputs(w)
    dev = torch.device("cuda:0")
    rows = w.batch * w.q_len
    qs = inp["q_start"].astype(np.int64)
    row_lens = np.minimum(np.maximum(qs[:, None] + np.arange(w.q_len)[None, :] + 1, 0),
                          inp["lens"].astype(np.int64)[:, None])
    row_bytes = (w.d_c + w.d_r) * 2
    read_bytes = int(row_lens.sum()) * row_bytes          # every row reads its own prefix
    unique_bytes = int(inp["lens"].astype(np.int64).sum()) * row_bytes
    n_units = args.units or runner.balanced_units(row_lens.reshape(-1), runner.compute_units(dev))
    st = runner.VerifyStep(inp, dev, n_units=n_units)
    for _ in range(args.warmup):
        st.run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        st.rows()
        st.absorb()
        ev[i][0].record(stream)
        st.attend()
        ev[i][1].record(stream)
        st.combine()
        st.out_proj()
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    ms_dec = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    ms_dec_plain = ms_pf = None
    if not args.no_compare:
        ms_dec_plain, ms_pf = _verify_comparisons(args, inp, dev, n_units, stream)
    achieved = read_bytes / (ms_dec * 1e-3) / 1e9
    flops = int(row_lens.sum()) * w.n_heads * (2 * (w.d_c + w.d_r) + 2 * w.d_c)
    return {
        "metric": "MLA multi-token verify draft tokens/s (V3 shape, 1 GPU)",
        "value": round(rows / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "draft_tokens": w.q_len, "heads": w.n_heads,
                   "d_c": w.d_c, "d_r": w.d_r, "rows": rows,
                   "split": f"balanced {st.n_units} units, row groups of {st.group}",
                   "unique_cache_bytes": unique_bytes, "seed": w.seed},
        "roofline": {"bound": "hbm", "kernel": "mla_decode_partial_grouped (verify rows)",
                     "achieved": round(achieved, 3), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": _traffic(w.name, _kernel_sha()),
                     "ms_per_launch": round(ms_dec, 6), "algorithmic_bytes_per_launch": read_bytes,
                     "unique_bytes_per_launch": unique_bytes,
                     "unique_gbs": round(unique_bytes / (ms_dec * 1e-3) / 1e9, 3),
                     "note": "every draft row reads its own prefix (algorithmic bytes); the rows of one "
                             "sequence run side by side on one XCD, so repeats are served by its L2"},
        "plain_balanced_ms_per_launch": None if ms_dec_plain is None else round(ms_dec_plain, 6),
        "roofline_mfma": {"achieved": round(flops / (ms_dec * 1e-3) / 1e12, 3), "peak": MFMA_BF16_PEAK_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(flops / (ms_dec * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
        "prefill_chunk_ms_per_step": None if ms_pf is None else round(ms_pf, 6),
    } | ({} if args.no_cpu_baseline else {"cpu_baseline": cpu_baseline_verify(inp, args.cpu_seconds)})


def _verify_comparisons(args, inp, dev, n_units, stream):
    """Decode-launch ms of the same verify rows on the plain balanced split (each draft row
    scheduled on its own) and step ms of the same inputs through mla_prefill_chunk."""
    import numpy as np
    import torch

    from mla_latent_kv_31_amd import runner

    sp = runner.VerifyStep(inp, dev, n_units=n_units, grouped=False)
    n_sp = max(5, args.steps // 10)
    for _ in range(3):
        sp.run()
    torch.cuda.synchronize()
    ev_sp = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_sp)]
    for a, b in ev_sp:
        sp.rows()
        sp.absorb()
        a.record(stream)
        sp.attend()
        b.record(stream)
        sp.combine()
        sp.out_proj()
    torch.cuda.synchronize()
    ms_dec_plain = float(np.mean([a.elapsed_time(b) for a, b in ev_sp]))
    del sp
    # the same verify through mla_prefill_chunk, for comparison
    pf = runner.PrefillStep(inp, dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_pf = max(5, args.steps // 10)
    for _ in range(3):
        pf.run()
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(n_pf):
        pf.run()
    stop.record(stream)
    torch.cuda.synchronize()
    ms_pf = start.elapsed_time(stop) / n_pf
    return ms_dec_plain, ms_pf


def bench_precomposed(args, w) -> dict:
    """Precomposed weights on one decode step's query rows: the fused query product (c^Q . w_qcat
    + epilogue) and the fused output product (z . W_UV W_O), each against the library's unfused
    counterpart on the same rows (mla_absorb_query from q_C; mla_out_proj then
    mla_output_projection).  Both fused products read their precomposed weights once per step."""
    import numpy as np
    import torch

    from mla_latent_kv_31_amd import _lib as L
    from mla_latent_kv_31_amd import runner
    from mla_workloads import gen

    dev = torch.device("cuda:0")
    inp = gen.make_precomposed_inputs(w)
    R, H, dq, dc, dr, dk, dv, dm = w.batch, w.n_heads, w.d_cq, w.d_c, w.d_r, w.d_k, w.d_v, w.d_model
    d = runner.dims_for(w)
    t = {k: runner.to_device(inp[k], dev) for k in ("w_uq", "w_qr", "w_uk", "w_uv", "w_o", "c_q", "z", "o", "pos")}
    w_qcat = torch.empty((dq, H, dc + dr), dtype=torch.bfloat16, device=dev)
    w_uvo = torch.empty((H, dc, dm), dtype=torch.bfloat16, device=dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    ev0.record(stream)
    L.mla_precompose_query(d, dq, t["w_uq"], t["w_uk"], t["w_qr"], w_qcat)
    L.mla_precompose_out(d, dm, t["w_uv"], t["w_o"], w_uvo)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_precompose = ev0.elapsed_time(ev1)
    wsq = L.mla_absorb_query_precomposed_workspace_bytes(d, dq, R)
    wso = L.mla_out_proj_fused_workspace_bytes(d, dm, R)
    wsp = L.mla_output_projection_workspace_bytes(d, dm, R)
    ws = torch.empty(max(wsq, wso, wsp) // 4, dtype=torch.float32, device=dev)
    q_hat = torch.empty((R, H, dc + dr), dtype=torch.float16, device=dev)
    out = torch.empty((R, dm), dtype=torch.float32, device=dev)
    q_c = torch.randn((R, H, dk), device=dev).to(torch.bfloat16)
    q_r = torch.randn((R, H, dr), device=dev).to(torch.bfloat16)
    o_h = torch.empty((R, H, dv), dtype=torch.float32, device=dev)
    ops = {
        "fused_query": lambda: L.mla_absorb_query_precomposed(d, dq, t["c_q"], w_qcat, t["pos"], R, q_hat, ws, wsq),
        "fused_output": lambda: L.mla_out_proj_fused(d, dm, t["z"], w_uvo, R, out, ws, wso),
        "absorb_query": lambda: L.mla_absorb_query(d, q_c, q_r, t["w_uk"], t["pos"], R, q_hat),
        "out_proj": lambda: L.mla_out_proj(d, t["z"], t["w_uv"], R, o_h),
        "output_projection": lambda: L.mla_output_projection(d, dm, t["o"], t["w_o"], R, out, ws, wsp),
    }
    ms = {}
    for name, fn in ops.items():
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            fn()
        ev1.record(stream)
        torch.cuda.synchronize()
        ms[name] = ev0.elapsed_time(ev1) / args.steps
    ms_fused = ms["fused_query"] + ms["fused_output"]
    ms_unfused = ms["absorb_query"] + ms["out_proj"] + ms["output_projection"]
    bytes_fused_out = H * dc * dm * 2 + R * H * dc * 4 + R * dm * 4
    ach = bytes_fused_out / (ms["fused_output"] * 1e-3) / 1e9
    return {
        "metric": "MLA precomposed-weight products, ms per decode step (V3 shape, 1 GPU)",
        "value": round(ms_fused, 6), "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_fused, 6), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "rows": R, "heads": H, "d_cq": dq, "d_c": dc, "d_r": dr, "d_model": dm,
                   "seed": w.seed},
        "ms": {k: round(v, 6) for k, v in ms.items()},
        "unfused_ms_per_step": round(ms_unfused, 6),
        "unfused_note": "absorb_query starts from q_C (the c^Q . W_UQ product before it is upstream of the path)",
        "weight_bytes": {"w_qcat": dq * H * (dc + dr) * 2, "w_uvo": H * dc * dm * 2, "w_uk": H * dc * dk * 2,
                         "w_uv": H * dc * dv * 2, "w_o": H * dv * dm * 2},
        "precompose_ms_once": round(ms_precompose, 3),
        "roofline": {"bound": "hbm", "kernel": "mla_out_proj_fused", "achieved": round(ach, 3), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                     "ms_per_launch": round(ms["fused_output"], 6), "algorithmic_bytes_per_launch": bytes_fused_out},
    } | ({} if args.no_cpu_baseline else {"cpu_baseline": cpu_baseline_precomposed(inp, args.cpu_seconds)})


def cpu_baseline_kv_append(inp: dict, seconds: float) -> dict:
    """The fp64 oracle's cache-write steps on rows of the same workload until `seconds` pass."""
    import oracle.mla_oracle as O
    from mla_workloads import gen

    w = inp["workload"]
    dt = inp["dtype"]
    w_dkv, w_kr = gen.as_f64(inp["w_dkv"], dt), gen.as_f64(inp["w_kr"], dt)
    n = 0
    t0 = time.perf_counter()
    while n < inp["h"].shape[0]:
        h = gen.as_f64(inp["h"][n:n + 1], dt)
        O.cache_rows(O.rms_normalize(O.kv_latent(h, w_dkv), gen.RMS_EPS),
                     O.rope_key(h, w_kr, inp["positions"][n:n + 1], w.rope_base))
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    nbytes = _kv_append_bytes(w, n)
    return {"value": round(nbytes / el / 1e9, 6), "unit": "GB/s", "cores": _blas_threads(), "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"first {n} of {inp['h'].shape[0]} new rows (fp64 NumPy; algorithmic bytes counted) "
                      f"in {el:.1f} s"}


def _kv_append_bytes(w, rows: int) -> int:
    """Algorithmic HBM bytes of one cache write: both weight matrices, the new hidden states, the
    written rows (bf16) and the row addresses."""
    return 2 * w.d_model * (w.d_c + w.d_r) + 2 * rows * w.d_model + rows * 2 * (w.d_c + w.d_r) + 8 * rows


def bench_kv_append(args, w) -> dict:
    """Cache write of new tokens: mla_kv_append per step (weight-read bound at decode batch)."""
    import numpy as np
    import torch

    import mla_latent_kv_31_amd as M
    from mla_latent_kv_31_amd import runner
    from mla_workloads import gen

    inp = gen.make_kv_append_inputs(w)
    dev = torch.device("cuda:0")
    to = lambda a: runner.to_device(a, dev)  # noqa: E731
    R = inp["h"].shape[0]
    d = runner.dims_for(w)
    pool, table = to(inp["pool"]), to(inp["page_table"])
    c = M.cache(pool, table, to(np.zeros(w.batch, np.int32)))
    h, w_dkv, w_kr = to(inp["h"]), to(inp["w_dkv"]), to(inp["w_kr"])
    seq, pos = to(inp["seq_ids"]), to(inp["positions"])
    ws_bytes = M.mla_kv_append_workspace_bytes(d, w.d_model, R)
    ws = torch.empty(max(ws_bytes // 4, 4), dtype=torch.float32, device=dev)

    def step():
        M.mla_kv_append(d, c, w.d_model, h, w_dkv, w_kr, seq, pos, R, gen.RMS_EPS, ws, ws_bytes)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    nbytes = _kv_append_bytes(w, R)
    gbs = nbytes / (ms * 1e-3) / 1e9
    rec = {
        "metric": "MLA cache-write GB/s (V3 shape, 1 GPU)",
        "value": round(gbs, 3), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "rows": R, "d_model": w.d_model, "d_c": w.d_c, "d_r": w.d_r,
                   "page_size": w.page_size, "seed": w.seed, "workspace_bytes": ws_bytes,
                   "kv_append_kernel": "mfma" if ws_bytes > 0 else "generic"},
        "rows_per_s": round(R / (ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "kernel": "mla_kv_append (both launches)", "achieved": round(gbs, 3),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "ms_per_launch": round(ms, 6), "algorithmic_bytes_per_launch": nbytes},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_kv_append(inp, min(args.cpu_seconds, 5.0))
    return rec


COPY_PROBE_KERNEL = "neg_kernel"  # the calibration copy: torch.neg over a float32 buffer (1 read, 1 write)


def traffic_from_counters(workload: str, fetch_csv: str, write_csv: str, copy_mb: int) -> dict:
    """HBM bytes per decode launch from two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
    WRITE_SIZE, both in KiB per dispatch), each scaled by what the same counter reads for the plain
    copy of --copy-probe-mb MiB that the profiled runs launched first."""
    import csv
    import statistics

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        return vals

    out = {"workload": workload, "kernel_source_sha": _kernel_sha(), "copy_probe_bytes": copy_mb << 20}
    for counter, path, tag in (("FETCH_SIZE", fetch_csv, "read"), ("WRITE_SIZE", write_csv, "write")):
        v = per_kernel(path, counter)
        copy = [x for (k, _), x in v.items() if COPY_PROBE_KERNEL in k]
        dec = [x for (k, _), x in v.items() if "decode_mfma" in k]
        if not copy or not dec:
            raise SystemExit(f"{path}: copy probe or decode kernel missing")
        factor = (copy_mb << 20) / (max(copy) * 1024.0)  # the probe moves copy_mb MiB each way
        out[f"{tag}_factor"] = round(factor, 4)
        out[f"{tag}_bytes_per_launch"] = round(statistics.median(dec) * 1024.0 * factor)
    out["hbm_bytes_per_launch"] = out["read_bytes_per_launch"] + out["write_bytes_per_launch"]
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    # The warm-up runs long enough (~0.1 s) for the clocks to settle at their sustained level
    # under the board power limit; shorter runs time a ramping clock.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--split-tokens", type=int, default=None,
                    help="fixed split-K chunks of this many tokens instead of the balanced split")
    ap.add_argument("--units", type=int, default=None, help="units of the balanced split (default: one per CU)")
    ap.add_argument("--fused", action="store_true",
                    help="decode step with the fused merge + value projection instead of mla_combine* then mla_out_proj")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="launch one plain device copy of this many MiB first (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                    help="write profiles/decode_traffic_<workload>.json from two rocprofv3 --pmc runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true",
                    help="verify workloads: skip the plain-split and prefill comparisons (counter runs)")
    ap.add_argument("--fp8", action="store_true",
                    help="decode workloads: FP8 latent cache (the bf16 pool quantised on the GPU first)")
    ap.add_argument("--unabsorbed", action="store_true",
                    help="prefill workloads: time the unabsorbed path (decompress + attend) instead")
    args = ap.parse_args()

    if args.traffic_from:
        rec = traffic_from_counters(args.workload, args.traffic_from[0], args.traffic_from[1], args.copy_probe_mb)
        with open(os.path.join(ROOT, "profiles", f"decode_traffic_{args.workload}.json"), "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from mla_latent_kv_31_amd import _lib as L
    from mla_latent_kv_31_amd import runner
    from mla_workloads import gen

    w = gen.WORKLOADS[args.workload]
    if args.copy_probe_mb:  # a plain streaming copy of known size, for counter calibration
        src = torch.empty(args.copy_probe_mb << 18, dtype=torch.float32, device=torch.device("cuda:0"))
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if w.kind == "prefill":
        print(json.dumps(bench_prefill_unabsorbed(args, w) if args.unabsorbed else bench_prefill(args, w)), flush=True)
        return 0
    if w.kind == "kv_append":
        print(json.dumps(bench_kv_append(args, w)), flush=True)
        return 0
    if w.kind == "verify":
        print(json.dumps(bench_verify(args, w)), flush=True)
        return 0
    if w.kind == "precomposed":
        print(json.dumps(bench_precomposed(args, w)), flush=True)
        return 0
    if w.kind != "decode":
        print(f"workload {w.name} is not a decode, prefill, verify or cache-write workload", file=sys.stderr)
        return 2
    inp = gen.make_decode_inputs(w)
    dev = torch.device("cuda:0")
    flags = 0
    inp_dev = inp
    if args.fp8:  # FP8 rows of the same latents, quantised on the GPU (mla_quantize_rows_fp8)
        P, ps, _ = inp["pool"].shape
        src = runner.to_device(inp["pool"], dev)
        pool8 = torch.empty((P, ps, L.MLA_FP8_ROW_BYTES), dtype=torch.uint8, device=dev)
        L.mla_quantize_rows_fp8(runner.dims_for(w), src, P * ps, pool8)
        torch.cuda.synchronize()
        del src
        inp_dev = dict(inp, pool=pool8)
        flags = L.MLA_FLAG_CACHE_FP8
    fused = args.fused
    if args.split_tokens:
        st = runner.DecodeStep(inp_dev, args.split_tokens, dev, flags=flags, fused=fused)
    else:
        n_units = args.units or runner.balanced_units(inp["lens"], runner.compute_units(dev))
        st = runner.DecodeStep(inp_dev, 0, dev, n_units=n_units, flags=flags, fused=fused)
    lens = inp["lens"].astype(np.int64)
    total_tokens = int(lens.sum())
    row_bytes = L.MLA_FP8_ROW_BYTES if args.fp8 else (w.d_c + w.d_r) * 2
    cache_bytes = total_tokens * row_bytes
    flops_decode = total_tokens * (2 * w.n_heads * (w.d_c + w.d_r) + 2 * w.n_heads * w.d_c)
    flops_proj = w.batch * 2 * w.n_heads * w.d_c * (w.d_k + w.d_v)

    # The copy-bandwidth probe runs first, outside the timed region; it is the measured denominator
    # reported beside the published peak, and it brings the board's clocks from idle to their
    # sustained level before the warm-up steps (reported as "pre_timed").
    copy = measured_copy_gbs(dev)
    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # The same step captured once in a HIP graph and replayed (one host launch per step), also
    # measured before the warm-up steps, over at least 100 replays.
    graph = runner.CapturedStep(st)
    graph.run()
    torch.cuda.synchronize()
    n_graph = max(args.steps, 100)
    start.record(stream)
    for _ in range(n_graph):
        graph.run()
    stop.record(stream)
    torch.cuda.synchronize()
    ms_graph = start.elapsed_time(stop) / n_graph
    for _ in range(args.warmup):
        st.run()
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        st.absorb()
        ev[i][0].record(stream)
        st.attend()
        ev[i][1].record(stream)
        st.finish()
    stop.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    ms_decode = float(np.mean(launch_ms))
    copy_gbs = copy["gbs"]
    # After the timed region: the part after the decode both ways on the same partials, the fused
    # merge + value projection and mla_combine* followed by mla_out_proj (median of 50 each).
    finish = None
    if L.mla_combine_out_proj_supported(st.d):
        def _median_ms(fn, n=50):
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
            for a_, b_ in evs:
                a_.record(stream)
                fn()
                b_.record(stream)
            torch.cuda.synchronize()
            return float(np.median([a_.elapsed_time(b_) for a_, b_ in evs]))

        def _unfused():
            st.combine()
            st.out_proj()

        ms_f = _median_ms(st.combine_out_proj)
        ms_u = _median_ms(_unfused)
        finish = {"fused_ms": round(ms_f, 6), "combine_then_out_proj_ms": round(ms_u, 6),
                  "note": "median time of the calls after the decode launch, on the same partials: the fused "
                          "merge + value projection against mla_combine* then mla_out_proj"}

    sha = _kernel_sha()
    traffic = None if args.fp8 else _traffic(w.name, sha)
    achieved = cache_bytes / (ms_decode * 1e-3) / 1e9
    rec = {
        "metric": "MLA decode cache GB/s (V3 shape, 1 GPU)" + (", FP8 cache" if args.fp8 else ""),
        "value": round(cache_bytes / (ms_step * 1e-3) / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.n_heads, "d_c": w.d_c, "d_r": w.d_r,
                   "d_k": w.d_k, "d_v": w.d_v, "page_size": w.page_size,
                   "split": f"fixed {st.split_tokens}" if st.n_units is None else f"balanced {st.n_units} units",
                   "partials": st.S * (st.B if st.n_units is None else 1), "cache_tokens": total_tokens, "seed": w.seed,
                   "decode_kernel": "mfma" if st.uses_mfma() else "generic",
                   "cache_format": "fp8 e4m3, 656 B rows" if args.fp8 else "bf16, 1,152 B rows"},
        "tokens_per_s": round(w.batch / (ms_step * 1e-3), 1),
        "cache_tokens_per_s": round(total_tokens / (ms_step * 1e-3), 1),
        "tflops": round((flops_decode + flops_proj) / (ms_step * 1e-3) / 1e12, 3),
        "wall_s": round(t_wall, 4),
        "pre_timed": {"gpu_ms": round(copy["gpu_ms"] + (1 + n_graph) * ms_graph, 1),
                      "work": f"before the warm-up steps: the copy-bandwidth probe ({copy['copies']} plain 1 GiB "
                              f"device copies), then the graph-replay measurement ({n_graph} replays of the same step); "
                              "from idle the board needs about 100 decode steps of load before its clocks settle"},
        "step_calls": ("absorb, decode, fused merge + value projection" if st.fused
                       else "absorb, decode, merge, value projection"),
        "after_decode": finish,
        "graph": {"ms_per_step": round(ms_graph, 6), "value": round(cache_bytes / (ms_graph * 1e-3) / 1e9, 3),
                  "tokens_per_s": round(w.batch / (ms_graph * 1e-3), 1), "replays": n_graph,
                  "note": "the same launches captured in one HIP graph and replayed"},
        "roofline": {"bound": "hbm", "kernel": "mla_decode_partial", "achieved": round(achieved, 3),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "ms_per_launch": round(ms_decode, 6),
                     "ms_per_launch_median": round(float(np.median(launch_ms)), 6),
                     "algorithmic_bytes_per_launch": cache_bytes, "kernel_source_sha": sha,
                     "measured_copy_gbs": copy_gbs, "frac_of_measured_copy": round(achieved / copy_gbs, 4)},
        "roofline_mfma": {"achieved": round(flops_decode / (ms_decode * 1e-3) / 1e12, 3),
                          "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(flops_decode / (ms_decode * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = (cpu_baseline_fp8 if args.fp8 else cpu_baseline)(inp, args.cpu_seconds)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
