"""Benchmark of one token-chunked DiT block forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config large] [--no-cpu-baseline]
    python bench.py --op final_layer [--steps K] [--warmup W]

A step is one full block forward (pass 1 K/V, pass 2 Q/attention/out-proj,
SwiGLU MLP) over the whole token sequence, preceded by a device copy that
restores the input x (the forward overwrites x in place). Inputs are seeded
synthetic arrays already resident in HBM when timing starts. Prints one JSON
line. The dominant kernel (attention) is timed per launch with HIP events on
the stream the library launches on, over a second pass of K steps.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "DiT-block tokens/s & % bf16 MFMA peak at 32k tokens; peak workspace bytes"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
FINAL_N, FINAL_D, FINAL_OUT = 32768, 5120, 64


# HBM traffic records: FETCH_SIZE and WRITE_SIZE of one launch at the bench
# shape, each scaled by what the same counter reads for a plain copy kernel of
# known size (``--probe`` runs both; ``--record-traffic`` writes the record).
COPY_BYTES = 1 << 30  # the calibration kernel reads and writes 1 GiB
TRAFFIC = {
    "attention": {
        "record": "attention_large_32k_traffic.json",
        "kernel": "dit::attention_bf16_kernel",
        "sources": ["memory_bounded_chunked_amd/csrc/attention.hip", "memory_bounded_chunked_amd/csrc/common.hpp"],
        "workload": "8192 query rows x 32768 keys, 40 heads x 128, bf16 (one launch of the 32k-token block)",
        # Q slab + K + V^T + O, each bf16 [rows][5120]
        "algorithmic_bytes": (8192 + 32768 + 32768 + 8192) * 5120 * 2,
    },
    "gate_up": {
        "record": "gate_up_large_8192_traffic.json",
        "kernel": "dit::gemm_kernel<unsigned short, unsigned short, 3,",
        "sources": ["memory_bounded_chunked_amd/csrc/gemm.hip", "memory_bounded_chunked_amd/csrc/common.hpp",
                    "memory_bounded_chunked_amd/csrc/kernels.hpp"],
        "workload": "SwiGLU gate/up projection of one 8192-token slab: [8192 x 5120] x [2 x 13824 x 5120]^T "
                    "-> h [8192 x 13824], bf16 (two launches: 256x256 and 256x128 tiles)",
        # activations + gate/up weight rows + h, bf16
        "algorithmic_bytes": (8192 * 5120 + 2 * 13824 * 5120 + 8192 * 13824) * 2,
    },
    "modnorm": {
        "record": "modnorm_large_8192_traffic.json",
        "kernel": "dit::modnorm_kernel<unsigned short, unsigned short,",
        "sources": ["memory_bounded_chunked_amd/csrc/modnorm.hip", "memory_bounded_chunked_amd/csrc/common.hpp"],
        "workload": "norm1 of one 8192-token slab: bf16 x [8192 x 5120] -> bf16 [8192 x 5120], fp32 shift/scale",
        # x in + normalised slab out, bf16, + shift and scale fp32
        "algorithmic_bytes": 2 * 8192 * 5120 * 2 + 2 * 5120 * 4,
    },
    "norm2": {
        "record": "norm2_large_8192_traffic.json",
        "kernel": "dit::modnorm_kernel<float, unsigned short,",
        "sources": ["memory_bounded_chunked_amd/csrc/modnorm.hip", "memory_bounded_chunked_amd/csrc/common.hpp"],
        "workload": "norm2 of one 8192-token slab: fp32 staged residual [8192 x 5120] -> bf16 [8192 x 5120]",
        # fp32 stage in + bf16 out + shift and scale fp32
        "algorithmic_bytes": 8192 * 5120 * (4 + 2) + 2 * 5120 * 4,
    },
    "final_layer": {
        "record": "final_layer_32k_traffic.json",
        "kernel": "dit::final_layer_kernel",
        "sources": ["memory_bounded_chunked_amd/csrc/final_layer.hip", "memory_bounded_chunked_amd/csrc/common.hpp"],
        "workload": "output head: 32768 bf16 rows x 5120 -> 64 fp32 outputs",
        # x bf16 + w_out fp32 + shift/scale fp32 + out fp32
        "algorithmic_bytes": 32768 * 5120 * 2 + 64 * 5120 * 4 + 2 * 5120 * 4 + 32768 * 64 * 4,
    },
}


def _sources_sha(files) -> str:
    import hashlib
    return hashlib.sha256(b"".join(open(os.path.join(ROOT, f), "rb").read() for f in files)).hexdigest()


def measured_traffic(kind: str) -> float | None:
    """HBM bytes per launch of ``kind`` from its committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE record, if the kernel sources are still the measured ones."""
    spec = TRAFFIC[kind]
    path = os.path.join(ROOT, "profiles", spec["record"])
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if _sources_sha(rec["source_files"]) != rec["source_sha256"]:
        return None
    return rec["traffic_bytes_per_launch"]


def traffic_probe(kind: str) -> int:
    """One launch of ``kind`` at the bench shape on random inputs, then the copy
    kernel used to calibrate the counters (run under rocprofv3 --pmc)."""
    import torch

    from memory_bounded_chunked_amd import block as B
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(0)
    if kind == "attention":
        d, h, n, ca = 5120, 40, 32768, 8192
        q = torch.randn(ca, d, device=dev, generator=g).bfloat16()
        k = torch.randn(n, d, device=dev, generator=g).bfloat16()
        vt = torch.randn(d, n, device=dev, generator=g).bfloat16()
        o = torch.empty(ca, d, device=dev, dtype=torch.bfloat16)
        run = lambda: B.attention(q, k, vt, o, h)  # noqa: E731
    elif kind == "gate_up":
        m, d, f = 8192, 5120, 13824
        a_in = torch.randn(m, d, device=dev, generator=g).bfloat16()
        w = (torch.randn(2 * f, d, device=dev, generator=g) / d ** 0.5).bfloat16()
        h = torch.empty(m, f, device=dev, dtype=torch.bfloat16)
        run = lambda: B.linear("bf16", "gateup", a_in, w, h, f, up_offset=f)  # noqa: E731
    elif kind in ("modnorm", "norm2"):
        m, d = 8192, 5120
        xin = torch.randn(m, d, device=dev, generator=g)
        if kind == "modnorm":
            xin = xin.bfloat16()
        sh, sc = torch.randn(d, device=dev, generator=g) * 0.3, torch.randn(d, device=dev, generator=g) * 0.3
        out = torch.empty(m, d, device=dev, dtype=torch.bfloat16)
        run = lambda: B.modnorm(xin, sh, sc, out)  # noqa: E731
    else:
        n, d, od = FINAL_N, FINAL_D, FINAL_OUT
        x = torch.randn(n, d, device=dev, generator=g).bfloat16()
        sh, sc = torch.randn(d, device=dev, generator=g) * 0.3, torch.randn(d, device=dev, generator=g) * 0.3
        w = torch.randn(od, d, device=dev, generator=g) / d ** 0.5
        out = torch.empty(n, od, device=dev)
        run = lambda: B.final_layer(x, sh, sc, w, out=out)  # noqa: E731
    a = torch.randn(COPY_BYTES // 4, device=dev, generator=g)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    run()
    torch.mul(a, 1.0, out=b)  # the copy kernel: reads and writes COPY_BYTES
    torch.cuda.synchronize()
    log(f"[probe] {kind}: one launch + copy kernel done")
    return 0


def record_traffic(kind: str, fetch_csv: str, write_csv: str) -> int:
    """Write profiles/<record> from the counter_collection.csv of a FETCH_SIZE
    run and of a WRITE_SIZE run of ``--probe kind`` (host only)."""
    import csv
    spec = TRAFFIC[kind]

    def rows_of(path, key):
        return [float(r["Counter_Value"]) for r in csv.DictReader(open(path)) if key in r["Kernel_Name"]]

    def total(path, key):  # one launch of the step: all dispatches of its kernel
        return sum(rows_of(path, key))

    def last(path, key):  # the copy kernel runs last
        return rows_of(path, key)[-1]

    fk, wk = total(fetch_csv, spec["kernel"]), total(write_csv, spec["kernel"])
    cf, cw = last(fetch_csv, "AUnaryFunctor"), last(write_csv, "AUnaryFunctor")
    fs, ws = COPY_BYTES / (cf * 1024), COPY_BYTES / (cw * 1024)
    traffic = fk * 1024 * fs + wk * 1024 * ws
    rec = {
        "kernel": spec["kernel"],
        "workload": spec["workload"],
        "source_sha256": _sources_sha(spec["sources"]),
        "source_files": spec["sources"],
        "fetch_size_kib": fk, "write_size_kib": wk,
        "copy_kernel": "torch.mul(a, 1.0, out=b) on 1 GiB fp32: reads 1 GiB, writes 1 GiB",
        "copy_fetch_size_kib": cf, "copy_write_size_kib": cw,
        "fetch_scale": fs, "write_scale": ws,
        "traffic_bytes_per_launch": traffic,
        "algorithmic_bytes_per_launch": spec["algorithmic_bytes"],
        "commands": [f"TMPDIR=/tmp rocprofv3 --pmc {c} --output-format csv -d traffic_{kind}_{c} -o t "
                     f"-- python3 bench.py --probe {kind}" for c in ("FETCH_SIZE", "WRITE_SIZE")]
                    + [f"python3 bench.py --record-traffic {kind} <FETCH_SIZE counter_collection.csv> "
                       f"<WRITE_SIZE counter_collection.csv>"],
    }
    path = os.path.join(ROOT, "profiles", spec["record"])
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    log(f"[traffic] {kind}: {traffic / 1e6:.1f} MB per launch (algorithmic {spec['algorithmic_bytes'] / 1e6:.1f} MB)"
        f" -> {path}")
    return 0


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(shape, inputs, rows: int) -> dict:
    """The fp64 oracle on a bounded sample: norm1 and K/V for all N tokens plus
    the remaining steps for ``rows`` sampled query rows; extrapolated to N rows."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle.dit_block as O
    from memory_bounded_chunked_amd import synth

    x = synth.to_f64(inputs["x"])
    mod = inputs["mod"].astype(np.float64)
    w = O.block_weights_f64({k: synth.to_f64(v) for k, v in inputs.items() if k[:2] in ("w_", "s_")})
    d = shape.d
    sh1, sc1 = mod[0], mod[1]
    t0 = time.perf_counter()
    n1 = O.modulate(O.layer_norm(x, shape.eps), sh1, sc1)
    k = O.linear(n1, w["qkv"][d:2 * d])
    v = O.linear(n1, w["qkv"][2 * d:])
    del n1
    t_kv = time.perf_counter() - t0
    sel = synth.sample_rows(shape.n_tokens, rows, seed=1)
    t1 = time.perf_counter()
    xr = x[sel]
    n1r = O.modulate(O.layer_norm(xr, shape.eps), sh1, sc1)
    o = O.attention(O.linear(n1r, w["qkv"][:d]), k, v, shape.n_heads)
    x1 = xr + mod[2] * O.linear(o, w["o"])
    n2 = O.modulate(O.layer_norm(x1, shape.eps), mod[3], mod[4])
    f = shape.ffn
    h = O.silu(O.linear(n2, w["gu"][:f])) * O.linear(n2, w["gu"][f:])
    _ = x1 + mod[5] * O.linear(h, w["down"])
    t_rows = time.perf_counter() - t1
    t_full = t_kv + t_rows * shape.n_tokens / len(sel)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": shape.n_tokens / t_full, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"fp64 oracle: norm1+K/V for all {shape.n_tokens} tokens ({t_kv:.1f} s) + steps for "
                       f"{len(sel)} sampled query rows ({t_rows:.1f} s); full block extrapolated "
                       f"to {t_full:.0f} s"),
            "measured_s": round(t_kv + t_rows, 2), "cpu_count": os.cpu_count()}


def bench_final_layer(args) -> int:
    """The output head after the last block (dit_final_layer): a step is one head
    call over all tokens: 32768 bf16 token rows of width 5120 (the large block's
    residual stream) to 64 fp32 outputs each (a 1x2x2 patch of 16 latent channels)."""
    import numpy as np
    import torch

    from memory_bounded_chunked_amd import block as B
    from memory_bounded_chunked_amd import synth

    n, d, od = FINAL_N, FINAL_D, FINAL_OUT
    dev = "cuda:0"
    inp = synth.make_final_inputs(n, d, od, "bf16", seed=0)
    t = {k: B.tensor_from_stored(v, dev) for k, v in inp.items()}
    out = torch.empty((n, od), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        B.final_layer(t["x"], t["shift"], t["scale"], t["w_out"], out=out, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    B.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    k_ms, k_n = B.profile_read()["final"]
    B.profile_enable(False)
    avg = k_ms / k_n
    flops = 2.0 * n * d * od
    achieved = flops / (avg / 1e3) / 1e12
    hbm_bytes = n * d * 2 + od * d * 4 + 2 * d * 4 + n * od * 4
    log(f"[bench] final layer: {ms:.4f} ms/step, kernel {avg:.4f} ms, {achieved:.1f} TFLOP/s fp32")
    result = {
        "metric": "output-head tokens/s (fp32 modulated LayerNorm + projection) at 32k tokens",
        "value": round(n / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded PCG64 inputs at the workload's shapes)",
        "config": {"workload": f"DiT output head: N={n} bf16 token rows, d={d} -> {od} fp32 outputs, batch 1",
                   "n_tokens": n, "d": d, "out_dim": od, "workspace_bytes": 0},
        "roofline": {"kernel": "final_layer", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_F32_TFLOPS, 4),
                     "traffic": measured_traffic("final_layer"), "avg_launch_ms": round(avg, 4),
                     "flops_per_launch": flops,
                     "hbm_gbs_algorithmic": round(hbm_bytes / (avg / 1e3) / 1e9, 1)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info

        import oracle.dit_block as O
        # Slabs of 4096 token rows in order, repeated over the sequence until at
        # least 10 s of oracle work has run.
        sh, sc, wo = (inp[k].astype(np.float64) for k in ("shift", "scale", "w_out"))
        rows, r0, t0 = 0, 0, time.perf_counter()
        while time.perf_counter() - t0 < 10.0:
            O.final_layer(synth.to_f64(inp["x"][r0:r0 + 4096]), sh, sc, wo)
            rows += min(4096, n - r0)
            r0 = (r0 + 4096) % n
        dt = time.perf_counter() - t0
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        result["cpu_baseline"] = {"value": round(rows / dt, 1), "unit": "tokens/s", "cores": threads,
                                  "kind": "oracle",
                                  "sample": f"fp64 oracle head on {rows} token rows in 4096-row slabs ({dt:.1f} s)"}
    print(json.dumps(result), flush=True)
    return 0


def library_reference(config: str) -> int:
    """The platform libraries on the same box and the same shapes as this
    library's kernels: torch's F.linear (hipBLASLt) on the block's projection
    shapes and torch's flash SDPA on one attention launch, each timed beside
    the kernel of this library that does the same product (bf16 weights, the
    plain-store epilogue; attention with n_kv keys). A context measurement;
    nothing here is on the block's path. One JSON line."""
    import torch
    import torch.nn.functional as F

    from memory_bounded_chunked_amd import block as B
    from memory_bounded_chunked_amd import synth

    shape = synth.CONFIGS[config]
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(0)
    d, ffn, heads, dh = shape.d, shape.ffn, shape.n_heads, shape.head_dim
    ca, cm, n = shape.attn_chunk or shape.n_tokens, shape.mlp_chunk or shape.n_tokens, shape.n_tokens

    def timeit(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out = {}
    for name, m, k, nn in (("q", ca, d, d), ("kv", ca, d, 2 * d), ("gate_up", cm, d, 2 * ffn), ("down", cm, ffn, d)):
        a = torch.randn(m, k, device=dev, generator=g).bfloat16()
        w = (torch.randn(nn, k, device=dev, generator=g) * k ** -0.5).bfloat16()
        o = torch.empty(m, nn, device=dev, dtype=torch.bfloat16)
        flops = 2.0 * m * k * nn
        t_lib = timeit(lambda: B.linear("bf16", "store", a, w, o, nn))
        t_ref = timeit(lambda: F.linear(a, w))
        out[name] = {"shape": [m, k, nn], "this_ms": round(t_lib, 4), "this_tflops": round(flops / t_lib / 1e9, 1),
                     "hipblaslt_ms": round(t_ref, 4), "hipblaslt_tflops": round(flops / t_ref / 1e9, 1)}
        log(f"[reference] {name}: this {t_lib:.3f} ms, hipBLASLt {t_ref:.3f} ms")
        del a, w, o
    q = torch.randn(ca, d, device=dev, generator=g).bfloat16()
    k = torch.randn(n, d, device=dev, generator=g).bfloat16()
    vt = torch.randn(d, n, device=dev, generator=g).bfloat16()
    o = torch.empty(ca, d, device=dev, dtype=torch.bfloat16)
    flops = 4.0 * ca * n * d
    t_lib = timeit(lambda: B.attention(q, k, vt, o, heads), reps=5)
    att = {"shape": [ca, n, heads, dh], "this_ms": round(t_lib, 4), "this_tflops": round(flops / t_lib / 1e9, 1)}
    # torch's layout: (batch, heads, tokens, dh), contiguous
    qs = q.view(ca, heads, dh).transpose(0, 1).contiguous().unsqueeze(0)
    ks = k.view(n, heads, dh).transpose(0, 1).contiguous().unsqueeze(0)
    vs = vt.view(heads, dh, n).transpose(1, 2).contiguous().unsqueeze(0)
    del q, k, vt, o
    from torch.nn.attention import SDPBackend, sdpa_kernel
    for be in (SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION):
        try:  # the named backend only: no fallback to the unfused product
            with sdpa_kernel([be]):
                t_ref = timeit(lambda: F.scaled_dot_product_attention(qs, ks, vs), reps=5)
            att[f"sdpa_{be.name.lower()}_ms"] = round(t_ref, 4)
            att[f"sdpa_{be.name.lower()}_tflops"] = round(flops / t_ref / 1e9, 1)
            log(f"[reference] attention: this {t_lib:.3f} ms, SDPA {be.name} {t_ref:.3f} ms")
        except RuntimeError as ex:
            att[f"sdpa_{be.name.lower()}"] = f"unavailable: {str(ex)[:80]}"
    out["attention"] = att
    print(json.dumps({"reference": {"workload": shape.name, "device": torch.cuda.get_device_name(0), **out}}))
    return 0


def copy_roofline(config: str) -> int:
    """The HBM-bound norm kernels against a plain copy of the same bytes, each
    launch timed alone from a cold cache (a 1 GiB buffer is rewritten before
    every launch, more than the last-level cache holds): norm1 (bf16 in, bf16
    out) against torch's bf16 copy, norm2 (fp32 in, bf16 out) against torch's
    fp32 -> bf16 copy, at one slab of the configuration and at 65536 rows. The
    copy is the streaming rate this machine reaches with the same bytes. One JSON
    line; medians of 7 launches."""
    import statistics

    import torch

    from memory_bounded_chunked_amd import block as B
    from memory_bounded_chunked_amd import synth

    shape = synth.CONFIGS[config]
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(0)
    flush = torch.empty(1 << 28, device=dev, dtype=torch.float32)

    def cold(fn, reps=7):
        ts = []
        for _ in range(reps):
            flush.add_(1.0)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return statistics.median(ts)

    out = []
    d = shape.d
    for rows in sorted({shape.mlp_chunk or shape.n_tokens, 65536}):
        x = torch.randn(rows, d, device=dev, generator=g).bfloat16()
        xf = torch.randn(rows, d, device=dev, generator=g)
        y = torch.empty(rows, d, device=dev, dtype=torch.bfloat16)
        sh = torch.randn(d, device=dev, generator=g) * 0.1
        sc = torch.randn(d, device=dev, generator=g) * 0.1
        b1, b2 = rows * d * 4, rows * d * 6
        t = {"copy_bf16": cold(lambda: y.copy_(x)), "norm1": cold(lambda: B.modnorm(x, sh, sc, y)),
             "copy_f32_bf16": cold(lambda: y.copy_(xf)), "norm2": cold(lambda: B.modnorm(xf, sh, sc, y))}
        rec = {"rows": rows, "d": d}
        for k, ms in t.items():
            nb = b1 if k in ("copy_bf16", "norm1") else b2
            rec[k] = {"us": round(ms * 1e3, 1), "tb_s": round(nb / (ms * 1e-3) / 1e12, 2)}
        out.append(rec)
        log(f"[copy] {rows} rows: " + ", ".join(f"{k} {v['us']} us {v['tb_s']} TB/s" for k, v in rec.items()
                                               if isinstance(v, dict)))
        del x, xf, y
    print(json.dumps({"copy_roofline": {"workload": shape.name, "cold_cache": True, "sizes": out}}))
    return 0


def secondary_configs(steps: int) -> dict:
    """Short timing of the other block configurations at their own chunk
    settings (two warm-ups, `steps` timed forwards each, HIP events on the
    library's stream), so that one default run records them beside the large
    block: the mid block (also with two key ranges per query, its measured
    best, and unchunked, as its workload also defines), the long clip with
    FFN feature slices and the int8-weight block."""
    import torch

    from memory_bounded_chunked_amd import block as B
    from memory_bounded_chunked_amd import synth
    dev = "cuda:0"
    out = {}
    for name, splits, unchunked in (("mid", 1, False), ("mid", 2, False), ("mid", 1, True), ("longclip", 1, False),
                                    ("int8", 1, False)):
        key = name if splits == 1 else f"{name}_splits{splits}"
        key += "_unchunked" if unchunked else ""
        try:
            out[key] = _time_secondary(B, synth, dev, name, splits, steps, unchunked)
        except Exception as e:  # reported in the record; the headline line still prints
            out[key] = {"error": f"{type(e).__name__}: {e}"}
            log(f"[bench] secondary {key} failed: {e}")
        torch.cuda.empty_cache()
    return out


def _time_secondary(B, synth, dev, name, splits, steps, unchunked=False) -> dict:
    """One configuration of secondary_configs: its record (unchunked: one
    attention slice of all tokens and one MLP slab, the stock schedule)."""
    import torch
    shape = synth.CONFIGS[name]
    t0 = time.perf_counter()
    inputs = synth.make_inputs(shape, seed=0)
    blk, x0, mod = B.block_from_inputs(shape, inputs, dev)
    del inputs
    try:
        if splits != 1:
            blk.set_attention_splits(splits)
        ca, cm, fc = shape.attn_chunk, shape.mlp_chunk, shape.ffn_chunk
        if unchunked:
            ca, cm = 0, shape.n_tokens
        ws_bytes = blk.peak_workspace(shape.n_tokens, ca, cm, fc)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        x = x0.clone()
        stream = torch.cuda.current_stream()

        def step():
            x.copy_(x0)
            blk.forward(x, mod, ca, cm, fc, workspace=ws, stream=stream)

        def timed(fn) -> float:
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(steps):
                fn()
            ev1.record(stream)
            torch.cuda.synchronize()
            return ev0.elapsed_time(ev1) / steps

        for _ in range(2):
            step()
        torch.cuda.synchronize()
        ms = timed(step)
        copy_ms = timed(lambda: x.copy_(x0))  # the restoring copy inside each step, alone
    finally:
        blk.close()
    tflops = shape.flops / (ms / 1e3) / 1e12
    log(f"[bench] secondary {name} (chunks {ca}/{cm}, key ranges {splits}): {ms:.3f} ms/step ({tflops:.0f} TFLOP/s) "
        f"incl. setup "
        f"{time.perf_counter() - t0:.1f}s")
    return {
        "n_tokens": shape.n_tokens, "d": shape.d, "dtype": shape.dtype,
        "attn_chunk_tokens": ca, "mlp_chunk_tokens": cm, "ffn_chunk_features": fc,
        **({"attention_splits": splits} if splits != 1 else {}),
        "steps": steps, "ms_per_step": round(ms, 3), "copy_ms_per_step": round(copy_ms, 3),
        "tokens_per_s": round(shape.n_tokens / (ms / 1e3), 1),
        "tflops": round(tflops, 1), "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "peak_workspace_bytes": ws_bytes,
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="large")
    ap.add_argument("--attn-chunk", type=int, default=None)
    ap.add_argument("--mlp-chunk", type=int, default=None)
    ap.add_argument("--ffn-chunk", type=int, default=None)
    ap.add_argument("--attn-splits", type=int, default=1,
                    help="key ranges per query in attention (dit_block_set_attention_splits)")
    ap.add_argument("--cpu-rows", type=int, default=2048)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--qk", action="store_true", help="with QK RMSNorm and RoPE (a widening of the path)")
    ap.add_argument("--lora", type=int, default=0, metavar="RANK",
                    help="with rank-RANK activation-space adapters on all seven projections (a widening)")
    ap.add_argument("--op", choices=("block", "final_layer"), default="block",
                    help="block forward (default) or the output head after the last block")
    ap.add_argument("--probe", choices=tuple(TRAFFIC), default=None,
                    help="one launch of a kernel plus the calibration copy, for rocprofv3 --pmc")
    ap.add_argument("--reference", action="store_true",
                    help="time torch's F.linear (hipBLASLt) and flash SDPA beside this library's kernels on the "
                         "configuration's shapes (context, not the block)")
    ap.add_argument("--copy-roofline", action="store_true",
                    help="the norm kernels against a plain copy of the same bytes, each from a cold cache")
    ap.add_argument("--record-traffic", nargs=3, metavar=("KERNEL", "FETCH_CSV", "WRITE_CSV"), default=None,
                    help="write the traffic record of KERNEL from two counter_collection.csv files")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the short timing of the other configurations that the default run adds")
    ap.add_argument("--secondary-steps", type=int, default=5)
    args = ap.parse_args()
    if args.record_traffic:
        return record_traffic(*args.record_traffic)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the block path is "
              "single-GPU: no collectives)", file=sys.stderr)
        return 2
    if args.probe:
        return traffic_probe(args.probe)
    if args.reference:
        return library_reference(args.config)
    if args.copy_roofline:
        return copy_roofline(args.config)
    if args.op == "final_layer":
        return bench_final_layer(args)

    import torch

    from memory_bounded_chunked_amd import block as B
    from memory_bounded_chunked_amd import synth

    shape = synth.CONFIGS[args.config]
    ca = shape.attn_chunk if args.attn_chunk is None else args.attn_chunk
    cm = shape.mlp_chunk if args.mlp_chunk is None else args.mlp_chunk
    fc = shape.ffn_chunk if args.ffn_chunk is None else args.ffn_chunk
    dev = "cuda:0"
    t0 = time.perf_counter()
    inputs = synth.make_inputs(shape, seed=0)
    log(f"[bench] inputs for {shape.name} drawn in {time.perf_counter() - t0:.1f}s")
    rope = None
    if args.qk:
        qk_in = synth.make_qk_inputs(shape, 0)
        inputs = {**inputs, "q_norm": qk_in["q_norm"], "k_norm": qk_in["k_norm"]}
        rope = (torch.from_numpy(qk_in["cos"]).to(dev), torch.from_numpy(qk_in["sin"]).to(dev))
    blk, x0, mod = B.block_from_inputs(shape, inputs, dev)
    if args.attn_splits != 1:
        blk.set_attention_splits(args.attn_splits)
    lora_flops = 0.0
    if args.lora:
        lora = synth.make_lora(shape, args.lora, seed=0)
        blk.set_lora({k: (B.tensor_from_stored(a, dev), B.tensor_from_stored(b, dev), al)
                      for k, (a, b, al) in lora.items()})
        # A then B of each adapter: 2*N*r*(in + out) over q, k, v, o (d, d), gate, up (d, F), down (F, d)
        lora_flops = 2.0 * shape.n_tokens * args.lora * (11 * shape.d + 3 * shape.ffn)
    x = x0.clone()
    ws_bytes = blk.peak_workspace(shape.n_tokens, ca, cm, fc)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        x.copy_(x0)
        blk.forward(x, mod, ca, cm, fc, workspace=ws, stream=stream, rope=rope)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = ev0.elapsed_time(ev1) / args.steps
    log(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step (wall {wall:.3f}s)")

    # per-kernel HIP-event timing over a second pass of the same steps
    B.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = B.profile_read()
    B.profile_enable(False)
    kernels = {k: {"total_ms_per_step": round(t / args.steps, 4), "launches_per_step": n // args.steps,
                   "avg_launch_ms": round(t / n, 4) if n else None} for k, (t, n) in prof.items()}
    # the HBM-bound norms: algorithmic bytes of their launches (rows in, rows out,
    # shift and scale) over their summed launch time
    e = 4 if shape.dtype == "f32" else 2
    n_tok, d_ = shape.n_tokens, shape.d
    norm_bytes = {  # per forward: norm1 runs over every token twice (pass 1 and pass 2), norm2 once
        "modnorm": 2 * n_tok * d_ * (e + e) + prof["modnorm"][1] // args.steps * 2 * d_ * 4,
        "norm2": n_tok * d_ * (4 + e) + prof["norm2"][1] // args.steps * 2 * d_ * 4,
    }
    for kname, nb in norm_bytes.items():
        t_step = kernels[kname]["total_ms_per_step"]
        if t_step:
            kernels[kname]["hbm_gbs"] = round(nb / (t_step / 1e3) / 1e9, 1)
            kernels[kname]["hbm_frac"] = round(nb / (t_step / 1e3) / 1e9 / PEAK_HBM_GBS, 4)
    log("[bench] per-kernel: " + json.dumps(kernels))

    n, d = shape.n_tokens, shape.d
    flops = shape.flops
    tflops = flops / (ms / 1e3) / 1e12
    peak = PEAK_F32_TFLOPS if shape.dtype == "f32" else PEAK_BF16_TFLOPS
    att_t, att_n = prof["attention"]
    ca_eff = n if ca == 0 else min(ca, n)
    # Algorithmic FLOPs of one attention launch: 4*d per (query, key) pair
    # (QK^T and PV, 2*d each) x (ca_eff query rows x N keys).
    att_flops_launch = 4.0 * d * ca_eff * n
    att_avg_ms = att_t / att_n if att_n else None
    att_tflops = att_flops_launch / (att_avg_ms / 1e3) / 1e12 if att_avg_ms else None
    roofline = {
        "kernel": "attention",
        "bound": "mfma",
        "achieved": round(att_tflops, 1) if att_tflops else None,
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(att_tflops / peak, 4) if att_tflops else None,
        "traffic": (measured_traffic("attention") if args.config == "large" and ca == 8192 and args.attn_splits == 1
                    else None),
        "avg_launch_ms": round(att_avg_ms, 4) if att_avg_ms else None,
        "flops_per_launch": att_flops_launch,
    }
    result = {
        "metric": METRIC,
        "value": round(n / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "w8_bf16": "w8a16-bf16"}[shape.dtype],
        "data": "synthetic (seeded PCG64 inputs at the workload's shapes)",
        "config": {
            "workload": (f"{shape.name} DiT block forward: d={d}, {shape.n_heads}x{shape.head_dim} heads, "
                         f"SwiGLU F={shape.ffn}, N={n} tokens, batch 1"
                         + (", QK RMSNorm + RoPE" if args.qk else "")
                         + (f", rank-{args.lora} adapters on q/k/v/o/gate/up/down" if args.lora else "")),
            "n_tokens": n, "attn_chunk_tokens": ca, "mlp_chunk_tokens": cm, "ffn_chunk_features": fc,
            **({"attention_splits": args.attn_splits} if args.attn_splits != 1 else {}),
            "peak_workspace_bytes": ws_bytes,
            "tflops": round(tflops, 1),
            "frac_bf16_peak": round(tflops / peak, 4),
            "flops_per_step": flops,
            **({"lora_rank": args.lora, "lora_flops_per_step": lora_flops} if args.lora else {}),
        },
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": None,
    }
    blk.close()
    del x, x0, ws
    torch.cuda.empty_cache()
    default_run = (args.config == "large" and not (args.qk or args.lora) and args.attn_splits == 1
                   and args.attn_chunk is None and args.mlp_chunk is None and args.ffn_chunk is None)
    if default_run and not args.no_secondary:
        result["secondary"] = secondary_configs(args.secondary_steps)
    if not args.no_cpu_baseline and not args.lora:
        log("[bench] cpu_baseline: fp64 oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(shape, inputs, args.cpu_rows)
        log(f"[bench] cpu_baseline done: {result['cpu_baseline']['sample']}")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
