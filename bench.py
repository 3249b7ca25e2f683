"""Benchmark of the 4-bit codebook GEMV on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--copies R] [--no-secondary]
                    [--secondary tiny,down,smalln,gateup,prefill_down,fused,gather,affine,nvfp4,x8,pages]

A step is one q4_gemv call on the lm_head workload (M x K = 151936 x 2048,
x bf16 unit-RMS, y fp32): the projection the metric is quoted on.  Inputs are
resident in HBM before timing starts.  Each step reads a different one of R
packed copies of the matrix, so that the 256 MB Infinity Cache and the L2
cannot serve the weights (R * 166 MB >= 600 MB).  The K timed steps are
captured in one HIP graph (as a decode step is) and replayed between two
events on the replay stream; --eager adds the same calls launched one by one.

Byte model (deep-fold "Decode V2", section 6 bench: GB/s = packed + scale +
x over the median time; the y write is added here):
    bytes = M*K/2 (codes) + M*K/32 (fp16 scales) + 2K (x) + 4M (y).

Output: one JSON line with the metric, the per-launch kernel time measured
with HIP events on the launch stream, the HBM roofline fraction against the
8 TB/s peak, secondary workloads (down-projection GEMV, small-N GEMM), and the
fp64 oracle timed on the host cores as a CPU baseline.  For context it also
times library-independent references the same way: an empty one-element
kernel (the per-launch floor of a graph-replayed kernel) and torch's device
copy of each workload's code plane (its bytes read once and written once).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
COPY_PROBE_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_lm_head_hbm_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "bit_weight_gemv_amd", "csrc", f)
                  for f in ("q4_gemv.hip", "q4_lut.h", "q4_device.h")]


def kernel_source_hash():
    """sha256 of the GEMV's sources with their // comments and blank lines
    removed: an edit of a comment leaves the measured kernel as it was, so
    it does not void the committed counter figures; any code change does."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, encoding="utf-8") as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per lm_head GEMV call from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256") != kernel_source_hash():
            return None
        return int(float(kv["hbm_bytes_per_call"]))
    except (OSError, KeyError, ValueError):
        return None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gemv_bytes(M, K, N=1):
    return M * K // 2 + M * K // 32 + 2 * K * N + 4 * M * N


def _upload_bits(torch, a, dtype, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(dtype)


def prepare(torch, q4, wl, name, dev, copies, n_tokens=None):
    """Generate the seeded workload, pack it on the GPU, replicate it."""
    c = wl.CONFIGS[name]
    M, K = c["M"], c["K"]
    t = time.time()
    W = wl.weights(M, K, c["seed"])
    log(f"{name}: generated W {M}x{K} in {time.time() - t:.1f}s")
    Wd = torch.from_numpy(W).to(dev)
    codes, scales, status = q4.q4_pack(Wd)
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise RuntimeError(f"q4_pack flagged the {name} weights: {int(status.item())}")
    del Wd
    reps = [(codes, scales)]
    for _ in range(copies - 1):
        reps.append((codes.clone(), scales.clone()))
    N = c["N"] if n_tokens is None else n_tokens
    if N == 1:
        xb = wl.activation(K, c["seed"], c["x"])
        x = _upload_bits(torch, xb, torch.bfloat16, dev)
    else:
        xb = wl.activations(N, K, c["seed"], c["x"])
        x = _upload_bits(torch, xb, torch.bfloat16, dev)
    torch.cuda.synchronize()
    return W, xb, reps, x


def time_calls(torch, fn, reps, steps, warmup):
    """Warm up, then time `steps` back-to-back calls (rotating over the
    copies) between two events on the launch stream, with no event or sync
    between the calls.  Returns (wall ms per step, event ms per call)."""
    for i in range(warmup):
        fn(*reps[i % len(reps)])
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        fn(*reps[(warmup + i) % len(reps)])
    end.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    return wall_ms, start.elapsed_time(end) / steps


WARMUP_SECONDS = 0.1


def time_graph(torch, fn, reps, steps, warmup):
    """The timed region: `steps` calls (rotating over the copies) captured once
    in a HIP graph and replayed, bracketed by two events on the replay stream
    and by host synchronisation.  Warm-up replays the same graph until at
    least `warmup` calls and WARMUP_SECONDS have passed.  Returns (event ms per call, wall ms per
    call)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(*reps[0])  # initialise the stream before capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                fn(*reps[i % len(reps)])
        torch.cuda.synchronize()
        # Warm-up: at least `warmup` calls and at least WARMUP_SECONDS of
        # replays (the GPU's clocks take some 20 ms of sustained load to
        # settle; a shorter warm-up times the ramp).
        done, t_w = 0, time.perf_counter()
        while done < max(1, warmup) or time.perf_counter() - t_w < WARMUP_SECONDS:
            g.replay()
            torch.cuda.synchronize()
            done += steps
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record(s)
        g.replay()
        end.record(s)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ms = start.elapsed_time(end) / steps
    del g
    return ms, wall_ms


def secondary_entry(sname, sc, N, g_ms, w_ms):
    sb = gemv_bytes(sc["M"], sc["K"], N)
    gbs = sb / (g_ms * 1e-3) / 1e9
    log(f"{sname} N={N}: {g_ms * 1e3:.2f} us/call, {gbs:.0f} GB/s")
    return {
        "workload": f"{sname} {sc['M']}x{sc['K']} N={N}",
        "us_per_call": round(g_ms * 1e3, 3),
        "us_per_step_wall": round(w_ms * 1e3, 3),
        "achieved_GBs": round(gbs, 1),
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "bytes": sb,
    }


# Fused decode projections (one x, the epilogue in the kernel) against the
# same work unfused (q4_gemv per matrix, then torch's epilogue ops), both
# graph-replayed over rotating copies.  Shapes of a decoder layer with
# hidden 2048, 16 query and 2 key/value heads of 128, MLP width 11008.
FUSED_WORKLOADS = {
    "qkv_bias": dict(Ms=(2048, 256, 256), K=2048, seed=5, x="unit_rms", copies=220),
    "gateup_swiglu": dict(Ms=(11008, 11008), K=2048, seed=2, x="unit_rms", copies=25),
    "down_residual": dict(Ms=(2048,), K=11008, seed=1, x="swiglu", copies=50),
}


def fused_bytes(name, Ms, K):
    w = sum(M * K // 2 + M * K // 32 for M in Ms) + 2 * K
    if name == "qkv_bias":
        return w + sum(8 * M for M in Ms)       # bias read + y written
    if name == "gateup_swiglu":
        return w + 4 * Ms[0]                     # y written
    return w + 8 * Ms[0]                         # residual read + y written


def fused_secondaries(torch, q4, wl, dev, steps, warmup):
    out = []
    for name, fc in FUSED_WORKLOADS.items():
        Ms, K = fc["Ms"], fc["K"]
        W = wl.weights(sum(Ms), K, fc["seed"])
        Wd = torch.from_numpy(W).to(dev)
        codes, scales, status = q4.q4_pack(Wd)
        torch.cuda.synchronize()
        if int(status.item()) != 0:
            raise RuntimeError(f"q4_pack flagged the {name} weights")
        del Wd, W
        reps = [(codes, scales)] + [(codes.clone(), scales.clone()) for _ in range(fc["copies"] - 1)]
        x = _upload_bits(torch, wl.activation(K, fc["seed"], fc["x"]), torch.bfloat16, dev)
        g = torch.Generator(device="cpu").manual_seed(fc["seed"])
        bias = [torch.randn(M, generator=g).to(dev) for M in Ms]
        if name == "gateup_swiglu":
            ys = [torch.empty(Ms[0], device=dev)]
            yu = torch.empty(sum(Ms), device=dev)
        else:
            ys = [torch.empty(M, device=dev) for M in Ms]
        res = torch.randn(Ms[0], generator=g).to(dev)

        def split(cd, sl):
            parts, r0 = [], 0
            for M in Ms:
                parts.append((cd[r0:r0 + M], sl[r0:r0 + M]))
                r0 += M
            return parts

        if name == "qkv_bias":
            def fused(cd, sl):
                q4.q4_gemv_fused([(c, s, b) for (c, s), b in zip(split(cd, sl), bias)], x, "separate", ys)

            def unfused(cd, sl):
                for (c, s), b, y in zip(split(cd, sl), bias, ys):
                    q4.q4_gemv(c, s, x, y)
                    y.add_(b)
        elif name == "gateup_swiglu":
            def fused(cd, sl):
                (cg, sg), (cu, su) = split(cd, sl)
                q4.q4_gemv_fused([(cg, sg, None), (cu, su, None)], x, "swiglu", ys)

            def unfused(cd, sl):
                q4.q4_gemv(cd, sl, x, yu)  # gate and up as one [2M, K] GEMV
                torch.mul(torch.nn.functional.silu(yu[:Ms[0]]), yu[Ms[0]:], out=ys[0])
        else:
            def fused(cd, sl):
                q4.q4_gemv_fused([(cd, sl, None)], x, "separate", ys, [ys[0]])  # residual in place

            def unfused(cd, sl):
                q4.q4_gemv(cd, sl, x, res)
                ys[0].add_(res)
        f_ms, f_wall = time_graph(torch, fused, reps, steps, warmup)
        u_ms, u_wall = time_graph(torch, unfused, reps, steps, warmup)
        nb = fused_bytes(name, Ms, K)
        gbs = nb / (f_ms * 1e-3) / 1e9
        log(f"fused {name}: {f_ms * 1e3:.2f} us/call ({gbs:.0f} GB/s), unfused {u_ms * 1e3:.2f} us")
        out.append({
            "workload": f"fused {name} Ms={'+'.join(map(str, Ms))} K={K} N=1",
            "us_per_call": round(f_ms * 1e3, 3),
            "us_per_step_wall": round(f_wall * 1e3, 3),
            "achieved_GBs": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "bytes": nb,
            "unfused_us_per_call": round(u_ms * 1e3, 3),
            "speedup_vs_unfused": round(u_ms / f_ms, 3),
        })
        del reps, x, bias, ys, res
        torch.cuda.empty_cache()
    return out


PAGES_TABLE = os.path.join(ROOT, "tests", "golden", "decode_v2_linear_bench.tsv")
COLD_BYTES = 640 << 20   # rotated copies per shape: past the 256 MB Infinity Cache


def pages_table():
    """The per-launch GEMV bench table of the deep-fold "Decode V2" page
    (section 6): kind, M, K, median us and GB/s on the page's consumer NVIDIA
    card, as transcribed in the golden fixture."""
    rows = []
    with open(PAGES_TABLE) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                kind, M, K, us, gbs = line.split("\t")
                rows.append((kind, int(M), int(K), float(us), float(gbs)))
    return rows


def pages_secondaries(torch, q4, wl, dev, steps, warmup):
    """The GEMV on every shape of the page's bench table (but lm_head, the
    headline): W ~ N(0, 0.02^2) seeded per shape, x unit-RMS (SwiGLU-like for
    the down projections, K of 11008 or 27648), enough packed copies (views
    of one buffer) that the timed graph reads past the Infinity Cache; the
    graph holds at least one call per copy.  The page's own figures ride
    along as context (other hardware, their GB/s omits y)."""
    out = []
    for i, (kind, M, K, p_us, p_gbs) in enumerate(pages_table()):
        if kind == "lm_head":
            continue
        seed = 100 + i
        W = torch.from_numpy(wl.weights(M, K, seed)).to(dev)
        codes, scales, status = q4.q4_pack(W)
        torch.cuda.synchronize()
        del W
        if int(status.item()) != 0:
            raise RuntimeError(f"q4_pack flagged the {kind} weights")
        wbytes = codes.numel() + 2 * scales.numel()
        R = max(1, min(4096, -(-COLD_BYTES // wbytes)))
        big_c = torch.empty((R,) + tuple(codes.shape), dtype=codes.dtype, device=dev)
        big_s = torch.empty((R,) + tuple(scales.shape), dtype=scales.dtype, device=dev)
        big_c[:] = codes
        big_s[:] = scales
        del codes, scales
        reps = [(big_c[r], big_s[r]) for r in range(R)]
        x = _upload_bits(torch, wl.activation(K, seed, "swiglu" if K in (11008, 27648) else "unit_rms"),
                         torch.bfloat16, dev)
        y = torch.empty(M, dtype=torch.float32, device=dev)

        def fn(cd, sl, x=x, y=y):
            q4.q4_gemv(cd, sl, x, y)
        n_calls = max(steps, R)
        ms, wall = time_graph(torch, fn, reps, n_calls, warmup)
        nb = gemv_bytes(M, K)
        pb = nb - 4 * M  # the page's convention: packed + scale + x
        log(f"pages {kind} {M}x{K}: {ms * 1e3:.2f} us/call, {nb / (ms * 1e-3) / 1e9:.0f} GB/s "
            f"(page: {p_us} us, {p_gbs} GB/s)")
        out.append({"workload": f"pages table {kind} {M}x{K} N=1", "us_per_call": round(ms * 1e3, 3),
                    "us_per_step_wall": round(wall * 1e3, 3), "bytes": nb,
                    "achieved_GBs": round(nb / (ms * 1e-3) / 1e9, 1),
                    "frac_of_hbm_peak": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "pages_convention_GBs": round(pb / (ms * 1e-3) / 1e9, 1),
                    "copies_rotated": R, "calls_per_graph": n_calls,
                    "page_us": p_us, "page_GBs": p_gbs,
                    "page_hardware": "consumer NVIDIA card of the page's lab log (context only)"})
        del reps, big_c, big_s, x, y
        torch.cuda.empty_cache()
    return out


def gather_secondaries(torch, q4, wl, dev, steps, warmup):
    """The packed row gather on the tied-embedding table (the lm_head matrix,
    151936 x 2048): one decode token and a 32-token chunk, fp32 and bf16
    rows; ids drawn afresh for every call from a seeded stream."""
    c = wl.CONFIGS["lm_head"]
    M, K = c["M"], c["K"]
    W = torch.from_numpy(wl.weights(M, K, c["seed"])).to(dev)
    codes, scales, status = q4.q4_pack(W)
    torch.cuda.synchronize()
    del W
    torch.cuda.empty_cache()
    g = torch.Generator(device="cpu").manual_seed(9)
    out = []
    for n in (1, 32):
        idsets = [(torch.randint(0, M, (n,), generator=g, dtype=torch.int32).to(dev),) for _ in range(64)]
        for dt, name, elt in ((torch.float32, "f32", 4), (torch.bfloat16, "bf16", 2)):
            o = torch.empty((n, K), dtype=dt, device=dev)
            st = torch.empty(1, dtype=torch.int32, device=dev)

            def fn(ids, o=o, st=st):
                q4.q4_gather_rows(codes, scales, ids, dt, o, st)
            ms, wall = time_graph(torch, fn, idsets, steps, warmup)
            nb = n * (K // 2 + K // 32 + 4) + n * K * elt
            log(f"gather {name} n={n}: {ms * 1e3:.2f} us/call")
            out.append({"workload": f"gather rows of the tied lm_head table {M}x{K}, n={n}, out {name}",
                        "us_per_call": round(ms * 1e3, 3), "us_per_step_wall": round(wall * 1e3, 3),
                        "bytes": nb, "achieved_GBs": round(nb / (ms * 1e-3) / 1e9, 2)})
    del codes, scales
    torch.cuda.empty_cache()
    return out


def affine_secondaries(torch, q4, wl, dev, steps, warmup):
    """The affine format's GEMV ((code - z) * s per 64-block, one more fp16
    plane than NF4) on the lm_head and down shapes."""
    out = []
    for name, copies in (("lm_head", 4), ("down", 50)):
        c = wl.CONFIGS[name]
        M, K = c["M"], c["K"]
        W = torch.from_numpy(wl.weights(M, K, c["seed"])).to(dev)
        codes, scales, zeros, status = q4.q4_pack_affine(W)
        torch.cuda.synchronize()
        if int(status.item()) != 0:
            raise RuntimeError(f"q4_pack_affine flagged the {name} weights")
        del W
        reps = [(codes, scales, zeros)] + [(codes.clone(), scales.clone(), zeros.clone()) for _ in range(copies - 1)]
        x = _upload_bits(torch, wl.activation(K, c["seed"], c["x"]), torch.bfloat16, dev)
        y = torch.empty(M, dtype=torch.float32, device=dev)

        def fn(cd, sl, zr):
            q4.q4_gemv_affine(cd, sl, zr, x, y)
        ms, wall = time_graph(torch, fn, reps, steps, warmup)
        nb = gemv_bytes(M, K) + M * K // 32
        gbs = nb / (ms * 1e-3) / 1e9
        log(f"affine {name}: {ms * 1e3:.2f} us/call, {gbs:.0f} GB/s")
        out.append({"workload": f"affine-format GEMV {name} {M}x{K} N=1", "us_per_call": round(ms * 1e3, 3),
                    "us_per_step_wall": round(wall * 1e3, 3), "achieved_GBs": round(gbs, 1),
                    "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "bytes": nb})
        del reps, codes, scales, zeros, x, y
        torch.cuda.empty_cache()
    # The prefill product on the prefill shape (11008 x 2048), chunks of 32,
    # 16, 8, 4 and 2 tokens.
    c = wl.CONFIGS["smalln"]
    M, K = c["M"], c["K"]
    W = torch.from_numpy(wl.weights(M, K, c["seed"])).to(dev)
    codes, scales, zeros, status = q4.q4_pack_affine(W)
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise RuntimeError("q4_pack_affine flagged the prefill weights")
    del W
    reps = [(codes, scales, zeros)] + [(codes.clone(), scales.clone(), zeros.clone()) for _ in range(44)]
    X = _upload_bits(torch, wl.activations(32, K, c["seed"], c["x"]), torch.bfloat16, dev)
    for n in (32, 16, 8, 4, 2):
        Xn = X[:n].contiguous()
        Y = torch.empty((n, M), dtype=torch.float32, device=dev)

        def fn(cd, sl, zr, Xn=Xn, Y=Y):
            q4.q4_gemm_smalln_affine(cd, sl, zr, Xn, Y)
        ms, wall = time_graph(torch, fn, reps, steps, warmup)
        nb = gemv_bytes(M, K, n) + M * K // 32
        log(f"affine prefill N={n}: {ms * 1e3:.2f} us/call")
        out.append({"workload": f"affine-format prefill {M}x{K} N={n}", "us_per_call": round(ms * 1e3, 3),
                    "us_per_step_wall": round(wall * 1e3, 3), "achieved_GBs": round(nb / (ms * 1e-3) / 1e9, 1),
                    "bytes": nb})
    del reps, codes, scales, zeros, X
    torch.cuda.empty_cache()
    return out


def fused_format_secondaries(torch, q4, wl, dev, steps, warmup, fmt):
    """The fused decode projections of the affine or NVFP4-style format: the
    gate/up pair with the SwiGLU epilogue (2 x 11008 x 2048, each matrix
    packed on its own) and down with the residual added in place
    (2048 x 11008), each against its unfused form (the format's GEMV per
    matrix, then torch's epilogue)."""
    out = []
    pack = q4.q4_pack_affine if fmt == "affine" else q4.q4_pack_nvfp4
    gemv = q4.q4_gemv_affine if fmt == "affine" else q4.q4_gemv_nvfp4
    fused = q4.q4_gemv_fused_affine if fmt == "affine" else q4.q4_gemv_fused_nvfp4
    label = "affine-format" if fmt == "affine" else "NVFP4-style"
    for name, Ms, K, copies, seed in (("gateup_swiglu", (11008, 11008), 2048, 25, 71),
                                      ("down_residual", (2048,), 11008, 50, 72)):
        mats = []
        for i, M in enumerate(Ms):
            Wd = torch.from_numpy(wl.weights(M, K, seed + i)).to(dev)
            *planes, status = pack(Wd)
            torch.cuda.synchronize()
            if int(status.item()) != 0:
                raise RuntimeError(f"{label} pack flagged the {name} weights")
            mats.append(tuple(planes))
            del Wd
        reps = [tuple(mats)] + [tuple(tuple(p.clone() for p in m) for m in mats) for _ in range(copies - 1)]
        x = _upload_bits(torch, wl.activation(K, seed, "unit_rms"), torch.bfloat16, dev)
        y = torch.empty(Ms[0], dtype=torch.float32, device=dev)
        tmp = [torch.empty(M, dtype=torch.float32, device=dev) for M in Ms]
        if name == "gateup_swiglu":
            def f(*ms):
                fused([m + (None,) for m in ms], x, "swiglu", [y])

            def u(*ms):
                for m, t in zip(ms, tmp):
                    gemv(*m, x, t)
                torch.mul(torch.nn.functional.silu(tmp[0]), tmp[1], out=y)
        else:
            def f(*ms):
                fused([ms[0] + (None,)], x, "separate", [y], [y])  # residual in place

            def u(*ms):
                gemv(*ms[0], x, tmp[0])
                y.add_(tmp[0])
        f_ms, f_wall = time_graph(torch, f, reps, steps, warmup)
        u_ms, _ = time_graph(torch, u, reps, steps, warmup)
        per_row = (K // 2 + K // 16 + 0) if fmt == "nvfp4" else (K // 2 + 2 * (K // 32))
        nb = sum(Ms) * per_row + (4 * len(Ms) if fmt == "nvfp4" else 0) + 2 * K + 4 * Ms[0] + (
            4 * Ms[0] if name == "down_residual" else 0)
        gbs = nb / (f_ms * 1e-3) / 1e9
        log(f"{fmt} fused {name}: {f_ms * 1e3:.2f} us/call ({gbs:.0f} GB/s), unfused {u_ms * 1e3:.2f} us")
        out.append({"workload": f"{label} fused {name} Ms={'+'.join(map(str, Ms))} K={K} N=1",
                    "us_per_call": round(f_ms * 1e3, 3), "us_per_step_wall": round(f_wall * 1e3, 3),
                    "achieved_GBs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "bytes": nb,
                    "unfused_us_per_call": round(u_ms * 1e3, 3), "speedup_vs_unfused": round(u_ms / f_ms, 3)})
        del reps, mats, x, y, tmp
        torch.cuda.empty_cache()
    return out


def nvfp4_secondaries(torch, q4, wl, dev, steps, warmup):
    """The NVFP4-style format's GEMV (E2M1 codes, an E4M3 scale per 16
    weights, an f32 tensor scale) on the lm_head and down shapes."""
    out = []
    for name, copies in (("lm_head", 4), ("down", 50)):
        c = wl.CONFIGS[name]
        M, K = c["M"], c["K"]
        W = torch.from_numpy(wl.weights(M, K, c["seed"])).to(dev)
        codes, scales, ts, status = q4.q4_pack_nvfp4(W)
        torch.cuda.synchronize()
        if int(status.item()) != 0:
            raise RuntimeError(f"q4_pack_nvfp4 flagged the {name} weights")
        del W
        reps = [(codes, scales)] + [(codes.clone(), scales.clone()) for _ in range(copies - 1)]
        x = _upload_bits(torch, wl.activation(K, c["seed"], c["x"]), torch.bfloat16, dev)
        y = torch.empty(M, dtype=torch.float32, device=dev)

        def fn(cd, sl):
            q4.q4_gemv_nvfp4(cd, sl, ts, x, y)
        ms, wall = time_graph(torch, fn, reps, steps, warmup)
        nb = M * K // 2 + M * K // 16 + 4 + 2 * K + 4 * M
        gbs = nb / (ms * 1e-3) / 1e9
        log(f"nvfp4 {name}: {ms * 1e3:.2f} us/call, {gbs:.0f} GB/s")
        out.append({"workload": f"NVFP4-style GEMV {name} {M}x{K} N=1", "us_per_call": round(ms * 1e3, 3),
                    "us_per_step_wall": round(wall * 1e3, 3), "achieved_GBs": round(gbs, 1),
                    "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "bytes": nb})
        del reps, codes, scales, ts, x, y
        torch.cuda.empty_cache()
    # The prefill product on the prefill shape (11008 x 2048), chunks of 32,
    # 16, 8, 4 and 2 tokens.
    c = wl.CONFIGS["smalln"]
    M, K = c["M"], c["K"]
    W = torch.from_numpy(wl.weights(M, K, c["seed"])).to(dev)
    codes, scales, ts, status = q4.q4_pack_nvfp4(W)
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise RuntimeError("q4_pack_nvfp4 flagged the prefill weights")
    del W
    reps = [(codes, scales)] + [(codes.clone(), scales.clone()) for _ in range(44)]
    X = _upload_bits(torch, wl.activations(32, K, c["seed"], c["x"]), torch.bfloat16, dev)
    for n in (32, 16, 8, 4, 2):
        Xn = X[:n].contiguous()
        Y = torch.empty((n, M), dtype=torch.float32, device=dev)

        def fn(cd, sl, Xn=Xn, Y=Y):
            q4.q4_gemm_smalln_nvfp4(cd, sl, ts, Xn, Y)
        ms, wall = time_graph(torch, fn, reps, steps, warmup)
        nb = M * K // 2 + M * K // 16 + 4 + 2 * K * n + 4 * M * n
        log(f"nvfp4 prefill N={n}: {ms * 1e3:.2f} us/call")
        out.append({"workload": f"NVFP4-style prefill {M}x{K} N={n}", "us_per_call": round(ms * 1e3, 3),
                    "us_per_step_wall": round(wall * 1e3, 3), "achieved_GBs": round(nb / (ms * 1e-3) / 1e9, 1),
                    "bytes": nb})
    del reps, codes, scales, ts, X
    torch.cuda.empty_cache()
    return out


def x8_secondaries(torch, q4, wl, dev, steps, warmup):
    """The affine format's GEMV on int8 activations (one and two words) on
    the lm_head shape; the activation quantisation timed as its own call."""
    out = []
    c = wl.CONFIGS["lm_head"]
    M, K = c["M"], c["K"]
    W = torch.from_numpy(wl.weights(M, K, c["seed"])).to(dev)
    codes, scales, zeros, status = q4.q4_pack_affine(W)
    torch.cuda.synchronize()
    del W
    reps = [(codes, scales, zeros)] + [(codes.clone(), scales.clone(), zeros.clone()) for _ in range(3)]
    x = _upload_bits(torch, wl.activation(K, c["seed"], c["x"]), torch.bfloat16, dev)
    y = torch.empty(M, dtype=torch.float32, device=dev)
    for words in (1, 2):
        q1, q2, d = q4.q4_quantize_x8(x, words)

        def fn(cd, sl, zr, q1=q1, q2=q2, d=d):
            q4.q4_gemv_affine_x8(cd, sl, zr, q1, q2, d, y)
        ms, wall = time_graph(torch, fn, reps, steps, warmup)
        nb = gemv_bytes(M, K) + M * K // 32 - 2 * K + K * words + K // 8
        gbs = nb / (ms * 1e-3) / 1e9
        log(f"affine x8 ({words} word) lm_head: {ms * 1e3:.2f} us/call, {gbs:.0f} GB/s")
        out.append({"workload": f"affine-format GEMV on int8 activations ({words} word) lm_head {M}x{K} N=1",
                    "us_per_call": round(ms * 1e3, 3), "us_per_step_wall": round(wall * 1e3, 3),
                    "achieved_GBs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "bytes": nb})

        def qfn(xx, words=words, q1=q1, q2=q2, d=d):
            q4.q4_quantize_x8(xx, words, q1, q2, d)
        qms, qwall = time_graph(torch, qfn, [(x,)], steps, warmup)
        log(f"quantize x8 ({words} word) K={K}: {qms * 1e3:.2f} us/call")
        out.append({"workload": f"activation quantisation to int8 ({words} word) K={K}",
                    "us_per_call": round(qms * 1e3, 3), "us_per_step_wall": round(qwall * 1e3, 3)})
    del reps, codes, scales, zeros, x, y
    torch.cuda.empty_cache()
    return out


def context_bandwidth(torch, dev, steps=20):
    """Bandwidth context from a library-independent kernel: torch's device
    copy of COPY_PROBE_BYTES, replayed as a graph; (read + written bytes) / s
    in GB/s."""
    src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dsts = [torch.empty_like(src) for _ in range(2)]

    def cp(d):
        d.copy_(src)
    ms, _ = time_graph(torch, cp, [(d,) for d in dsts], steps, 2)
    del src, dsts
    torch.cuda.empty_cache()
    return 2 * COPY_PROBE_BYTES / (ms * 1e-3) / 1e9


def code_plane_copy_us(torch, reps, steps, warmup):
    """Bandwidth context from a library-independent kernel: torch's device
    copy of the same code plane (every byte read once and written once, so
    twice the GEMV's code bytes), graph-replayed over the same rotating
    copies, each into a destination of its own; microseconds per call."""
    pairs = [(cd, torch.empty_like(cd)) for cd, _ in reps]

    def cp(cd, dst):
        dst.copy_(cd)
    ms, _ = time_graph(torch, cp, pairs, steps, warmup)
    del pairs
    return ms * 1e3


_FLOOR_LIB = None
FLOOR_GRIDS = ((256, 256), (512, 256), (1024, 256), (2048, 256), (4096, 256), (1024, 512), (2048, 512))


def read_floor_us(torch, reps, steps, warmup):
    """The plain streaming read of the same bytes (each copy's code plane and
    scale plane once, no arithmetic; libq4floor.so, a reference kernel kept
    out of libq4), graph-replayed over the same rotating copies; the best of
    a sweep of grid shapes.  Returns (microseconds per call, grid, block)."""
    import ctypes
    global _FLOOR_LIB
    if _FLOOR_LIB is None:
        from bit_weight_gemv_amd import build as b
        if not os.path.exists(b.FLOOR_LIB):
            raise RuntimeError("libq4floor.so not built; run python -m bit_weight_gemv_amd.build")
        L = ctypes.CDLL(b.FLOOR_LIB)
        L.q4floor_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint64,
                                   ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        L.q4floor_read.restype = ctypes.c_int
        _FLOOR_LIB = L
    out = torch.zeros(256, dtype=torch.int32, device=reps[0][0].device)
    best = None
    for grid, block in FLOOR_GRIDS:
        def rd(cd, sl, grid=grid, block=block):
            rc = _FLOOR_LIB.q4floor_read(cd.data_ptr(), cd.numel() * cd.element_size(), sl.data_ptr(),
                                         sl.numel() * sl.element_size(), out.data_ptr(), grid, block,
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if rc != 0:
                raise RuntimeError(f"q4floor_read returned {rc}")
        ms, _ = time_graph(torch, rd, reps, steps, warmup)
        if best is None or ms < best[0]:
            best = (ms, grid, block)
    return best[0] * 1e3, best[1], best[2]


def empty_kernel_us(torch, dev, steps, warmup):
    """Launch floor: one one-element torch kernel per call, graph-replayed."""
    t = torch.zeros(1, device=dev)

    def one(_):
        t.add_(1.0)
    ms, _ = time_graph(torch, one, [(None,)], steps, warmup)
    return ms * 1e3


def cpu_info():
    """The host CPU as /proc/cpuinfo describes it: the model string plus the
    vendor, family / model / stepping numbers, clock and cache fields (a
    virtualised host may print a short model string), and the CPU counts."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" not in line:
                    if fields:
                        break  # the first processor's block is enough
                    continue
                k, v = (t.strip() for t in line.split(":", 1))
                if k in ("model name", "vendor_id", "cpu family", "model", "stepping", "cpu MHz",
                         "cache size", "siblings", "cpu cores") and k not in fields:
                    fields[k] = v
    except OSError:
        pass
    desc = fields.get("model name")
    extra = ", ".join(f"{k} {fields[k]}" for k in ("vendor_id", "cpu family", "model", "stepping",
                                                    "cpu MHz", "cache size") if k in fields)
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"cpu_model": desc, "cpu_detail": extra or None, "host_logical_cpus": os.cpu_count(),
            "affinity_cpus": affinity}


def cpu_threads():
    """Threads for the oracle: every CPU this process may run on, or the
    CPU share the environment grants when OMP_NUM_THREADS names a smaller one
    (on a shared GPU host that is the share of one GPU)."""
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and 0 < int(share) < aff:
        return int(share), f"OMP_NUM_THREADS={share} (the CPU share granted to this process)"
    return aff, "every CPU in the process's affinity mask"


def cpu_baseline(oracle, wl, W, xb, name):
    """The oracle's fp64 GEMV over the whole matrix on the host cores, as it
    stands: rows split over T threads (T = the CPUs granted to the process),
    repeated for about 10 s, median; and the same call on one thread, median
    of three (identical sums: rows are only split)."""
    c = wl.CONFIGS[name]
    M, K = c["M"], c["K"]
    threads, why = cpu_threads()
    codes, scales, st = oracle.pack(W, threads=threads)
    assert st == 0
    times = []
    y_ref = S = None
    t_start = time.time()
    while True:
        t = time.perf_counter()
        y_ref, S = oracle.gemv(codes, scales, M, K, xb, threads=threads)
        times.append(time.perf_counter() - t)
        if time.time() - t_start > 10.0 or len(times) >= 400:
            break
    sec = float(np.median(times))
    t1 = []
    for _ in range(3):
        t = time.perf_counter()
        oracle.gemv(codes, scales, M, K, xb, threads=1)
        t1.append(time.perf_counter() - t)
    sec1 = float(np.median(t1))
    out = {
        "value": round(gemv_bytes(M, K) / sec / 1e9, 3),
        "unit": "GB/s",
        "us_per_call": round(sec * 1e6, 1),
        "cores": threads,
        "threads_rule": why,
        "value_1_thread": round(gemv_bytes(M, K) / sec1 / 1e9, 4),
        "us_per_call_1_thread": round(sec1 * 1e6, 1),
        "kind": "oracle",
        "sample": f"full {name} GEMV {M}x{K} (fp64 oracle, rows split over {threads} threads), "
                  f"{len(times)} calls in {time.time() - t_start:.1f}s, median; one thread: median of 3",
    }
    out.update(cpu_info())
    return out, y_ref, S


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=4)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--secondary", default="tiny,down,smalln,gateup,prefill_down,fused,gather,affine,nvfp4,x8,pages",
                    help="comma-separated secondary workloads to time "
                         "(tiny, down, smalln, gateup, prefill_down, fused, gather, affine, nvfp4, x8, pages)")
    ap.add_argument("--eager", action="store_true",
                    help="also time the calls launched one by one from Python")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run 3 plain 256 MiB device copies first (calibrates rocprofv3 "
                         "FETCH_SIZE/WRITE_SIZE against a copy of known size)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the path is measured on one MI355X; "
              f"--gpus {args.gpus} is not supported (row-sharded multi-GPU use is a design note, not built).",
              flush=True)
        sys.exit(2)

    import torch

    import bit_weight_gemv_amd as q4
    import workloads as wl

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    q4.lib()

    if args.copy_probe:
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy probe: 3 x {COPY_PROBE_BYTES} B device copies")

    name = "lm_head"
    c = wl.CONFIGS[name]
    M, K = c["M"], c["K"]
    W, xb, reps, x = prepare(torch, q4, wl, name, dev, args.copies)
    y = torch.empty(M, dtype=torch.float32, device=dev)

    def step(codes, scales):
        q4.q4_gemv(codes, scales, x, y)

    k_mean_ms, wall_ms = time_graph(torch, step, reps, args.steps, args.warmup)
    eager = None
    if args.eager:
        e_wall, e_ms = time_calls(torch, step, reps, args.steps, args.warmup)
        eager = {"us_per_call_events": round(e_ms * 1e3, 3), "us_per_step_wall": round(e_wall * 1e3, 3)}
    nbytes = gemv_bytes(M, K)
    value = nbytes / (wall_ms * 1e-3) / 1e9
    achieved = nbytes / (k_mean_ms * 1e-3) / 1e9
    log(f"lm_head: {k_mean_ms * 1e3:.2f} us/call (events), {wall_ms * 1e3:.2f} us/step (wall), "
        f"{achieved:.0f} GB/s" + (f"; eager {eager}" if eager else ""))

    # y of the last call for the argmax check against the oracle
    q4.q4_gemv(reps[0][0], reps[0][1], x, y)
    y_gpu = y.cpu().numpy()
    floors = None
    if not args.no_secondary:
        rf_us, rf_grid, rf_block = read_floor_us(torch, reps, args.steps, args.warmup)
        floors = {"empty_kernel_us": round(empty_kernel_us(torch, dev, args.steps, args.warmup), 3),
                  "lm_head_code_plane_copy_us": round(code_plane_copy_us(torch, reps, args.steps, args.warmup), 3),
                  "lm_head_read_floor_us": round(rf_us, 3),
                  "lm_head_read_floor_grid": f"{rf_grid}x{rf_block}",
                  "lm_head_gemv_over_read_floor": round(k_mean_ms * 1e3 / rf_us, 4)}
        log(f"floors: {floors}")

    secondary = []
    if not args.no_secondary:
        del reps
        torch.cuda.empty_cache()
        chosen = [n.strip() for n in args.secondary.split(",") if n.strip()]
        # tiny (256 x 512, 72 KB) stays in cache and is launch-bound: one copy,
        # timed for its microseconds only.
        # prefill_down: the prefill sweep on the down projection's shape
        # (rows of 11008 weights), through q4_gemm_smalln_ws with scratch
        # memory for the K split (allocated once, outside the timed region).
        for sname, cname, ncopies, ntok in (("tiny", "tiny", 1, None), ("down", "down", 50, None),
                                            ("smalln", "smalln", 45, 32), ("gateup", "gateup", 25, None),
                                            ("prefill_down", "down", 50, 32)):
            if sname not in chosen:
                continue
            sc = wl.CONFIGS[cname]
            _, _, sreps, sx = prepare(torch, q4, wl, cname, dev, ncopies, n_tokens=ntok)
            if ntok is None:
                sy = torch.empty(sc["M"], dtype=torch.float32, device=dev)

                def sstep(cd, sl, sx=sx, sy=sy):
                    q4.q4_gemv(cd, sl, sx, sy)
                N = 1
            else:
                sy = torch.empty((ntok, sc["M"]), dtype=torch.float32, device=dev)
                sws = q4.gemm_workspace(sc["M"], sc["K"], ntok, dev) if sname == "prefill_down" else None

                def sstep(cd, sl, sx=sx, sy=sy, sws=sws):
                    if sname == "prefill_down":
                        q4.q4_gemm_smalln_ws(cd, sl, sx, sws, sy)
                    else:
                        q4.q4_gemm_smalln(cd, sl, sx, sy)
                N = ntok
            sg, sw = time_graph(torch, sstep, sreps, args.steps, args.warmup)
            secondary.append(secondary_entry(sname, sc, N, sg, sw))
            secondary[-1]["code_plane_copy_us"] = round(code_plane_copy_us(torch, sreps, args.steps, args.warmup), 3)
            rf_us, rf_grid, rf_block = read_floor_us(torch, sreps, args.steps, args.warmup)
            secondary[-1]["read_floor_us"] = round(rf_us, 3)
            secondary[-1]["read_floor_grid"] = f"{rf_grid}x{rf_block}"
            secondary[-1]["over_read_floor"] = round(sg * 1e3 / rf_us, 4)
            log(f"{sname}: read floor {rf_us:.2f} us ({rf_grid}x{rf_block})")
            if ntok is not None:
                # The prefill sweep: the first n tokens of the same chunk.
                for n in ((16, 8, 4, 2, 1) if sname == "smalln" else (16, 8, 4, 3, 2)):
                    sxn = sx[:n].contiguous()
                    syn = torch.empty((n, sc["M"]), dtype=torch.float32, device=dev)

                    def nstep(cd, sl, sxn=sxn, syn=syn, sws=sws):
                        if sname == "prefill_down":
                            q4.q4_gemm_smalln_ws(cd, sl, sxn, sws, syn)
                        else:
                            q4.q4_gemm_smalln(cd, sl, sxn, syn)
                    ng, nw = time_graph(torch, nstep, sreps, args.steps, args.warmup)
                    secondary.append(secondary_entry(sname, sc, n, ng, nw))
                    del sxn, syn
            del sreps, sx, sy
            if ntok is not None:
                del sws
            torch.cuda.empty_cache()
        if "fused" in chosen:
            secondary.extend(fused_secondaries(torch, q4, wl, dev, args.steps, args.warmup))
        if "gather" in chosen:
            secondary.extend(gather_secondaries(torch, q4, wl, dev, args.steps, args.warmup))
        if "affine" in chosen:
            secondary.extend(affine_secondaries(torch, q4, wl, dev, args.steps, args.warmup))
            secondary.extend(fused_format_secondaries(torch, q4, wl, dev, args.steps, args.warmup, "affine"))
        if "nvfp4" in chosen:
            secondary.extend(nvfp4_secondaries(torch, q4, wl, dev, args.steps, args.warmup))
            secondary.extend(fused_format_secondaries(torch, q4, wl, dev, args.steps, args.warmup, "nvfp4"))
        if "x8" in chosen:
            secondary.extend(x8_secondaries(torch, q4, wl, dev, args.steps, args.warmup))
        if "pages" in chosen:
            secondary.extend(pages_secondaries(torch, q4, wl, dev, args.steps, args.warmup))

    result = {
        "metric": "4-bit GEMV us/call + achieved HBM GB/s (% of peak), MxK=151936x2048, N=1",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "us_per_call": round(k_mean_ms * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "dtype_note": "fp16 table, fp32 accumulate: 4-bit codes; levels held as fp16 (rounded by at most "
                      "2^-11 relative); bf16 x converted exactly to fp16 under a power of two (or widened to "
                      "fp32 when a wave's activations span more than 2^28); products exact in "
                      "v_dot2_f32_f16; sums in fp32. A reading of the page's 'FP32 LUT x scale x x' that "
                      "stays inside the acceptance bound by proof",
        "data": "synthetic (seeded SplitMix64 normals; W ~ N(0, 0.02^2), x unit-RMS bf16)",
        "config": {"workload": "lm_head GEMV 151936x2048, N=1", "M": M, "K": K, "N": 1,
                   "copies_rotated": args.copies, "bytes_per_call": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": "q4::gemv_kernel<4,1,0,4,false,true,true,false>",
                     "kernel_us": round(k_mean_ms * 1e3, 3),
                     "timing": "HIP graph of the timed calls, events on the replay stream"},
        "eager": eager,
        "secondary": secondary,
        "machine": {"gpu": torch.cuda.get_device_name(dev), "hip": torch.version.hip,
                    "torch": torch.__version__},
    }
    if not args.no_secondary:
        copy_gbs = context_bandwidth(torch, dev)
        log(f"context: torch device copy {copy_gbs:.0f} GB/s (read + written)")
        result["context"] = {
            "torch_copy_GBs": round(copy_gbs, 1),
            "lm_head_over_torch_copy": round(achieved / copy_gbs, 4),
            "how": f"torch's {COPY_PROBE_BYTES >> 20} MiB device-to-device copy, graph-replayed",
            "floors": floors,
            "floors_how": "empty_kernel_us: a one-element torch kernel per call (the launch floor); "
                          "*code_plane_copy_us (also per secondary workload): torch's device copy of the "
                          "same code plane (its bytes read and written once each); *read_floor_us (also "
                          "per secondary workload): libq4floor.so's plain streaming read of the code and "
                          "scale planes, best of a sweep of grid shapes; all graph-replayed over the same "
                          "rotating copies"}
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        cb, y_ref, S = cpu_baseline(oracle, wl, W, xb, name)
        result["cpu_baseline"] = cb
        ok, ratio = oracle.within_tolerance(y_gpu, y_ref, S)
        top2 = np.sort(y_ref)[-2:]
        result["parity"] = {"within_tolerance": ok, "worst_ratio": round(ratio, 4),
                            "argmax_gpu": oracle.argmax(y_gpu), "argmax_oracle": oracle.argmax(y_ref),
                            "top2_gap_oracle": float(top2[1] - top2[0])}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
