"""Benchmark: fp16 NT GEMM (fp32 accumulation) at M = N = K = 8192 on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --pmc-pass        # short run for rocprofv3 --pmc counter passes
    python bench.py --vendor-sweep    # fp16 -> fp16 products against torch.mm, one JSON line

A step is one gemm_nt_f16f32 launch over the 8192^3 synthetic workload
(A, B ~ normal(0,1) * 0.1 rounded to fp16, seed 4), inputs resident in HBM.
W untimed steps, then exactly K timed steps between two device
synchronisations; one JSON line on stdout.

Besides the headline, the same line carries:
  roofline      the GEMM kernel against the dense fp16 MFMA peak, its
                duration from HIP events recorded on the launch stream, and the
                L2-miss traffic measured with rocprofv3 counters when the committed
                summary matches the current kernel source;
  cpu_baseline  the CPU oracle (numpy float64) on a bounded row sample of the
                same workload, timed on this host;
  step_us       every timed launch's own duration (HIP events between the
                launches), so that a clock still ramping up under a short
                warm-up shows in the record;
  secondary     frag_copy (2^20 tiles, every num / layout / direction) in GB/s
                against HBM bandwidth, cold (three rotating buffer sets, more
                than the 256 MB last-level cache holds) and warm (one set
                reused), the batched 4096 x (128x64x64) product and the
                16384x8x16384 skinny product (cold and warm), the single
                16x8x16 tile and 128x64x64 workgroup (us per call), the
                8192^3 launch with other types and storage orders, and two
                ceilings from bench_ceiling.hip: the MFMA pipe alone on the
                workload's operand values and on zeros, and a plain copy of
                frag_copy's size.
"""

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fp16 NT GEMM TFLOP/s (fp32 acc) at 8192^3; % of MFMA fp16 peak"
PEAK_TFLOPS = 2516.6       # MI355X dense fp16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
GEMM_SOURCES = ["fp16_matrix_core_amd/csrc/gemm_kernels.hpp", "fp16_matrix_core_amd/csrc/gemm_nt.hip",
                "fp16_matrix_core_amd/csrc/layout.hpp", "fp16_matrix_core_amd/csrc/kernels.hpp"]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_nt_8192_l2_miss_traffic.txt")
CEILING_LIB = os.path.join(ROOT, "libbench_ceiling.so")
PMC_GEMM_LAUNCHES = 30     # counter passes: launches of the 8192^3 product ...
PMC_MFMA_LAUNCHES = 6      # ... and of the MFMA-only loop


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_source_hash():
    """Hash of the GEMM kernel sources with comments and whitespace removed, so that
    the counter summary stays matched to the kernel across comment-only edits."""
    import re
    h = hashlib.sha256()
    for p in GEMM_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel_hash):
    """L2-miss bytes per launch from the committed counter summary, if it matches this kernel source."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    kv = {}
    for line in open(TRAFFIC_SUMMARY):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != kernel_hash:
        return None
    try:
        return float(kv["l2_miss_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class StreamTimer:
    """HIP events recorded on the stream the kernels are launched on."""

    def __init__(self, torch, stream):
        self.torch = torch
        self.stream = stream

    def time(self, fn, reps):
        t = self.torch
        start = t.cuda.Event(enable_timing=True)
        end = t.cuda.Event(enable_timing=True)
        start.record(self.stream)
        for _ in range(reps):
            fn()
        end.record(self.stream)
        end.synchronize()
        return start.elapsed_time(end) / reps      # ms per call


def cpu_baseline(A, B, target_s=10.0):
    """The oracle (float64 numpy: ref and bound) on a row sample of the 8192^3 workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:                                   # threadpoolctl missing: report affinity
        threads = len(os.sched_getaffinity(0))
    N, K = B.shape
    rows = 256
    oracle.gemm_nt_rows(A, B, np.arange(rows))          # warm the BLAS threads
    t0 = time.perf_counter()
    oracle.gemm_nt_rows(A, B, np.arange(rows))
    dt = time.perf_counter() - t0
    rows = int(min(A.shape[0], rows * target_s / max(dt, 1e-3)))
    rows = max(256, rows - rows % 256)
    t0 = time.perf_counter()
    oracle.gemm_nt_rows(A, B, np.arange(rows))
    dt = time.perf_counter() - t0
    flop = 2.0 * rows * N * K
    return {"value": round(flop / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of the 8192^3 product (ref and |A||B| bound, float64), {dt:.1f} s"}


def bench_frag(torch, f, stream, reps=20, sets=3, rounds=3):
    """frag_copy GB/s over 2^20 tiles (256 MiB moved per call).

    cold: three rotating buffer sets (768 MiB, more than the last-level cache
    holds, so every call streams from HBM); warm: one set called repeatedly.
    Each of the 18 combinations is timed once per round, the rounds sweeping
    all of them in turn, and reported as its median over the rounds.
    """
    from fp16_matrix_core_amd import inputs
    n_tiles = inputs.FRAG_TILES
    nbytes = n_tiles * 128
    bits = torch.from_numpy(inputs.frag_bits().view(np.int16)).cuda()
    srcs = [bits.clone() for _ in range(sets)]
    dsts = [torch.empty_like(bits) for _ in range(sets)]
    timer = StreamTimer(torch, stream)
    runs = {}
    for _ in range(rounds):
        for num in (1, 2, 4):
            for col in (0, 1):
                for direction, dname in ((0, "load"), (1, "store"), (2, "roundtrip")):
                    name = f"num{num}_{'col' if col else 'row'}_{dname}"
                    for kind, nsets in (("cold", sets), ("warm", 1)):
                        i = [0]

                        def call():
                            k = i[0] % nsets
                            i[0] += 1
                            f.frag_copy_raw(srcs[k].data_ptr(), dsts[k].data_ptr(), n_tiles, num, col, direction,
                                            stream.cuda_stream)
                        for _ in range(3):
                            call()
                        ms = timer.time(call, reps)
                        runs.setdefault((kind, name), []).append(2 * nbytes / (ms * 1e-3) / 1e9)
    cold = {name: round(statistics.median(v), 1) for (kind, name), v in runs.items() if kind == "cold"}
    warm = {name: round(statistics.median(v), 1) for (kind, name), v in runs.items() if kind == "warm"}
    vals = list(cold.values())
    return {"unit": "GB/s", "bytes_per_call": 2 * nbytes, "peak": PEAK_HBM_GBS, "rounds": rounds,
            "min_frac": round(min(vals) / PEAK_HBM_GBS, 4), "max_frac": round(max(vals) / PEAK_HBM_GBS, 4),
            "results": cold, "warm": warm}


def bench_batched(torch, f, stream, reps=20):
    from fp16_matrix_core_amd import inputs
    A, B = inputs.batched_small()
    a, b = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    sets = [(a, b, torch.empty((4096, 128, 64), dtype=torch.float32, device="cuda"))]
    sets += [(a.clone(), b.clone(), torch.empty_like(sets[0][2])) for _ in range(2)]
    i = [0]

    def call():
        x, y, o = sets[i[0] % 3]
        i[0] += 1
        f.gemm_nt_batched(x, y, o)
    for _ in range(3):
        call()
    ms = StreamTimer(torch, stream).time(call, reps)

    def warm_call():
        f.gemm_nt_batched(*sets[0])
    for _ in range(3):
        warm_call()
    ms_warm = StreamTimer(torch, stream).time(warm_call, reps)
    flop = 2.0 * 4096 * 128 * 64 * 64
    nbytes = 4096 * (128 * 64 * 2 + 64 * 64 * 2 + 128 * 64 * 4)
    return {"plan": f.plan(128, 64, 64, 4096), "us": round(ms * 1e3, 2), "TFLOP/s": round(flop / ms / 1e9, 2),
            "GB/s": round(nbytes / ms / 1e6, 1), "hbm_frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4),
            "warm_us": round(ms_warm * 1e3, 2), "warm_GB/s": round(nbytes / ms_warm / 1e6, 1),
            "timing": "us/GB/s: three rotating buffer sets (705 MB, streamed from HBM); warm_*: one set reused"}


def bench_skinny(torch, f, stream, reps=20):
    from fp16_matrix_core_amd import inputs
    A, B = inputs.skinny()
    a, b = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    o = torch.empty((16384, 8), dtype=torch.float32, device="cuda")
    sets = [(a, b, o), (a.clone(), b.clone(), torch.empty_like(o))]
    i = [0]

    def call():
        x, y, z = sets[i[0] % 2]
        i[0] += 1
        f.gemm_nt(x, y, z)
    for _ in range(3):
        call()
    ms = StreamTimer(torch, stream).time(call, reps)

    def warm_call():
        f.gemm_nt(*sets[0])
    for _ in range(3):
        warm_call()
    ms_warm = StreamTimer(torch, stream).time(warm_call, reps)
    flop = 2.0 * 16384 * 8 * 16384
    nbytes = 16384 * 16384 * 2 + 8 * 16384 * 2 + 16384 * 8 * 4
    return {"plan": f.plan(16384, 8, 16384), "us": round(ms * 1e3, 2), "TFLOP/s": round(flop / ms / 1e9, 2),
            "GB/s": round(nbytes / ms / 1e6, 1), "hbm_frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4),
            "warm_us": round(ms_warm * 1e3, 2), "warm_GB/s": round(nbytes / ms_warm / 1e6, 1),
            "timing": "us/GB/s: two alternating buffer sets (1.08 GB); warm_*: one set (538 MB) reused"}


def bench_small(torch, f, stream, reps=200):
    """The single 16x8x16 tile and the single 128x64x64 workgroup: time per call
    (launch-latency bound) through the raw entry point, inputs resident."""
    from fp16_matrix_core_amd import inputs
    out = {}
    A1, B1 = inputs.single_tile()
    A2, B2 = inputs.single_workgroup()[:2]
    sp = stream.cuda_stream
    for name, (A, B) in (("single_tile_16x8x16", (A1, B1)), ("single_workgroup_128x64x64", (A2, B2))):
        (M, K), N = A.shape, B.shape[0]
        a, b = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        o = torch.empty((M, N), dtype=torch.float32, device="cuda")

        def call():
            f.gemm_nt_raw(a.data_ptr(), b.data_ptr(), o.data_ptr(), M, N, K, K, K, N, sp)
        for _ in range(10):
            call()
        ms = StreamTimer(torch, stream).time(call, reps)
        out[name] = {"plan": f.plan(M, N, K), "us": round(ms * 1e3, 2)}
    return out


def bench_types(torch, f, stream, a, b, reps=20):
    """The 8192^3 launch with bfloat16 operands, 16-bit outputs and accumulation (gemm_nt_ex)."""
    from fp16_matrix_core_amd import inputs
    n = 8192
    A16, B16 = inputs.large_square_bf16(n)
    abf = torch.from_numpy(A16.view("int16")).cuda()
    bbf = torch.from_numpy(B16.view("int16")).cuda()
    outs = {"f32": torch.zeros((n, n), dtype=torch.float32, device="cuda"),
            "f16": torch.zeros((n, n), dtype=torch.float16, device="cuda"),
            "bf16": torch.zeros((n, n), dtype=torch.bfloat16, device="cuda")}
    code = {"f32": f.F32, "f16": f.F16, "bf16": f.BF16}
    res = {}
    for name, (x, y, ab, ot, acc) in {
            "bf16_in_f32_out": (abf, bbf, "bf16", "f32", False),
            "bf16_in_bf16_out": (abf, bbf, "bf16", "bf16", False),
            "f16_in_f16_out": (a, b, "f16", "f16", False),
            "f16_in_f32_out_accumulate": (a, b, "f16", "f32", True)}.items():
        o = outs[ot]

        def call():
            f.gemm_nt_ex_raw(x.data_ptr(), y.data_ptr(), o.data_ptr(), n, n, n, n, n, n, 1, 0, 0, 0,
                             code[ab], code[ot], acc, stream.cuda_stream)
        for _ in range(20):
            call()
        ms = StreamTimer(torch, stream).time(call, reps)
        tf = 2.0 * n ** 3 / ms / 1e9
        res[name] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(tf, 2), "frac": round(tf / PEAK_TFLOPS, 4)}
    return res


def bench_layouts(torch, f, stream, A, B, reps=20):
    """The 8192^3 fp16 -> fp32 launch with operands stored with K indexing their rows (gemm_ex)."""
    import numpy as np
    n = 8192
    a_mk = torch.from_numpy(A).cuda()
    b_nk = torch.from_numpy(B).cuda()
    a_km = torch.from_numpy(np.ascontiguousarray(A.T)).cuda()
    b_kn = torch.from_numpy(np.ascontiguousarray(B.T)).cuda()
    o = torch.empty((n, n), dtype=torch.float32, device="cuda")
    res = {}
    for name, (x, y, ao, bo) in {"nn_b_stored_KxN": (a_mk, b_kn, f.K_CONTIGUOUS, f.MN_CONTIGUOUS),
                                 "tt_a_stored_KxM": (a_km, b_nk, f.MN_CONTIGUOUS, f.K_CONTIGUOUS),
                                 "tn_both_stored_Kx": (a_km, b_kn, f.MN_CONTIGUOUS, f.MN_CONTIGUOUS)}.items():
        def call():
            f.gemm_ex_raw(x.data_ptr(), y.data_ptr(), o.data_ptr(), n, n, n, n, n, n, 1, 0, 0, 0,
                          ao, bo, f.F16, f.F32, False, stream.cuda_stream)
        for _ in range(20):
            call()
        ms = StreamTimer(torch, stream).time(call, reps)
        tf = 2.0 * n ** 3 / ms / 1e9
        res[name] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(tf, 2), "frac": round(tf / PEAK_TFLOPS, 4)}
    del a_km, b_kn
    return res


def ceiling_lib():
    import ctypes
    if not os.path.exists(CEILING_LIB):
        raise RuntimeError(f"{CEILING_LIB} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(CEILING_LIB)
    L.ceiling_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, ctypes.c_void_p]
    L.ceiling_mfma.restype = ctypes.c_int
    L.ceiling_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    L.ceiling_copy.restype = ctypes.c_int
    L.ceiling_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.ceiling_stream.restype = ctypes.c_int
    return L


def bench_ceilings(torch, stream, a, reps=10):
    """MFMA-only loops (one workgroup of 4 wavefronts per CU, 256 accumulators per
    lane) on the 8192^3 workload's A values and on zeros; a plain copy of the
    2^28 bytes a fragment copy moves (three rotating sets)."""
    L = ceiling_lib()
    sp = stream.cuda_stream
    grid = 256
    sink = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    ops = {"workload": a.reshape(-1), "zeros": torch.zeros_like(a.reshape(-1))}
    timer = StreamTimer(torch, stream)
    res = {"unit": "TFLOP/s", "grid": grid}
    for mi, iters in ((16, 4096), (32, 2048)):
        flop = 2.0 * grid * 4 * iters * (64 * 16 * 16 * 32 if mi == 16 else 16 * 32 * 32 * 16)
        for name, buf in ops.items():
            nb = buf.numel() * buf.element_size()

            def call():
                rc = L.ceiling_mfma(buf.data_ptr(), nb, sink.data_ptr(), mi, iters, grid, sp)
                if rc != 0:
                    raise RuntimeError(f"ceiling_mfma failed ({rc})")
            for _ in range(5):
                call()
            ms = timer.time(call, reps)
            res[f"mfma{mi}x{mi}_{name}"] = round(flop / ms / 1e9, 1)
    nbytes = 1 << 27                    # 128 MiB read + 128 MiB written per call
    bufs = [(torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0),
             torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")) for _ in range(3)]
    shapes = {}
    for shape, label in ((0, "1x512"), (1, "2x256"), (2, "4x256"), (3, "1x256")):
        i = [0]

        def copy():
            s_, d_ = bufs[i[0] % 3]
            i[0] += 1
            if L.ceiling_copy(s_.data_ptr(), d_.data_ptr(), nbytes, shape, sp) != 0:
                raise RuntimeError("ceiling_copy failed")
        for _ in range(5):
            copy()
        ms = timer.time(copy, 20)
        shapes[label] = round(2 * nbytes / (ms * 1e-3) / 1e9, 1)
    res["copy_shapes_GB/s"] = shapes
    res["copy_2^28B_GB/s"] = max(shapes.values())
    del bufs
    # Streams with the read/write mix of the batched product (per problem 24 KiB
    # read: A 128x64 and B 64x64 fp16; 32 KiB written) and of the skinny one's A
    # (32 KiB read per unit), in several launch shapes: one workgroup per unit,
    # or fewer workgroups taking units in turn, each unit's writes waiting for
    # its reads (as in the products) or not (overlapped); the best is the ceiling.
    def stream_ceiling(units, rd, wr, nsets, shapes):
        sets = [(torch.empty(units * rd // 4, dtype=torch.float32, device="cuda").fill_(1.0),
                 torch.empty(units * wr // 4, dtype=torch.float32, device="cuda")) for _ in range(nsets)]
        out = {}
        for grid, overlap in shapes:
            i = [0]

            def stream():
                s_, d_ = sets[i[0] % nsets]
                i[0] += 1
                if L.ceiling_stream(s_.data_ptr(), d_.data_ptr(), units, rd, wr, grid, overlap, sp) != 0:
                    raise RuntimeError("ceiling_stream failed")
            for _ in range(5):
                stream()
            ms = timer.time(stream, 20)
            label = f"{'overlapped' if overlap else 'dependent'}_grid{grid if grid else units}"
            out[label] = round(units * (rd + wr) / (ms * 1e-3) / 1e9, 1)
        del sets
        return out, max(out.values())
    shapes = ((0, 0), (2048, 0), (1536, 1), (2048, 1))
    res["batched_mix_shapes_GB/s"], res["batched_mix_4096x(24KiB_read+32KiB_write)_GB/s"] = \
        stream_ceiling(4096, 24576, 32768, 3, shapes)
    res["read_shapes_GB/s"], res["read_16384x32KiB_GB/s"] = stream_ceiling(16384, 32768, 16, 2, ((0, 0), (4096, 0)))
    return res


def pmc_pass(torch, f):
    """A short program for rocprofv3 counter passes: PMC_GEMM_LAUNCHES 8192^3
    launches, three copies of 1 GiB (the counter calibration), PMC_MFMA_LAUNCHES
    MFMA-only loops on the workload's values, and one call of each frag_copy
    variant (2^20 tiles)."""
    from fp16_matrix_core_amd import inputs
    A, B = inputs.large_square()
    a, b = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    out = torch.empty((8192, 8192), dtype=torch.float32, device="cuda")
    for _ in range(PMC_GEMM_LAUNCHES):      # the summaries use the later, clock-settled ones
        f.gemm_nt(a, b, out)
    torch.cuda.synchronize()
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    L = ceiling_lib()
    sink = torch.empty(256 * 256, dtype=torch.float32, device="cuda")
    sp = torch.cuda.current_stream().cuda_stream
    flat = a.reshape(-1)
    for _ in range(PMC_MFMA_LAUNCHES):
        if L.ceiling_mfma(flat.data_ptr(), flat.numel() * 2, sink.data_ptr(), 16, 4096, 256, sp) != 0:
            raise RuntimeError("ceiling_mfma failed")
    torch.cuda.synchronize()
    del src, dst
    n_tiles = inputs.FRAG_TILES
    img = torch.from_numpy(inputs.frag_bits().view(np.int16)).cuda()
    frag = torch.empty_like(img)
    for num in (1, 2, 4):
        for col in (0, 1):
            for direction in (0, 1, 2):
                f.frag_copy_raw(img.data_ptr(), frag.data_ptr(), n_tiles, num, col, direction, sp)
    torch.cuda.synchronize()
    log(f"pmc pass done: {PMC_GEMM_LAUNCHES} x gemm_nt 8192^3, 3 x copy of 1 GiB, {PMC_MFMA_LAUNCHES} x MFMA loop, "
        "18 x frag_copy")


def bench_shards(torch, f, stream, a, b, reps=20):
    """What one GPU runs when the 8192^3 product is split by rows over P GPUs:
    A's first 8192/P rows against the whole B (fp16 -> fp32)."""
    n = 8192
    res = {}
    for P in (2, 4, 8):
        m = n // P
        o = torch.empty((m, n), dtype=torch.float32, device="cuda")

        def call():
            f.gemm_nt_raw(a.data_ptr(), b.data_ptr(), o.data_ptr(), m, n, n, n, n, n, stream.cuda_stream)
        for _ in range(20):
            call()
        ms = StreamTimer(torch, stream).time(call, reps)
        tf = 2.0 * m * n * n / ms / 1e9
        res[f"P{P}_{m}x{n}x{n}"] = {"plan": f.plan(m, n, n), "us": round(ms * 1e3, 2), "TFLOP/s": round(tf, 2),
                                     "frac": round(tf / PEAK_TFLOPS, 4)}
        del o
    return res


def bench_library(torch, stream, a, b, reps=20):
    """Context, not a ceiling: the vendor BLAS behind torch.mm on the same 8192^3
    fp16 operands (fp16 output, the only output type torch.mm gives for fp16
    operands; compare gemm_8192_types.f16_in_f16_out). B is passed as a
    contiguous K x N copy of its transpose."""
    n = 8192
    x = a.view(torch.float16)
    y = b.view(torch.float16).t().contiguous()
    o = torch.empty((n, n), dtype=torch.float16, device="cuda")

    def call():
        torch.mm(x, y, out=o)
    for _ in range(20):
        call()
    ms = StreamTimer(torch, stream).time(call, reps)
    tf = 2.0 * n ** 3 / ms / 1e9
    del y, o
    return {"torch_mm_f16_in_f16_out_8192": {"us": round(ms * 1e3, 2), "TFLOP/s": round(tf, 2),
                                              "frac": round(tf / PEAK_TFLOPS, 4)}}


def run_secondary(torch, f, stream, a, b, A, B):
    log("secondary: ceilings, frag_copy, batched, skinny, small, operand/output types, storage orders, row shards, vendor BLAS")
    sec = {"ceilings": bench_ceilings(torch, stream, a),
           "frag_copy": bench_frag(torch, f, stream),
           "batched_4096x128x64x64": bench_batched(torch, f, stream),
           "skinny_16384x8x16384": bench_skinny(torch, f, stream),
           "small": bench_small(torch, f, stream),
           "gemm_8192_types": bench_types(torch, f, stream, a, b),
           "gemm_8192_storage_orders": bench_layouts(torch, f, stream, A, B),
           "gemm_row_shards": bench_shards(torch, f, stream, a, b),
           "vendor_blas": bench_library(torch, stream, a, b)}
    # the bandwidth-bound kernels against what a plain copy moves on this machine
    copy = sec["ceilings"]["copy_2^28B_GB/s"]
    fc = sec["frag_copy"]
    fc["copy_ceiling_GB/s"] = copy
    fc["min_frac_of_copy"] = round(min(fc["results"].values()) / copy, 4)
    fc["max_frac_of_copy"] = round(max(fc["results"].values()) / copy, 4)
    for key in ("batched_4096x128x64x64", "skinny_16384x8x16384"):
        sec[key]["frac_of_copy"] = round(sec[key]["GB/s"] / copy, 4)
    mix = sec["ceilings"]["batched_mix_4096x(24KiB_read+32KiB_write)_GB/s"]
    sec["batched_4096x128x64x64"]["frac_of_same_mix_stream"] = round(sec["batched_4096x128x64x64"]["GB/s"] / mix, 4)
    rd = sec["ceilings"]["read_16384x32KiB_GB/s"]
    sec["skinny_16384x8x16384"]["frac_of_read_stream"] = round(sec["skinny_16384x8x16384"]["GB/s"] / rd, 4)
    return sec


SWEEP_SHAPES = [(1024, 1024, 1024), (2048, 2048, 2048), (3072, 3072, 3072), (4096, 4096, 4096),
                (5120, 5120, 5120), (8192, 8192, 8192), (4096, 4096, 1024), (8192, 8192, 1024),
                (8192, 8192, 2048), (6144, 6144, 2048), (1536, 1536, 8192), (512, 512, 16384),
                (1024, 1024, 4096), (768, 768, 2048), (2048, 8192, 8192), (1024, 8192, 8192),
                (8192, 1024, 8192), (1024, 8192, 1024), (2048, 2048, 8192), (16384, 8, 16384),
                (16384, 16, 16384)]


def vendor_sweep(torch, f, rounds=5):
    """Context, not part of the headline: fp16 operands -> fp16 output through
    gemm_nt and through torch.mm (the vendor BLAS; B passed as a contiguous K x N
    copy of its transpose) on the same data, interleaved, median per shape."""
    g = torch.Generator(device="cuda").manual_seed(0)
    stream = torch.cuda.current_stream()
    timer = StreamTimer(torch, stream)
    out = []
    for M, N, K in SWEEP_SHAPES:
        a = (torch.randn((M, K), device="cuda", generator=g) * 0.1).half()
        b = (torch.randn((N, K), device="cuda", generator=g) * 0.1).half()
        bt = b.t().contiguous()
        o_lib = torch.empty((M, N), dtype=torch.float16, device="cuda")
        o_own = torch.empty((M, N + (-N) % 8), dtype=torch.float16, device="cuda")[:, :N]
        calls = {"torch_mm": lambda: torch.mm(a, bt, out=o_lib), "gemm_nt": lambda: f.gemm_nt(a, b, out=o_own)}
        reps = max(5, min(200, int(2e12 / (2.0 * M * N * K))))
        for fn in calls.values():
            for _ in range(3):
                fn()
        t = {k: [] for k in calls}
        for _ in range(rounds):
            for k, fn in calls.items():
                t[k].append(timer.time(fn, reps) * 1e3)
        lib_us, own_us = statistics.median(t["torch_mm"]), statistics.median(t["gemm_nt"])
        out.append({"shape": [M, N, K], "plan": f.plan(M, N, K), "torch_mm_us": round(lib_us, 2),
                    "gemm_nt_us": round(own_us, 2), "speedup": round(lib_us / own_us, 3),
                    "outputs_identical": bool(torch.equal(o_lib, o_own))})
        del a, b, bt, o_lib, o_own
    return {"kind": "vendor_sweep", "dtype": "fp16 in, fp16 out", "data": "synthetic normal(0,1)*0.1",
            "rounds": rounds, "results": out}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--pmc-pass", action="store_true")
    ap.add_argument("--vendor-sweep", action="store_true", help="gemm_nt against torch.mm over SWEEP_SHAPES")
    ap.add_argument("--headline-first", action="store_true",
                    help="time the headline before the secondary measurements (default: after them)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the product is not sharded "
              "across GPUs in this build.", file=sys.stderr)
        sys.exit(2)

    import torch
    import fp16_matrix_core_amd as f
    from fp16_matrix_core_amd import inputs
    f.lib()
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a ROCm GPU")
    if args.pmc_pass:
        pmc_pass(torch, f)
        return
    if args.vendor_sweep:
        print(json.dumps(vendor_sweep(torch, f)), flush=True)
        return

    M = N = K = 8192
    log("generating 8192^3 inputs (seed 4)")
    A, B = inputs.large_square()
    a = torch.from_numpy(A).cuda()
    b = torch.from_numpy(B).cuda()
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    plan = f.plan(M, N, K)

    def step():
        f.gemm_nt_raw(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, K, K, N, sp)

    secondary = None
    if not args.no_secondary and not args.headline_first:
        secondary = run_secondary(torch, f, stream, a, b, A, B)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # One event before each timed launch and one after the last: the total
    # gives the average launch time, the differences each launch's own.
    events = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    events[0].record(stream)
    for i in range(args.steps):
        step()
        events[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [events[i].elapsed_time(events[i + 1]) for i in range(args.steps)]
    ms_event = events[0].elapsed_time(events[-1]) / args.steps
    ms_step = wall * 1e3 / args.steps
    flop = 2.0 * M * N * K
    tflops = flop / (ms_step * 1e-3) / 1e12
    achieved = flop / (ms_event * 1e-3) / 1e12
    log(f"{plan}: {ms_event * 1e3:.1f} us/launch (events), {achieved:.1f} TFLOP/s")

    if not args.no_secondary and args.headline_first:
        secondary = run_secondary(torch, f, stream, a, b, A, B)

    khash = gemm_source_hash()
    traffic = read_traffic(khash)
    srt = sorted(step_ms)
    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16", "acc_dtype": "fp32", "data": "synthetic",
        "config": {"workload": "gemm_nt M=N=K=8192, A (M,K) and B (N,K) fp16 row-major ~ normal(0,1)*0.1 "
                               "(seed 4), Out fp32 (M,N)", "M": M, "N": N, "K": K, "kernel": plan},
        "pct_of_peak": round(100 * achieved / PEAK_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_TFLOPS, 4), "traffic": traffic,
                     "traffic_kind": "L2-miss bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated on a 1 GiB "
                                     "copy); reads served by the 256 MB last-level cache count too",
                     "kernel": plan, "us_per_launch": round(ms_event * 1e3, 2), "source_hash": khash},
        "step_us": {"min": round(srt[0] * 1e3, 1), "median": round(srt[len(srt) // 2] * 1e3, 1),
                    "max": round(srt[-1] * 1e3, 1),
                    "each": [round(x * 1e3, 1) for x in step_ms] if len(step_ms) <= 50 else None},
        "order": "headline first" if args.headline_first or args.no_secondary else
                 "secondary measurements first, then the headline's warm-up and timed launches",
    }
    if secondary is not None:
        result["secondary"] = secondary
        ceil = secondary.get("ceilings", {}).get("mfma16x16_workload")
        if ceil:
            result["roofline"]["mfma_only_ceiling"] = ceil
            result["roofline"]["frac_of_mfma_only_ceiling"] = round(achieved / ceil, 4)
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on a row sample")
        result["cpu_baseline"] = cpu_baseline(A, B)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
