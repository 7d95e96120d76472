#!/usr/bin/env python3
"""Throughput bench of the block-scaled FP4 codec on one MI355X.

Headline step: MXFP4 quantize+pack of a 4096 x 7168 bf16 MoE dispatch
activation (Student-t(4) * 0.5, 8 hot channels x30) followed by the
dequantize back to bf16 -- every step of the MXFP4 path (block absmax,
UE8M0 scale, scaling, E2M1 rounding, packing, receiver).  Inputs are resident
in HBM; the step rotates over buffer sets whose footprint (> 512 MB) exceeds
the 256 MB Infinity Cache, so repeats are not served from it.

value = algorithmic bytes per step (every input read once and every output
written once, both kernels) / measured step time.  Per-kernel durations come
from HIP events recorded on the launch stream around each launch.

Also reported: a roofline object for the dominant kernel (HBM bound, 8 TB/s
peak; traffic from the committed rocprofv3 PMC summary when it was taken on
the current kernel sources), the oracle's throughput on a bounded CPU
sample, and a breakdown of the other operations of the codec at their own
workload shapes.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-breakdown]
                       [--no-cpu-baseline] [--cpu-seconds S] [--profile-mode {headline,copy,fp8col,alu}]
       python bench.py --summarize-trace DIR --out FILE --command CMD
       python bench.py --summarize-pmc F_HEAD,F_COPY,W_HEAD,W_COPY --out FILE --command CMD
"""
import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "FP4 quantize+pack / dequant throughput, GB/s and % of MI355X HBM peak"
HBM_PEAK_GBS = 8000.0
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_mxfp4_codec_4096x7168.txt")
KERNEL_SOURCES = ["block_scaled_fp4_amd/csrc/quant.hip", "block_scaled_fp4_amd/csrc/device_common.hpp"]


def source_digest():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# What each breakdown row is judged against.
BOUNDS = {
    "hbm": "HBM peak (8 TB/s) on algorithmic bytes: every input read once, every output written once",
    "hbm_two_pass": "HBM peak on the bytes of both passes: the tensor-scale (amax) pass reads the "
                    "input once more before the encode pass",
    "alu": "VALU issue rate (Philox4x32-10 draws or transform butterflies per element exceed the "
           "HBM time); the HBM fraction is given for reference and the VALU counters are in profiles/",
    "launch": "launch latency: the tensor is too small to reach streaming bandwidth",
}

# ------------------------------------------------------------------ timing
def graph_time(torch, fn, calls, chunk, check=None):
    """Mean duration of one fn(k) call over exactly `calls` calls
    (k = 0 .. calls - 1).  The calls are captured in ceil(calls / chunk)
    HIP graphs (call k in graph k // chunk, so buffer rotation by k carries
    across graphs); each graph is replayed once untimed, `check` runs, and
    then every graph is replayed once, in order, between two HIP events on
    the launch stream.  Host launch overhead is thus excluded, as for a
    graph-captured caller.  Falls back to eager launches (events around the
    loop) if capture is refused."""
    calls = max(1, calls)
    chunk = max(1, min(chunk, calls))
    for k in range(min(calls, 3)):
        fn(k)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    try:
        graphs = []
        for g0 in range(0, calls, chunk):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for k in range(g0, min(calls, g0 + chunk)):
                    fn(k)
            graphs.append(g)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        if check:
            check()
        a.record()
        for g in graphs:
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / calls, f"{len(graphs)} graphs"
    except Exception as e:                      # capture unsupported: time eagerly
        log(f"[bench] graph capture failed ({e}); timing eagerly")
        torch.cuda.synchronize()
        a.record()
        for k in range(calls):
            fn(k)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / calls, "eager"


# --------------------------------------------------------------- headline
def headline(args, torch, fp4, np, synth):
    """Step k: quantize buffer set k (bf16 -> codes + UE8M0) and dequantize
    set k + LAG (codes + UE8M0 -> bf16), over `nsets` rotating sets.  The
    dequantize thus reads codes written LAG steps (> 2 steps' traffic, more
    than the 256 MB Infinity Cache) earlier, not the ones just written, and
    every input is read from HBM."""
    rows, cols = 4096, 7168
    n = rows * cols
    q_bytes = 2 * n + n // 2 + n // 32          # read bf16, write codes + UE8M0
    dq_bytes = n // 2 + n // 32 + 2 * n         # read codes + UE8M0, write bf16
    dq_in = n // 2 + n // 32
    log(f"[bench] generating {rows}x{cols} moe_dispatch input")
    xb = synth.moe_dispatch(rows, cols, seed=2)
    x0 = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
    # enough sets that the dequantize inputs alone rotate over >= 512 MB
    nsets = max(args.sets, -(-(512 << 20) // dq_in))
    lag = 3
    sets = []
    for _ in range(nsets):
        sets.append(dict(x=x0.clone(),
                         p=torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda"),
                         s=torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda"),
                         y=torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")))
    foot = nsets * (q_bytes + 2 * n)
    log(f"[bench] {nsets} buffer sets, footprint {foot / 1e6:.0f} MB; quantize inputs rotate over "
        f"{nsets * 2 * n / 1e6:.0f} MB, dequantize inputs over {nsets * dq_in / 1e6:.0f} MB")

    def quant(k):
        S = sets[k % nsets]
        fp4.fp4_quantize(S["x"], "mxfp4", "rtn", packed=S["p"], scales=S["s"])

    def dequant(k):
        S = sets[(k + lag) % nsets]
        fp4.fp4_dequantize(S["p"], S["s"], rows, cols, "mxfp4", y=S["y"])

    def step(k):
        quant(k)
        dequant(k)

    if args.profile_mode == "headline":
        for k in range(nsets):
            quant(k)
        for k in range(args.warmup + args.steps):
            step(k)
        torch.cuda.synchronize()
        log("[bench] profile-mode headline done")
        return None

    # eager reference outputs of every set, to check the graph replays against
    for k in range(nsets):
        quant(k)
    for k in range(nsets):
        step(k)
    torch.cuda.synchronize()
    ref = [(S["p"].clone(), S["s"].clone(), S["y"].clone()) for S in sets]

    def check():
        for S, (p, s, y) in zip(sets, ref):
            assert torch.equal(S["p"], p) and torch.equal(S["s"], s) and torch.equal(S["y"], y), \
                "graph replay differs from the eager result"

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    # exactly --steps steps, in several graphs (at least four when steps allow)
    chunk = max(1, min(args.graph_steps, args.steps // 4))
    ms_step, mode = graph_time(torch, step, args.steps, chunk, check)
    # per-kernel legs: every set at least twice
    kcalls = max(args.steps, 2 * nsets)
    q_ms, _ = graph_time(torch, quant, kcalls, args.graph_steps)
    d_ms, _ = graph_time(torch, dequant, kcalls, args.graph_steps)
    check()
    # achievable-bandwidth reference: a plain device copy of the bf16 input
    # (read 2n + write 2n bytes) over the same rotating buffer sets
    c_ms, _ = graph_time(torch, lambda k: sets[k % nsets]["y"].copy_(sets[k % nsets]["x"]), kcalls,
                         args.graph_steps)
    log(f"[bench] {mode}: step {ms_step * 1e3:.2f} us ({args.steps} steps); quantize {q_ms * 1e3:.2f} us; "
        f"dequantize {d_ms * 1e3:.2f} us ({kcalls} calls each)")
    return dict(rows=rows, cols=cols, n=n, q_bytes=q_bytes, dq_bytes=dq_bytes, ms_step=ms_step,
                q_ms=q_ms, d_ms=d_ms, copy_GBps=4 * n / (c_ms * 1e-3) / 1e9, nsets=nsets, footprint=foot,
                xb=xb, steps=args.steps, mode=mode, graph_chunk=chunk, kernel_calls=kcalls, lag=lag)


def copy_probe(args, torch):
    """A plain device copy of known size (PMC calibration for FETCH/WRITE_SIZE)."""
    nbytes = 256 << 20
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(args.steps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"[bench] profile-mode copy: {args.steps} copies of {nbytes} bytes")


def fp8col_probe(args, torch, fp4, synth):
    """The FP8-column workload of the breakdown (65,536 x 7168 MXFP4 rows in 256
    Zipf(1.1) experts), converted `steps` times (PMC runs)."""
    T, H, E = 65536, 7168, 256
    counts, off = synth.expert_counts(T, E, seed=5)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    act = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
    pk, sc, _ = fp4.fp4_quantize(act, "mxfp4", "rtn")
    del act
    offd = torch.from_numpy(off).cuda()
    o8 = torch.empty(T * H, dtype=torch.uint8, device="cuda")
    s8 = torch.empty(T * H // 128, dtype=torch.float32, device="cuda")
    s8t = torch.empty(fp4.tokblk_scale_count(T, E, H), dtype=torch.float32, device="cuda")
    for _ in range(args.steps):
        fp4.mxfp4_row_to_fp8_col(pk, sc, offd, H, o8, s8)
        fp4.mxfp4_row_to_fp8_col_tokblk(pk, sc, offd, H, o8, s8t)
    torch.cuda.synchronize()
    log(f"[bench] profile-mode fp8col: {args.steps} conversions of each FP8-column layout")


def alu_probe(args, torch, fp4, np, synth):
    """The rows judged against the VALU issue rate, each launched `steps`
    times (PMC runs): NVFP4 SR quantize of 8192x8192 bf16 and of 4096x7168
    fp32 with a given S_t, and the FP4Quant encoders of the 8192x4096 TP tensor (RTN G=256, SR
    G=64 and G=256)."""
    g = torch.Generator(device="cuda").manual_seed(11)
    x = (torch.randn((8192, 8192), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    p = torch.empty((8192, 4096), dtype=torch.uint8, device="cuda")
    s = torch.empty((8192, 512), dtype=torch.uint8, device="cuda")
    ts = torch.tensor([np.float32(0.03 / 2688)], dtype=torch.float32, device="cuda")
    for k in range(args.steps):
        fp4.fp4_quantize(x, "nvfp4", "sr", seed=1, step=k, tscale="given", tensor_scale=ts, packed=p, scales=s)
    del x, p, s
    xf = torch.randn((4096, 7168), generator=g, device="cuda") * 0.5
    pf = torch.empty((4096, 3584), dtype=torch.uint8, device="cuda")
    sf = torch.empty((4096, 448), dtype=torch.uint8, device="cuda")
    tf = torch.tensor([np.float32(1.0 / 2688)], dtype=torch.float32, device="cuda")
    for k in range(args.steps):
        fp4.fp4_quantize(xf, "nvfp4", "sr", seed=1, step=k, tscale="given", tensor_scale=tf, packed=pf, scales=sf)
    del xf, pf, sf
    tb = synth.tp_tensor()
    xt = torch.from_numpy(tb.view(np.int16)).view(torch.bfloat16).cuda()
    for G in (64, 256):
        for k in range(args.steps):
            if G == 256:
                fp4.fp4quant_encode(xt, G)
            fp4.fp4quant_encode_ex(xt, G, "sr", 5, k)
    torch.cuda.synchronize()
    log(f"[bench] profile-mode alu: {args.steps} launches of each ALU-bound row")


# ------------------------------------------------------------ breakdown
def breakdown(args, torch, fp4, np, synth, deferred):
    out = []
    iters = args.breakdown_iters
    with_oracle = not args.no_cpu_baseline
    if with_oracle:
        sys.path.insert(0, ROOT)
        from oracle import formats as F
        from oracle import fp4quant as Q
        from oracle import fp8col as O8
        from oracle import nvfp4 as NV

    def timed(fn, reps):
        return graph_time(torch, fn, 3 * reps, reps)[0]

    def leg(fn, nbytes, what, *fargs, prep=None, **fkw):
        """An oracle leg: fn(*fargs, **fkw) -- or fn(*prep()) when a prep
        function builds the arguments, untimed -- on a host sample worth
        `nbytes` algorithmic bytes.  Everything is bound now; preparation and
        timing run after the GPU work."""
        state = {}

        def call():
            if prep is not None and "args" not in state:
                state["args"] = prep()
            fn(*(state["args"] if prep is not None else fargs), **fkw)
            return nbytes
        return (call, what)

    def nv_compute(x):
        return NV.quantize_packed(x, NV.tensor_scale(x))

    valu = read_valu_summary()

    def add(op, workload, nbytes, ms, note=None, oracle=None, bound="hbm", extra_bytes=0, valu_row=None,
            elements=None):
        """oracle: (callable returning the algorithmic bytes of one call on a
        host sample, description of the sample), timed single-threaded.
        bound: what the row is judged against (BOUNDS); extra_bytes: bytes a
        second pass moves beyond the algorithmic ones (the amax pass)."""
        gbs = nbytes / (ms * 1e-3) / 1e9
        e = dict(op=op, workload=workload, algorithmic_bytes=nbytes, us=round(ms * 1e3, 2),
                 GBps=round(gbs, 1), frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4),
                 bound=bound, judged_against=BOUNDS[bound])
        if extra_bytes:
            two = (nbytes + extra_bytes) / (ms * 1e-3) / 1e9
            e["two_pass_bytes"] = nbytes + extra_bytes
            e["two_pass_GBps"] = round(two, 1)
            e["frac_of_hbm_peak_two_pass"] = round(two / HBM_PEAK_GBS, 4)
        if valu_row is not None and valu_row in valu and elements:
            # VALU issue-bound time: instructions counted by rocprofv3 (profiles/), one
            # wave64 instruction per CU per cycle, against this run's time
            t_valu = valu[valu_row] * elements / 64 / (CUS * CLOCK_HZ)
            e["valu_instructions_per_element"] = valu[valu_row]
            e["frac_of_valu_peak"] = round(t_valu / (ms * 1e-3), 4)
        if note:
            e["note"] = note
        if with_oracle and oracle is not None:
            pending.append((e, oracle))
        out.append(e)
        log(f"[bench] {op:28s} {workload:40s} {ms * 1e3:9.1f} us {gbs:8.1f} GB/s")

    # The oracle legs run after every GPU timing: a GPU left idle for seconds
    # between timings starts the next one at lowered clocks.
    pending = []

    def time_oracles():
        try:
            from threadpoolctl import threadpool_limits
            one_thread = threadpool_limits(limits=1)        # numpy's BLAS on one thread
        except Exception:
            one_thread = None
        for e, (fn, what) in pending:
            try:
                fn()                                        # preparation, untimed
                r, calls, dt = oracle_rate(fn, args.oracle_row_seconds)
                e["oracle_GBps_1core"] = round(r, 6)
                e["oracle_sample"] = f"{what}, {calls} calls in {dt:.1f} s"
                log(f"[bench] oracle {e['op']:28s} {r * 1e3:9.2f} MB/s ({e['oracle_sample']})")
            except Exception as ex:                 # a timing leg must not cost the GPU line
                e["oracle_GBps_1core"] = None
                log(f"[bench] oracle timing of {e['op']} failed: {ex}")
        if one_thread is not None:
            one_thread.restore_original_limits()

    # C1: NVFP4 RTN round trip of a 256 x 2048 bf16 weight block (launch bound)
    xb = synth.weight_block()
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
    R, C = x.shape
    n = R * C
    p = torch.empty((R, C // 2), dtype=torch.uint8, device="cuda")
    s = torch.empty((R, C // 16), dtype=torch.uint8, device="cuda")
    ts = torch.empty(1, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    nb = 2 * n + n // 2 + n // 16 + 4
    o_q = o_dq = None
    if with_oracle:
        def prep_c1(xb=xb):
            xw = F.bf16_bits_to_f32(xb)
            stw = NV.tensor_scale(xw)
            return NV.quantize_packed(xw, stw) + (stw,)
        o_q = leg(nv_compute, nb, "the whole 256x2048 block", prep=lambda xb=xb: (F.bf16_bits_to_f32(xb),))
        o_dq = leg(NV.dequantize, nb, "the whole 256x2048 block", prep=prep_c1)
    add("nvfp4_quantize(rtn,compute)", "256x2048 bf16 weight block", nb,
        timed(lambda k: fp4.fp4_quantize(x, "nvfp4", "rtn", packed=p, scales=s, tensor_scale=ts), iters),
        "3 launches: amax, reduction of the partial maxima, encode", oracle=o_q, bound="launch")
    add("nvfp4_dequantize", "256x2048 bf16 weight block", nb,
        timed(lambda k: fp4.fp4_dequantize(p, s, R, C, "nvfp4", ts, y=y), iters), oracle=o_dq,
        bound="launch")

    # C1 shape at 8192 x 8192: the NVFP4 bandwidth row (4 rotating sets, 690 MB,
    # so that the 256 MB Infinity Cache cannot serve one call's data to the next)
    R, C = 8192, 8192
    n = R * C
    NS = 4
    g = torch.Generator(device="cuda").manual_seed(11)
    xs = [(torch.randn((R, C), generator=g, device="cuda") * 0.02).to(torch.bfloat16) for _ in range(NS)]
    ps = [torch.empty((R, C // 2), dtype=torch.uint8, device="cuda") for _ in range(NS)]
    ss = [torch.empty((R, C // 16), dtype=torch.uint8, device="cuda") for _ in range(NS)]
    ys = [torch.empty((R, C), dtype=torch.bfloat16, device="cuda") for _ in range(NS)]
    ts = torch.empty(1, dtype=torch.float32, device="cuda")
    nb = 2 * n + n // 2 + n // 16
    fp4.fp4_quantize(xs[0], "nvfp4", "rtn", packed=ps[0], scales=ss[0], tensor_scale=ts)
    o_g = o_c = o_d = o_sr = None
    if with_oracle:
        m = 64
        xh = xs[0][:m].float().cpu().numpy()
        sth = np.float32(ts.cpu().numpy()[0])
        nbm = nb * m // R
        o_g = leg(NV.quantize_packed, nbm, f"{m} rows, S_t given", xh, sth)
        o_c = leg(nv_compute, nbm, f"{m} rows, S_t from the sample", xh)
        o_d = leg(NV.dequantize, nbm, f"{m} rows",
                  prep=lambda xh=xh, sth=sth: NV.quantize_packed(xh, sth) + (sth,))
        o_sr = leg(NV.quantize_packed, nbm // 4, "16 rows", xh[:16], sth, "sr", seed=1, step=3)
    add("nvfp4_quantize(rtn,given)", "8192x8192 bf16", nb,
        timed(lambda k: fp4.fp4_quantize(xs[k % NS], "nvfp4", "rtn", tscale="given", tensor_scale=ts,
                                         packed=ps[k % NS], scales=ss[k % NS]), iters), oracle=o_g)
    add("nvfp4_quantize(rtn,compute)", "8192x8192 bf16", nb,
        timed(lambda k: fp4.fp4_quantize(xs[k % NS], "nvfp4", "rtn", tensor_scale=ts,
                                         packed=ps[k % NS], scales=ss[k % NS]), iters),
        "includes the amax pass (an extra read of x)", oracle=o_c, bound="hbm_two_pass",
        extra_bytes=2 * n)
    add("nvfp4_dequantize", "8192x8192 bf16", nb,
        timed(lambda k: fp4.fp4_dequantize(ps[k % NS], ss[k % NS], R, C, "nvfp4", ts, y=ys[k % NS]), iters),
        oracle=o_d)
    add("nvfp4_quantize(sr,given)", "8192x8192 bf16", nb,
        timed(lambda k: fp4.fp4_quantize(xs[k % NS], "nvfp4", "sr", seed=1, step=k, tscale="given",
                                         tensor_scale=ts, packed=ps[k % NS], scales=ss[k % NS]), iters),
        oracle=o_sr, bound="alu", valu_row="nvfp4 quantize sr, 8192x8192 bf16", elements=n)
    del xs, ps, ss, ys

    # MXFP4 with fp32 activations: quantize from fp32, dequantize to fp32 (4096 x 7168, 4 sets)
    R, C = 4096, 7168
    n = R * C
    xs = [torch.randn((R, C), generator=g, device="cuda") * 0.5 for _ in range(4)]
    ps = [torch.empty((R, C // 2), dtype=torch.uint8, device="cuda") for _ in range(4)]
    ss = [torch.empty((R, C // 32), dtype=torch.uint8, device="cuda") for _ in range(4)]
    ys = [torch.empty((R, C), dtype=torch.float32, device="cuda") for _ in range(4)]
    nb = 4 * n + n // 2 + n // 32
    add("mxfp4_quantize(rtn) f32 in", "4096x7168 fp32", nb,
        timed(lambda k: fp4.fp4_quantize(xs[k % 4], "mxfp4", "rtn", packed=ps[k % 4], scales=ss[k % 4]),
              iters))
    ts32 = torch.tensor([np.float32(1.0 / 2688)], dtype=torch.float32, device="cuda")
    ss16 = [torch.empty((R, C // 16), dtype=torch.uint8, device="cuda") for _ in range(4)]
    add("nvfp4_quantize(rtn,given) f32 in", "4096x7168 fp32", 4 * n + n // 2 + n // 16,
        timed(lambda k: fp4.fp4_quantize(xs[k % 4], "nvfp4", "rtn", tscale="given", tensor_scale=ts32,
                                         packed=ps[k % 4], scales=ss16[k % 4]), iters))
    add("nvfp4_quantize(sr,given) f32 in", "4096x7168 fp32", 4 * n + n // 2 + n // 16,
        timed(lambda k: fp4.fp4_quantize(xs[k % 4], "nvfp4", "sr", seed=1, step=k, tscale="given",
                                         tensor_scale=ts32, packed=ps[k % 4], scales=ss16[k % 4]), iters),
        bound="alu", valu_row="nvfp4 quantize sr, 4096x7168 fp32", elements=n)
    add("mxfp4_dequantize f32 out", "4096x7168 fp32", nb,
        timed(lambda k: fp4.fp4_dequantize(ps[k % 4], ss[k % 4], R, C, "mxfp4", None, torch.float32,
                                           ys[k % 4]), iters))
    del xs, ps, ss, ys, ss16

    # C3: FP4Quant codec on the 8192 x 4096 TP tensor, G = 64 and 256
    tb = synth.tp_tensor()
    R, C = tb.shape
    n = R * C
    x = torch.from_numpy(tb.view(np.int16)).view(torch.bfloat16).cuda()
    xs = [x] + [x.clone() for _ in range(3)]
    for G in (64, 256):
        pk = [torch.empty((R, C // 2), dtype=torch.uint8, device="cuda") for _ in range(4)]
        s1 = [torch.empty((R, C // G), dtype=torch.float32, device="cuda") for _ in range(4)]
        s2 = [torch.empty((R, C // G), dtype=torch.float32, device="cuda") for _ in range(4)]
        ys = [torch.empty((R, C), dtype=torch.bfloat16, device="cuda") for _ in range(4)]
        nb = 2 * n + n // 2 + 8 * (n // G)
        o_e = o_de = None
        if with_oracle:
            m = 64
            xq = F.bf16_bits_to_f32(tb[:m])
            o_e = leg(Q.encode_packed, nb * m // R, f"{m} rows", xq, G)
            o_de = leg(Q.decode64, nb * m // R, f"{m} rows (float64 output)",
                       prep=lambda xq=xq, G=G: Q.encode(xq, G) + (G,))
        add(f"fp4quant_encode(G={G})", "8192x4096 bf16 TP tensor", nb,
            timed(lambda k: fp4.fp4quant_encode(xs[k % 4], G, pk[k % 4], s1[k % 4], s2[k % 4]), iters),
            oracle=o_e, bound="alu" if G >= 256 else "hbm",
            valu_row=f"fp4quant encode rtn G={G}, 8192x4096 bf16", elements=n)
        add(f"fp4quant_decode(G={G})", "8192x4096 bf16 TP tensor", nb,
            timed(lambda k: fp4.fp4quant_decode(pk[k % 4], s1[k % 4], s2[k % 4], R, C, G, y=ys[k % 4]),
                  iters), oracle=o_de)
        o_sr = None
        if with_oracle:
            o_sr = leg(Q.encode_packed, nb * 16 // R, "16 rows", F.bf16_bits_to_f32(tb[:16]), G, "sr",
                       seed=5, step=2)
        add(f"fp4quant_encode_sr(G={G})", "8192x4096 bf16 TP tensor", nb,
            timed(lambda k: fp4.fp4quant_encode_ex(xs[k % 4], G, "sr", 5, k, pk[k % 4], s1[k % 4],
                                                   s2[k % 4]), iters),
            "stochastic-rounding variant (Philox draws per element)", oracle=o_sr, bound="alu",
            valu_row=f"fp4quant encode sr G={G}, 8192x4096 bf16", elements=n)
    del xs, pk, s1, s2, ys, x

    # C4: SR + error feedback step on an 8192 x 8192 weight (x fp32, r fp32, W bf16)
    R, C = 8192, 8192
    n = R * C
    W = (torch.randn((R, C), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    xf = W.float() + 1e-4 * torch.randn((R, C), generator=g, device="cuda")
    r = torch.zeros((R, C), dtype=torch.float32, device="cuda")
    ts = torch.empty(1, dtype=torch.float32, device="cuda")
    nb = 4 * n + 4 * n + 4 * n + 2 * n
    o_ec = o_eg = None
    if with_oracle:
        m = 16
        xe = xf[:m].cpu().numpy()
        re_ = np.zeros((m, C), np.float32)
        o_ec = leg(NV.errfeedback_qdq, nb * m // R, f"{m} rows, S_t from the sample", xe, re_, None,
                   "sr", seed=4, step=1)
        o_eg = leg(NV.errfeedback_qdq, nb * m // R, f"{m} rows", xe, re_, np.float32(1e-4), "sr",
                   seed=4, step=1)
    add("errfeedback_qdq(sr,compute)", "8192x8192 fp32 x + fp32 r -> bf16 W", nb,
        timed(lambda k: fp4.fp4_errfeedback_qdq(xf, r, W, None, "sr", 4, k, "compute", ts), max(iters // 2, 5)),
        "includes the amax pass over x + r (536,870,912 extra bytes read)", oracle=o_ec,
        bound="hbm_two_pass", extra_bytes=8 * n)
    add("errfeedback_qdq(sr,given)", "8192x8192 fp32 x + fp32 r -> bf16 W", nb,
        timed(lambda k: fp4.fp4_errfeedback_qdq(xf, r, W, None, "sr", 4, k, "given", ts), max(iters // 2, 5)),
        oracle=o_eg)
    del W, xf, r

    # C5: MXFP4 rows -> FP8 columns over 256 Zipf(1.1) expert shards, 65536 x 7168
    T, H, E = 65536, 7168, 256
    counts, off = synth.expert_counts(T, E, seed=5)
    act = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
    pk, sc, _ = fp4.fp4_quantize(act, "mxfp4", "rtn")
    del act
    offd = torch.from_numpy(off).cuda()
    o8 = torch.empty(T * H, dtype=torch.uint8, device="cuda")
    s8 = torch.empty(T * H // 128, dtype=torch.float32, device="cuda")
    nb = T * H // 2 + T * H // 32 + T * H + 4 * (T * H // 128)
    o_col = o_row = None
    if with_oracle:
        m = 512
        ph8, sh8 = pk[:m].cpu().numpy(), sc[:m].cpu().numpy()
        offm = np.minimum(off, m).astype(np.int64)             # the experts' tokens among the first m
        o_col = leg(O8.convert, nb * m // T, f"the first {m} tokens in their expert layout", ph8, sh8,
                    offm, H)
        o_row = leg(O8.convert_rows, nb * m // T, f"{m} tokens", ph8, sh8, H)
    add("mxfp4_row_to_fp8_col", "65536x7168, 256 Zipf(1.1) experts", nb,
        timed(lambda k: fp4.mxfp4_row_to_fp8_col(pk, sc, offd, H, o8, s8), max(iters // 2, 5)),
        oracle=o_col)
    # the same shards with FP8 blocks of 128 tokens per channel (the token-direction reading)
    nsc = fp4.tokblk_scale_count(T, E, H)
    s8t = torch.empty(nsc, dtype=torch.float32, device="cuda")
    nb_tok = T * H // 2 + T * H // 32 + T * H + 4 * H * int(sum((int(c) + 127) // 128 for c in counts))
    o_tok = None
    if with_oracle:
        o_tok = leg(O8.convert_token_blocks, nb_tok * m // T,
                    f"the first {m} tokens in their expert layout", ph8, sh8, offm, H)
    add("mxfp4_row_to_fp8_col_tokblk", "65536x7168, 256 Zipf(1.1) experts, 128-token blocks", nb_tok,
        timed(lambda k: fp4.mxfp4_row_to_fp8_col_tokblk(pk, sc, offd, H, o8, s8t), max(iters // 2, 5)),
        oracle=o_tok)
    del s8t
    # the same rows -> FP8 rows (no transpose): the dispatch receiver
    o8r, s8r = o8.view(T, H), s8.view(T, H // 128)
    add("mxfp4_row_to_fp8_row", "65536x7168", nb,
        timed(lambda k: fp4.mxfp4_row_to_fp8_row(pk, sc, H, o8r, s8r), max(iters // 2, 5)),
        oracle=o_row)
    del pk, sc, o8, s8, o8r, s8r
    deferred.append(time_oracles)         # run by the caller once the GPU work is done
    return out


# ---------------------------------------------------------------- sweep
def size_sweep(args, torch, fp4, np):
    """MXFP4 quantize and dequantize of bf16 [rows, 7168] over a range of
    sizes; a least-squares fit of time = bytes / BW + t0 separates the
    fixed cost of a launch (ramp-up, tail, the end-of-kernel cache write-back)
    from the streaming bandwidth.  Each size rotates enough buffer sets to
    exceed 768 MB, so the Infinity Cache cannot serve one call's data to the
    next."""
    cols = 7168
    res = {}
    pts = {"quantize": [], "dequantize": []}
    g = torch.Generator(device="cuda").manual_seed(12)
    for rows in args.sweep_rows:
        n = rows * cols
        per_set = 2 * n + n // 2 + n // 32 + 2 * n
        nsets = max(2, -(-(768 << 20) // per_set))
        x0 = (torch.randn((rows, cols), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
        sets = [dict(x=x0 if k == 0 else x0.clone(),
                     p=torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda"),
                     s=torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda"),
                     y=torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")) for k in range(nsets)]
        reps = max(40, nsets)

        def quant(k):
            S = sets[k % nsets]
            fp4.fp4_quantize(S["x"], "mxfp4", "rtn", packed=S["p"], scales=S["s"])

        def dequant(k):
            S = sets[k % nsets]
            fp4.fp4_dequantize(S["p"], S["s"], rows, cols, "mxfp4", y=S["y"])

        nb = 2 * n + n // 2 + n // 32
        for name, fn in (("quantize", quant), ("dequantize", dequant)):
            ms, _ = graph_time(torch, fn, 3 * reps, reps)
            pts[name].append((rows, nb, ms * 1e3))
        log(f"[bench] sweep {rows:6d} x {cols}: {nsets:3d} sets; quantize {pts['quantize'][-1][2]:8.2f} us; "
            f"dequantize {pts['dequantize'][-1][2]:8.2f} us")
        del sets, x0
    for name, pp in pts.items():
        b = np.array([q[1] for q in pp], np.float64)
        t = np.array([q[2] for q in pp], np.float64)
        A = np.stack([b, np.ones_like(b)], axis=1)
        (inv_bw, t0), *_ = np.linalg.lstsq(A, t, rcond=None)
        res[name] = dict(bw_fit_GBps=round(1e-3 / inv_bw, 1), t0_us=round(float(t0), 2),
                         frac_fit_of_hbm_peak=round(1e-3 / inv_bw / HBM_PEAK_GBS, 4),
                         points=[[r, int(nb), round(us, 2), round(nb / (us * 1e-6) / 1e9, 1)] for r, nb, us in pp])
        log(f"[bench] sweep fit {name}: {1e-3 / inv_bw:.0f} GB/s streaming + {t0:.2f} us per launch")
    res["op"] = f"mxfp4 rtn, bf16 [rows, {cols}]; points are [rows, algorithmic bytes, us, GB/s]"
    return res


# ---------------------------------------------------------- cpu baseline
def oracle_rate(fn, min_seconds):
    """GB/s of fn() (which returns the algorithmic bytes of one call), called
    until at least min_seconds have passed."""
    nbytes, calls = 0, 0
    t0 = time.perf_counter()
    while True:
        nbytes += fn()
        calls += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            return nbytes / dt / 1e9, calls, dt


def _oracle_roundtrip_chunk(xb_chunk):
    """Pool worker: the oracle's MXFP4 quantize + dequantize of one chunk of
    bf16 rows; returns the algorithmic bytes."""
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from oracle import formats as F
    from oracle import mxfp4
    x = F.bf16_bits_to_f32(xb_chunk)
    p, s = mxfp4.quantize_packed(x)
    mxfp4.dequantize(p, s, "bf16")
    n = x.size
    return 2 * (2 * n + n // 2 + n // 32)


def cpu_baseline_pool(xb, procs, rows_chunk=64, min_seconds=10.0):
    """The same oracle work spread over `procs` worker processes (spawned, one
    BLAS thread each), passing over the headline input until at least
    min_seconds have passed."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    try:
        chunks = [xb[r0:r0 + rows_chunk] for r0 in range(0, xb.shape[0], rows_chunk)]
        # an executor (not a Pool): a worker that dies raises instead of being respawned
        with ProcessPoolExecutor(max_workers=procs, mp_context=mp.get_context("spawn")) as ex:
            list(ex.map(_oracle_roundtrip_chunk, [c[:1] for c in chunks[:procs]]))  # workers up
            nbytes, passes = 0, 0
            t0 = time.perf_counter()
            while True:
                nbytes += sum(ex.map(_oracle_roundtrip_chunk, chunks))
                passes += 1
                dt = time.perf_counter() - t0
                if dt >= min_seconds:
                    break
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return nbytes / dt / 1e9, passes, dt


def cpu_baseline(xb, rows_chunk=512, min_seconds=10.0, max_seconds=30.0):
    """The oracle, untuned, on the host: quantize+dequantize of the headline
    input in chunks of `rows_chunk` rows, passing over the whole tensor until
    at least `min_seconds` of work (stopping early past `max_seconds`)."""
    sys.path.insert(0, ROOT)
    from oracle import formats as F
    from oracle import mxfp4
    rows_total = xb.shape[0]
    nbytes = 0
    rows_done = 0
    t0 = time.perf_counter()
    while True:
        for r0 in range(0, rows_total, rows_chunk):
            x = F.bf16_bits_to_f32(xb[r0:r0 + rows_chunk])
            p, s = mxfp4.quantize_packed(x)
            mxfp4.dequantize(p, s, "bf16")
            n = x.size
            nbytes += 2 * (2 * n + n // 2 + n // 32)
            rows_done += x.shape[0]
            if time.perf_counter() - t0 > max_seconds:
                break
        dt = time.perf_counter() - t0
        if dt >= min_seconds or dt > max_seconds:
            break
    one = nbytes / dt / 1e9
    one_sample = (f"{rows_done} rows ({rows_done / rows_total:.2f} passes over the "
                  f"{rows_total}x{xb.shape[1]} input, {rows_chunk}-row chunks), {dt:.1f} s")
    affinity, model = host_cpus()
    procs = min(CPU_SHARE, affinity)
    host = {"affinity_cores": affinity, "cpu_model": model,
            "cores_note": f"workers = min({CPU_SHARE}, affinity cores): a one-GPU job's share of "
                          f"this host's CPUs is {CPU_SHARE}"}
    try:
        rate, passes, dtp = cpu_baseline_pool(xb, procs, min_seconds=min_seconds)
    except Exception as ex:                         # the pooled leg must not cost the GPU line
        log(f"[bench] pooled oracle failed ({ex}); reporting the single-core leg")
        return dict({"value": round(one, 6), "unit": "GB/s", "cores": 1, "kind": "oracle",
                     "sample": f"quantize+dequantize of {one_sample}, single-threaded numpy"}, **host)
    return dict({"value": round(rate, 6), "unit": "GB/s", "cores": procs, "kind": "oracle",
                 "sample": f"quantize+dequantize of the {rows_total}x{xb.shape[1]} input in 64-row chunks "
                           f"over {procs} worker processes (one thread each), {passes} passes in {dtp:.1f} s",
                 "value_1core": round(one, 6), "sample_1core": one_sample}, **host)


CPU_SHARE = 16


def host_cpus():
    """(CPUs this process may run on, CPU model name from /proc/cpuinfo)."""
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return affinity, model


# ------------------------------------------------------------ PMC summary
VALU_SUMMARY = os.path.join(ROOT, "profiles", "valu_alu_rows_8192x8192_8192x4096.txt")


def read_valu_summary():
    """row label -> VALU instructions per element, from the committed counter summary."""
    out = {}
    if not os.path.exists(VALU_SUMMARY):
        return out
    for line in open(VALU_SUMMARY):
        if line.startswith("#") or line.startswith(" ") or line.startswith("row"):
            continue
        parts = line.split()
        if len(parts) < 8:
            continue
        label = " ".join(parts[:-7])
        try:
            out[label] = float(parts[-4])
        except ValueError:
            pass
    return out
def read_pmc_summary():
    if not os.path.exists(PMC_SUMMARY):
        return None
    kv = {}
    with open(PMC_SUMMARY) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    return kv


def _rocpd_rows(directory, query):
    """Rows of a query over every rocpd database (rocprofv3 default output) in a directory."""
    import sqlite3
    rows = []
    for fn in sorted(glob.glob(os.path.join(directory, "**", "*.db"), recursive=True)):
        con = sqlite3.connect(fn)
        try:
            rows += con.execute(query).fetchall()
        finally:
            con.close()
    return rows


def _short(name):
    return name.replace("fp4mi::(anonymous namespace)::", "").replace("void ", "").split("(")[0]


def summarize_trace(directory, out, command):
    """rocprofv3 --kernel-trace --stats output -> a duration table per kernel
    and launch shape (workgroups x threads), so that launches of one kernel at
    different sizes are not averaged together."""
    import statistics
    per, info = {}, {}
    for name, dur, gx, wx, vgpr, lds in _rocpd_rows(
            directory, "select name, duration, grid_x, workgroup_x, vgpr_count, lds_size from kernels"):
        key = (_short(name), int(gx) // max(int(wx), 1), int(wx))
        per.setdefault(key, []).append(dur / 1e3)
        info[key] = (vgpr, lds)
    lines = [f"# rocprofv3 kernel trace summary (durations in us; one row per kernel and launch shape)",
             f"# command: {command}", f"# source_digest: {source_digest()}",
             f"{'kernel':56s} {'workgroups x threads':>22s} {'calls':>6s} {'mean':>9s} {'median':>9s} "
             f"{'min':>9s} {'max':>9s} {'vgpr':>5s} {'lds':>7s}"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        shape = f"{k[1]} x {k[2]}"
        vg, ld = info[k]
        lines.append(f"{k[0][:56]:56s} {shape:>22s} {len(v):6d} {statistics.mean(v):9.2f} "
                     f"{statistics.median(v):9.2f} {min(v):9.2f} {max(v):9.2f} {vg:>5} {ld:>7}")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_pmc(dirs, out, command):
    """Four rocprofv3 --pmc runs (FETCH_SIZE / WRITE_SIZE on the headline and on a
    plain 256 MiB device copy) -> HBM bytes per launch of the headline kernels,
    each counter scaled so that the copy reads and writes exactly 256 MiB."""
    import statistics
    fh, fc, wh, wc = dirs.split(",")
    copy_bytes = 256 << 20

    def per_kernel(d, ctr):
        acc = {}
        for name, v in _rocpd_rows(d, f"select kernel_name, value from counters_collection "
                                      f"where counter_name = '{ctr}'"):
            acc.setdefault(_short(name), []).append(v * 1024.0)
        return {k: statistics.median(v) for k, v in acc.items()}

    f_copy = per_kernel(fc, "FETCH_SIZE")["__amd_rocclr_copyBuffer"]
    w_copy = per_kernel(wc, "WRITE_SIZE")["__amd_rocclr_copyBuffer"]
    kf, kw = copy_bytes / f_copy, copy_bytes / w_copy
    fetch, write = per_kernel(fh, "FETCH_SIZE"), per_kernel(wh, "WRITE_SIZE")
    n = 4096 * 7168
    alg = 2 * n + n // 2 + n // 32
    # template arguments: <bf16 input, MX, SR, ...> and <bf16 output, MX, ...>
    q = next(k for k in fetch if k.startswith("quantize_kernel<true, true, false"))
    d = next(k for k in fetch if k.startswith("dequantize_kernel<true, "))
    lines = ["# rocprofv3 PMC summary: HBM traffic of the MXFP4 headline kernels (4096x7168 bf16)",
             f"# command: {command}",
             f"# copy calibration: FETCH_SIZE reads {f_copy:.0f} B for a {copy_bytes} B copy (x{kf:.4f}); "
             f"WRITE_SIZE writes {w_copy:.0f} B (x{kw:.4f})",
             f"source_digest: {source_digest()}",
             "kernels: quantize dequantize",
             f"fetch_factor: {kf:.6f}", f"write_factor: {kw:.6f}",
             f"algorithmic_bytes_per_launch: {alg}",
             f"quantize_fetch_bytes: {fetch[q] * kf:.0f}", f"quantize_write_bytes: {write[q] * kw:.0f}",
             f"quantize_hbm_bytes_per_launch: {fetch[q] * kf + write[q] * kw:.0f}",
             f"dequantize_fetch_bytes: {fetch[d] * kf:.0f}", f"dequantize_write_bytes: {write[d] * kw:.0f}",
             f"dequantize_hbm_bytes_per_launch: {fetch[d] * kf + write[d] * kw:.0f}"]
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_pmc_kernel(dirs, out, command, prefix, alg, title):
    """FETCH_SIZE / WRITE_SIZE runs of a workload and of the 256 MiB copy ->
    HBM bytes per launch of the kernel whose short name starts with `prefix`,
    scaled by the copy calibration, against its algorithmic bytes."""
    import statistics
    fk, fc, wk, wc = dirs.split(",")
    copy_bytes = 256 << 20

    def per_kernel(d, ctr):
        acc = {}
        for name, v in _rocpd_rows(d, f"select kernel_name, value from counters_collection "
                                      f"where counter_name = '{ctr}'"):
            acc.setdefault(_short(name), []).append(v * 1024.0)
        return {k: statistics.median(v) for k, v in acc.items()}

    kf = copy_bytes / per_kernel(fc, "FETCH_SIZE")["__amd_rocclr_copyBuffer"]
    kw = copy_bytes / per_kernel(wc, "WRITE_SIZE")["__amd_rocclr_copyBuffer"]
    fetch, write = per_kernel(fk, "FETCH_SIZE"), per_kernel(wk, "WRITE_SIZE")
    k = next(n for n in fetch if n.startswith(prefix))
    fb, wb = fetch[k] * kf, write[k] * kw
    lines = [f"# rocprofv3 PMC summary: HBM traffic of {title}", f"# command: {command}",
             f"# copy calibration: FETCH_SIZE x{kf:.4f}, WRITE_SIZE x{kw:.4f} (256 MiB device copy)",
             f"kernel: {k}", f"fetch_bytes: {fb:.0f}", f"write_bytes: {wb:.0f}",
             f"hbm_bytes_per_launch: {fb + wb:.0f}", f"algorithmic_bytes_per_launch: {alg}",
             f"hbm_over_algorithmic: {(fb + wb) / alg:.4f}"]
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


# Elements per launch of the ALU-bound rows of --profile-mode alu (by kernel
# name prefix): 8192 x 8192 NVFP4 SR, 8192 x 4096 FP4Quant encoders.
ALU_ROWS = [("quantize_kernel<true, false, true", "nvfp4 quantize sr, 8192x8192 bf16", 8192 * 8192),
            ("nv_quantize_f32_kernel<true, false", "nvfp4 quantize sr, 4096x7168 fp32", 4096 * 7168),
            ("fq_encode_rows_kernel<true, 64, true", "fp4quant encode sr G=64, 8192x4096 bf16", 8192 * 4096),
            ("fq_encode_rows_kernel<true, 256, true", "fp4quant encode sr G=256, 8192x4096 bf16", 8192 * 4096),
            ("fq_encode_rows_kernel<true, 256, false", "fp4quant encode rtn G=256, 8192x4096 bf16", 8192 * 4096)]
CUS, CLOCK_HZ = 256, 2.4e9


def summarize_valu(dirs, trace_dir, out, command):
    """rocprofv3 --pmc runs (comma-separated output dirs) of --profile-mode alu
    and a --kernel-trace run of the same mode -> per kernel: VALU
    instructions per element and the VALU issue-bound time, against the
    traced duration.  The bound: a CU issues one wave64 VALU instruction per
    cycle (four SIMDs, four cycles each): t_valu = INSTS_VALU / (256 CUs x
    2.4 GHz).  (SQ_ACTIVE_INST_VALU, the SIMD quad-cycles spent on VALU
    work, equals INSTS_VALU to within 1% on these kernels, so the 64-bit
    integer products of Philox issue at the full rate.)"""
    import statistics
    ctr = {}
    for d in dirs.split(","):
        for name, cname, v in _rocpd_rows(d, "select kernel_name, counter_name, value from counters_collection"):
            ctr.setdefault((_short(name), cname), []).append(float(v))
    dur = {}
    for name, du in _rocpd_rows(trace_dir, "select name, duration from kernels"):
        dur.setdefault(_short(name), []).append(du / 1e3)
    lines = ["# rocprofv3 PMC summary: VALU work of the ALU-bound rows (medians per dispatch)",
             f"# command: {command}", f"# source_digest: {source_digest()}",
             "# t_valu = SQ_INSTS_VALU / (256 CUs x 2.4 GHz): one wave64 VALU instruction per CU per cycle",
             "# (SQ_ACTIVE_INST_VALU, SIMD quad-cycles of VALU work, is within 1% of SQ_INSTS_VALU);",
             "# frac = t_valu / traced median duration",
             f"{'row':44s} {'waves':>8s} {'VALU/wave':>10s} {'INT64/wave':>10s} {'VALU/elem':>10s} "
             f"{'t_valu us':>10s} {'traced us':>10s} {'frac':>6s}"]
    for prefix, label, n in ALU_ROWS:
        kn = next((k for (k, c) in ctr if k.startswith(prefix)), None)
        if kn is None:
            lines.append(f"{label:44s} (no counters)")
            continue

        def med(c):
            v = ctr.get((kn, c))
            return statistics.median(v) if v else float("nan")
        waves, valu, i64 = med("SQ_WAVES"), med("SQ_INSTS_VALU"), med("SQ_INSTS_VALU_INT64")
        t_valu = valu / (CUS * CLOCK_HZ) * 1e6
        kd = next((k for k in dur if k.startswith(prefix)), None)
        t = statistics.median(dur[kd]) if kd else float("nan")
        lines.append(f"{label:44s} {waves:8.0f} {valu / waves:10.1f} {i64 / waves:10.1f} {valu * 64 / n:10.2f} "
                     f"{t_valu:10.2f} {t:10.2f} {t_valu / t:6.3f}")
        for c in ("SQ_ACTIVE_INST_VALU", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_SALU", "GRBM_GUI_ACTIVE"):
            if (kn, c) in ctr:
                lines.append(f"    {c}: {med(c):.0f}")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--graph-steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=6)
    ap.add_argument("--breakdown-iters", type=int, default=30)
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--sweep-rows", type=lambda v: [int(r) for r in v.split(",")],
                    default=[128, 256, 512, 1024, 2048, 4096, 8192, 16384, 32768])
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum oracle time for each cpu_baseline leg")
    ap.add_argument("--oracle-row-seconds", type=float, default=1.0,
                    help="minimum oracle time per breakdown row")
    ap.add_argument("--profile-mode", choices=["headline", "copy", "fp8col", "alu"])
    ap.add_argument("--summarize-pmc", help="FETCH_headline,FETCH_copy,WRITE_headline,WRITE_copy dirs")
    ap.add_argument("--summarize-trace", help="rocprofv3 --kernel-trace output dir")
    ap.add_argument("--summarize-pmc-fp8col", help="FETCH_fp8col,FETCH_copy,WRITE_fp8col,WRITE_copy dirs")
    ap.add_argument("--summarize-valu", help="comma-separated --pmc output dirs of --profile-mode alu")
    ap.add_argument("--trace-dir", help="--kernel-trace output dir of the same mode (with --summarize-valu)")
    ap.add_argument("--out")
    ap.add_argument("--command", default="", help="the profiled command, recorded in the summary")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.out, args.command)
        return 0
    if args.summarize_valu:
        summarize_valu(args.summarize_valu, args.trace_dir, args.out, args.command)
        return 0
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.out, args.command)
        return 0
    if args.summarize_pmc_fp8col:
        sys.path.insert(0, ROOT)
        import synth
        T, H, E = 65536, 7168, 256
        counts, _ = synth.expert_counts(T, E, seed=5)
        base, ext = os.path.splitext(args.out)
        summarize_pmc_kernel(args.summarize_pmc_fp8col, args.out, args.command, "fp8col_tiles_kernel",
                             T * H // 2 + T * H // 32 + T * H + 4 * (T * H // 128),
                             "the MXFP4 -> FP8 column kernel (65536x7168, 256 Zipf(1.1) experts)")
        summarize_pmc_kernel(args.summarize_pmc_fp8col, base + "_tokblk" + ext, args.command,
                             "fp8col_tokblk_kernel",
                             T * H // 2 + T * H // 32 + T * H + 4 * H * sum((int(c) + 127) // 128 for c in counts),
                             "the MXFP4 -> FP8 column kernel with 128-token blocks (65536x7168, 256 Zipf(1.1) "
                             "experts)")
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the codec shards with no exchange (blocks and groups "
              "are independent), so run it with --gpus 1 and multiply by the GPU count.", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import block_scaled_fp4_amd as fp4
    import synth
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    if args.profile_mode == "copy":
        copy_probe(args, torch)
        return 0
    if args.profile_mode == "fp8col":
        fp8col_probe(args, torch, fp4, synth)
        return 0
    if args.profile_mode == "alu":
        alu_probe(args, torch, fp4, np, synth)
        return 0
    h = headline(args, torch, fp4, np, synth)
    if args.profile_mode:
        return 0
    total_bytes = h["q_bytes"] + h["dq_bytes"]
    value = total_bytes / (h["ms_step"] * 1e-3) / 1e9
    dom = "quantize" if h["q_ms"] >= h["d_ms"] else "dequantize"
    dom_ms = max(h["q_ms"], h["d_ms"])
    dom_bytes = h["q_bytes"] if dom == "quantize" else h["dq_bytes"]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = None
    pmc = read_pmc_summary()
    if pmc and pmc.get("source_digest") == source_digest() and dom in pmc.get("kernels", "").split():
        try:
            traffic = float(pmc[f"{dom}_hbm_bytes_per_launch"])
        except (KeyError, ValueError):
            traffic = None
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": f"mxfp4 {dom} (4096x7168 bf16)", "algorithmic_bytes_per_launch": dom_bytes}
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(h["ms_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "MXFP4 quantize+pack then dequantize of a 4096x7168 bf16 MoE dispatch "
                               "activation (Student-t(4)*0.5, 8 hot channels x30), RTN, UE8M0 scales",
                   "rows": h["rows"], "cols": h["cols"], "fmt": "mxfp4", "rounding": "rtn",
                   "buffer_sets": h["nsets"], "footprint_bytes": h["footprint"],
                   "dequantize_reads_set": f"k + {h['lag']} (codes written {h['lag']} steps earlier)"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "kernels_us": {"quantize": round(h["q_ms"] * 1e3, 2), "dequantize": round(h["d_ms"] * 1e3, 2)},
        "timing": (f"exactly {args.steps} steps in {h['mode']} of up to {h['graph_chunk']} steps, each "
                   f"replayed once between HIP events on the launch stream; per-kernel times over "
                   f"{h['kernel_calls']} calls"),
        "roofline": roof,
        "copy_reference_GBps": round(h["copy_GBps"], 1),
    }
    deferred = []
    if not args.no_breakdown:
        res["breakdown"] = breakdown(args, torch, fp4, np, synth, deferred)
    if not args.no_sweep:
        res["sweep"] = size_sweep(args, torch, fp4, np)
    for fn in deferred:
        fn()
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle for at least {args.cpu_seconds:.0f} s")
        res["cpu_baseline"] = cpu_baseline(h["xb"], min_seconds=args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
