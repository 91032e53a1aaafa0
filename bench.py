"""Benchmark of the FP8-AMAX scaled linear layer on one MI355X.

One step = the whole hot path over one batch of the workload: for every
activation (and gradient) quantised inside the step, amax -> compute_bias ->
scale-and-cast, then every FP8 product of the workload.  Weights that the
workload treats as static are quantised once before timing.  The default
workload is the Llama-2-70B-shaped single-layer inference (8192 tokens,
hidden 8192, QKV 8192->10240, O 8192->8192, gate/up 8192->28672, down
28672->8192).

Workload 6 is the chained FP8 MLP instead (Llama-2-7B MLP, 4096 tokens): one
step = the autograd Function's forward and backward (six quantisations, six
products, SwiGLU forward and backward), see bench_mlp.

Prints one JSON line: whole-step TFLOP/s (amax + bias + cast included) from
K timed steps; the roofline of the dominant kernel (the FP8 GEMM) and the
amax / cast HBM throughput from HIP events on the launch stream in K further
steps; amax and cast of each in-step tensor again with a flushed cache
("cold"); and the CPU oracle timed on a bounded sample of the same step.
"""
import argparse
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
PEAK_F16_TFLOPS = 2500.0      # MI355X dense fp16 / bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=5,
                    help="1..5 (synth.WORKLOADS) or 6 (synth.CHAINED_MLPS: the chained FP8 MLP)")
    ap.add_argument("--bias-steps", type=int, default=20,
                    help="chained MLP: untimed Adam steps whose per-tensor biases are logged")
    ap.add_argument("--cpu-tokens", type=int, default=16,
                    help="chained MLP: tokens of the CPU oracle's sample")
    ap.add_argument("--math", choices=["exact", "native-fp8"], default="exact",
                    help="product arithmetic: exact (fp16 MFMA on exactly widened FP8) or the native FP8 MFMA")
    ap.add_argument("--cpu-rows", type=int, default=512, help="rows of each product in the CPU sample")
    ap.add_argument("--cpu-cols", type=int, default=8192, help="columns of each product in the CPU sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold (cache-flushed) amax and cast measurement")
    ap.add_argument("--cold-reps", type=int, default=5)
    ap.add_argument("--no-epilogue-amax", action="store_true",
                    help="skip the epilogue measurements (output amax, accumulation) on the largest product")
    ap.add_argument("--no-delayed", action="store_true",
                    help="skip the delayed-scaling (cast with its amax folded in) measurement")
    ap.add_argument("--no-split", action="store_true",
                    help="products never split along the contraction (no workspace)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the step captured as a HIP graph and replayed")
    ap.add_argument("--quant", choices=["multi", "one-call", "three-calls"], default="multi",
                    help="how the timed steps quantise the in-step tensors: all in one fp8_quantize_multi "
                         "call, fp8_quantize per tensor, or fp8_amax -> fp8_compute_bias -> fp8_scale_cast "
                         "per tensor (the steps with per-kernel events always make the three calls, to "
                         "time each kernel)")
    ap.add_argument("--gemm", choices=["grouped", "single"], default="grouped",
                    help="how the timed steps run the products: one fp8_scaled_gemm_group call, or "
                         "fp8_scaled_gemm (fp8_scaled_gemm_ws when split) per product (the steps with "
                         "per-kernel events always run them one by one)")
    ap.add_argument("--overlap", action="store_true",
                    help="timed steps: quantise the first product's operands and run that product on "
                         "torch's stream while a second stream quantises the other tensors (then the "
                         "remaining products, after an event), with --quant multi --gemm grouped")
    ap.add_argument("--per-config", default="1,2,3,4,6",
                    help="other workloads measured in the same run (shorter: no graph, epilogue, "
                         "delayed or one-call extras; parity on an oracle sample)")
    ap.add_argument("--no-per-config", action="store_true")
    ap.add_argument("--no-native", action="store_true",
                    help="skip the same step on the native FP8 MFMA arithmetic")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy twice (HBM counter calibration)")
    ap.add_argument("--loop-gemm", type=float, metavar="SECONDS",
                    help="only run the workload's largest product back to back for SECONDS (sustained "
                         "rate; for reading power and clocks with amd-smi meanwhile)")
    ap.add_argument("--record-traffic", metavar="DIR",
                    help="only write profiles/gemm_traffic.json from rocprofv3 --pmc CSVs under DIR "
                         "(fetch/, write/, copy_fetch/, copy_write/)")
    return ap.parse_args()


def plan_of(w):
    """Launch order of one step: ('quant', tensor) before first use, then ('gemm', linear, pass)."""
    plan, done = [], set()
    for l in w.linears:
        for which in l.passes:
            need = {"fwd": (l.x, l.w), "dgrad": (l.dy, l.w), "wgrad": (l.dy, l.x)}[which]
            for n in need:
                if w.tensor(n).timed and n not in done:
                    plan.append(("quant", n))
                    done.add(n)
            plan.append(("gemm", l, which))
    return plan


def gemm_operands(l, which):
    """(a tensor, b tensor, output shape) of one product."""
    if which == "fwd":
        return l.x, l.w, (l.M, l.N)
    if which == "dgrad":
        return l.dy, l.w, (l.M, l.K)
    return l.dy, l.x, (l.N, l.K)


# Sources of the product kernels; the committed traffic record is valid only
# while they are unchanged.
GEMM_SOURCES = [os.path.join(ROOT, "fp8_precision_linear_amd", "csrc", f)
                for f in ("gemm_pipe.h", "gemm_kernel.h")]
COPY_BYTES = 256 * 1024 * 1024


def sources_sha(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_record(workload, path=None):
    """HBM bytes per launch from committed PMC counters, valid only for the
    workload and kernel sources they were taken on."""
    path = path or os.path.join(ROOT, "profiles", "gemm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != sources_sha(GEMM_SOURCES) or rec.get("workload") != workload:
        return None
    return rec


def epilogue_amax(fl, w, plan, q, outs, math, op_of, reps=9):
    """The largest product of the step three ways (interleaved, median of
    `reps`, gpu_us): alone; with the amax of its fp32 output folded in its epilogue
    (fp8_scaled_gemm_amax); and followed by a separate fp8_amax pass over
    that output, which is what quantising the output next would otherwise
    need."""
    import statistics

    import torch
    gemms = [i for i in plan if i[0] == "gemm"]
    if not gemms:
        return None
    _, l, which = max(gemms, key=lambda i: i[1].M * i[1].N * i[1].K)
    an, bn, _ = gemm_operands(l, which)
    a8, ba, _, fa = q[an]
    b8, bb, _, fb = q[bn]
    out = outs[(l.name, which)]
    amax = torch.empty(1, dtype=torch.float32, device="cuda")
    once = gpu_us

    plain = lambda: fl.scaled_gemm(op_of[which], a8, fa, ba, b8, fb, bb, math=math, out=out)
    fused = lambda: fl.scaled_gemm(op_of[which], a8, fa, ba, b8, fb, bb, math=math, out=out, amax=amax)

    def separate():
        plain()
        fl.amax(out.reshape(-1), out=amax)

    # the three variants interleaved, so that clock drift affects them alike
    ts = {"plain": [], "fused": [], "separate": []}
    for _ in range(reps):
        for k, fn in (("plain", plain), ("fused", fused), ("separate", separate)):
            ts[k].append(once(fn))
    t_plain, t_fused, t_sep = (statistics.median(ts[k]) for k in ("plain", "fused", "separate"))
    return {"product": f"{l.name}:{which}:{l.M}x{l.N}x{l.K}",
            "gemm_us": round(t_plain, 1), "gemm_with_epilogue_amax_us": round(t_fused, 1),
            "gemm_then_amax_pass_us": round(t_sep, 1),
            "saved_us": round(t_sep - t_fused, 1)}


def epilogue_accumulate(fl, w, plan, q, outs, math, op_of, reps=9):
    """The largest product of the step added into an fp32 buffer (a gradient
    accumulated over micro-batches) two ways (interleaved, median of `reps`,
    gpu_us): fp8_scaled_gemm_accumulate (the add in the product's epilogue),
    and the product into a second buffer followed by an elementwise add
    (torch's, 12 bytes an element); the plain product beside them.  The
    buffer's contents do not matter for the timing."""
    import statistics

    import torch
    gemms = [i for i in plan if i[0] == "gemm"]
    if not gemms:
        return None
    _, l, which = max(gemms, key=lambda i: i[1].M * i[1].N * i[1].K)
    an, bn, _ = gemm_operands(l, which)
    a8, ba, _, fa = q[an]
    b8, bb, _, fb = q[bn]
    out = outs[(l.name, which)]
    tmp = torch.empty_like(out)
    op = op_of[which]
    plain = lambda: fl.scaled_gemm(op, a8, fa, ba, b8, fb, bb, math=math, out=out)
    fused = lambda: fl.scaled_gemm_accumulate(op, a8, fa, ba, b8, fb, bb, out, math=math)

    def separate():
        fl.scaled_gemm(op, a8, fa, ba, b8, fb, bb, math=math, out=tmp)
        out.add_(tmp)

    ts = {"plain": [], "fused": [], "separate": []}
    for _ in range(reps):
        for k, fn in (("plain", plain), ("fused", fused), ("separate", separate)):
            ts[k].append(gpu_us(fn))
    t_plain, t_fused, t_sep = (statistics.median(ts[k]) for k in ("plain", "fused", "separate"))
    del tmp
    plain()   # the step's own output again
    return {"product": f"{l.name}:{which}:{l.M}x{l.N}x{l.K}",
            "gemm_us": round(t_plain, 1), "gemm_accumulate_us": round(t_fused, 1),
            "gemm_then_add_pass_us": round(t_sep, 1), "saved_us": round(t_sep - t_fused, 1)}


def small_batch_products(fl, w, plan, q, math, op_of, rows=(1, 8, 32, 64, 128, 256), reps=20):
    """The step's forward weights with only a few rows of activations (a
    served model decoding a small batch; 128 and 256 rows run the tiled
    kernels split along the contraction in the workspace the call is given):
    each product alone, `reps` calls
    back to back between events after a spin kernel, for each row count;
    the rate at which its weight streams from HBM.  The activation rows are
    the step's own codes (its first rows)."""
    import torch
    out = {}
    for _, l, which in (i for i in plan if i[0] == "gemm" and i[2] == "fwd"):
        an, bn, _ = gemm_operands(l, which)
        a8, ba, _, fa = q[an]
        b8, bb, _, fb = q[bn]
        line = {}
        for m in rows:
            x = a8[:m].contiguous()
            y = torch.empty(m, l.N, dtype=torch.float32, device="cuda")
            nb = fl.gemm_workspace_bytes(op_of[which], m, l.N, l.K)
            ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
            f = lambda: fl.scaled_gemm(op_of[which], x, fa, ba, b8, fb, bb, math=math, out=y,
                                       workspace=ws if nb else None)
            f()
            torch.cuda.synchronize()
            torch.cuda._sleep(200 * 2500)
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(reps):
                f()
            e.record()
            torch.cuda.synchronize()
            us = s.elapsed_time(e) * 1e3 / reps
            line[str(m)] = {"us": round(us, 1), "weight_gbs": round(l.N * l.K / (us * 1e-6) / 1e9, 1),
                            "weight_frac": round(l.N * l.K / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        out[f"{l.name}:{l.N}x{l.K}"] = line
    return out


def delayed_quant(fl, w, plan, q, x, reps=9):
    """Delayed scaling on the step's in-step tensors: one fp8_quantize_delayed
    call (the bias from the amax a previous call left, the cast, and its own
    input's amax folded in), against the current-step chain amax -> bias ->
    cast; each timed alone with HIP events, interleaved, median of `reps`.
    A 200 us spin kernel leads each timing, so that the host's argument
    checks and launches are done before the start event fires: the events
    time the GPU's work, not the host's."""
    import statistics

    import torch
    prev = torch.empty(1, dtype=torch.float32, device="cuda")

    def once(fn):
        return gpu_us(fn) * 1e-3

    per, t_chain, t_fused, elems = {}, 0.0, 0.0, 0
    for item in plan:
        if item[0] != "quant":
            continue
        n = item[1]
        codes, bias, amax, fmt = q[n]
        margin = w.tensor(n).margin
        fl.amax(x[n], out=prev)
        chain, fused = [], []
        for _ in range(reps):
            chain.append(once(lambda: (fl.amax(x[n], out=amax), fl.compute_bias(amax, fmt, margin, out=bias),
                                       fl.scale_cast(x[n], bias, fmt, out=codes))))
            fused.append(once(lambda: fl.quantize_delayed(x[n], fmt, prev, margin, out=codes, bias=bias)))
        tc, tf = statistics.median(chain), statistics.median(fused)
        k = x[n].numel()
        per[n] = {"chain_us": round(tc * 1e3, 1), "fused_us": round(tf * 1e3, 1),
                  "fused_gbs": round(3.0 * k / (tf * 1e-3) / 1e9, 1)}
        t_chain, t_fused, elems = t_chain + tc, t_fused + tf, elems + k
    if not per:
        return None
    gbs = 3.0 * elems / (t_fused * 1e-3) / 1e9
    return {"method": f"fp8_quantize_delayed: bias from the previous call's amax, cast, its input's "
                      f"amax folded in (3 B per element) vs amax -> bias -> cast (5 B); each alone, warm, HIP "
                      f"events after a spin that covers the host's launches, median of {reps}",
            "chain_us": round(t_chain * 1e3, 1), "fused_us": round(t_fused * 1e3, 1),
            "fused_gbs": round(gbs, 1), "fused_frac": round(gbs / PEAK_HBM_GBS, 4),
            "per_tensor": per}


COLD_FLUSH_BYTES = 768 << 20   # > the 256 MB Infinity Cache
COLD_CLEAN_BYTES = 512 << 20


def graph_replay(step, q, outs, steps):
    """The timed step captured once as a HIP graph (on a side stream: the
    library launches on torch's current stream, which capture redirects) and
    replayed `steps` times back to back, wall clock; every output (codes,
    biases, amaxes, products) compared bit for bit with the eager step's after
    the first replay, after the timed replays, and after one more replay that
    follows an eager step.  No host launch work per step: what launch-bound
    workloads would run at when a caller replays its step."""
    import torch

    def snapshot():
        snap = {}
        for n, (codes, bias, amax, _) in q.items():
            snap[n] = (codes.clone(), bias.clone(), amax.view(torch.int32).clone())
        for k, o in outs.items():
            snap[k] = o.view(torch.int32).clone()
        return snap

    torch.cuda.synchronize()
    step()
    torch.cuda.synchronize()
    eager = snapshot()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    def same_as_eager():
        got = snapshot()
        return all(all(torch.equal(a, b) for a, b in zip(eager[k], got[k])) if isinstance(eager[k], tuple)
                   else torch.equal(eager[k], got[k]) for k in eager)

    graph.replay()
    torch.cuda.synchronize()
    checks = [same_as_eager()]
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    checks.append(same_as_eager())
    # eager work in between, then one more replay
    step()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    checks.append(same_as_eager())
    same = all(checks)
    del graph
    return {"ms_per_step": round(ms, 4), "replays": steps, "outputs_identical_to_eager": bool(same)}


def gpu_us(fn, lead_us=200):
    """GPU time of the calls fn() makes, in us: HIP events on the launch
    stream around them, led by a spin kernel of `lead_us` so that the host's
    argument checks and launches are done before the start event fires (the
    events then time the GPU's work, not the host's)."""
    import torch
    torch.cuda.synchronize()
    torch.cuda._sleep(int(lead_us * 2500))  # >= lead_us at clocks up to 2.5 GHz
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) * 1e3


def products_call(b, flops, reps=5, rounds=3):
    """The timed step's products alone, as the step runs them (one
    fp8_scaled_gemm_group call): `reps` calls back to back between HIP
    events (after two untimed ones, with a spin kernel ahead so the host's
    launches are queued first), the median over `rounds` of the mean per
    call, and the TFLOP/s that gives; None where the step calls the products
    one by one.  Back to back because the clock sags after the GPU idles:
    a call timed alone after a synchronisation runs its first milliseconds
    slower (the 13B backward's six products ~8%)."""
    import statistics

    import torch
    if b.group is None:
        return None
    b.group.math = b.group_math = b.math
    per = []
    for _ in range(rounds):
        torch.cuda.synchronize()
        b.group.run()
        b.group.run()
        torch.cuda._sleep(200 * 2500)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            b.group.run()
        e.record()
        torch.cuda.synchronize()
        per.append(s.elapsed_time(e) * 1e3 / reps)
    us = statistics.median(per)
    tf = flops / (us * 1e-6) / 1e12
    return {"us": round(us, 1), "tflops": round(tf, 2), "frac_of_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
            "frac_of_mfma_used_peak": round(tf / mfma_used_peak("exact" if b.math == b.fl.MATH_EXACT
                                                                else "native-fp8"), 4)}


def one_call_quant(fl, w, plan, q, x, reps=9):
    """Each in-step quantisation two ways (interleaved, median of `reps`,
    gpu_us): fp8_quantize, and the three calls amax -> compute_bias ->
    scale_cast.  Same outputs bit for bit (checked here on the last
    repetition)."""
    import statistics

    import torch
    once = gpu_us

    per, chain_sum, one_sum = {}, 0.0, 0.0
    for item in plan:
        if item[0] != "quant":
            continue
        n = item[1]
        codes, bias, amax, fmt = q[n]
        margin = w.tensor(n).margin
        c2, b2, a2 = torch.empty_like(codes), torch.empty_like(bias), torch.empty_like(amax)
        chain, one = [], []
        for _ in range(reps):
            chain.append(once(lambda: (fl.amax(x[n], out=amax), fl.compute_bias(amax, fmt, margin, out=bias),
                                       fl.scale_cast(x[n], bias, fmt, out=codes))))
            one.append(once(lambda: fl.quantize(x[n], fmt, margin, out=c2, bias=b2, amax=a2)))
        assert torch.equal(codes, c2) and torch.equal(bias, b2) and torch.equal(amax.view(torch.int32),
                                                                               a2.view(torch.int32)), n
        cm, om = statistics.median(chain), statistics.median(one)
        chain_sum += cm
        one_sum += om
        per[n] = {"elements": x[n].numel(), "three_calls_us": round(cm, 2), "one_call_us": round(om, 2)}
    return {"method": "fp8_quantize vs fp8_amax -> fp8_compute_bias -> fp8_scale_cast, each tensor alone, "
                      "warm, HIP events after a spin that covers the host's launches, median of %d; outputs "
                      "identical" % reps,
            "three_calls_us": round(chain_sum, 2), "one_call_us": round(one_sum, 2), "per_tensor": per}


def cold_quant(fl, w, plan, q, x, reps, e3m4=True):
    """amax (with its clear) and cast of every in-step quantised tensor, each
    timed alone after flushing the Infinity Cache (outside the timing); median
    over `reps`, HIP events on the launch stream.  Two flushes:
      * clean: a 768 MiB scratch write, then a read of another 512 MiB buffer,
        so that the scratch's dirty lines are written back before the kernel
        runs and the cache holds nothing of use to it;
      * dirty: the scratch write alone; the timed kernel then also pays for
        writing those dirty lines back as its reads evict them.
    Each E4M3 tensor is also cast to E3M4 (its own bias, fmt_max 30), clean
    flush: that format has no hardware conversion and takes the integer path."""
    import statistics

    import torch
    scratch = torch.empty(COLD_FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    clean = torch.ones(COLD_CLEAN_BYTES // 4, dtype=torch.int32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, dirty=False):
        # flush, start event, kernel, end event queued back to back on the
        # launch stream: the flush ends before the start event on the GPU, and
        # no host-side launch latency falls between the two events
        ts = []
        for _ in range(reps):
            torch.cuda.synchronize()
            scratch.zero_()
            if not dirty:
                clean.sum()
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return statistics.median(ts)

    per, amax_b = {}, 0.0
    tot = {"amax_ms": 0.0, "cast_ms": 0.0, "elems": 0, "e3m4_ms": 0.0, "e3m4_elems": 0}
    for item in plan:
        if item[0] != "quant":
            continue
        n = item[1]
        codes, bias, amax, fmt = q[n]
        elems = x[n].numel()
        ta = timed(lambda: fl.amax(x[n], out=amax))
        tc = timed(lambda: fl.scale_cast(x[n], bias, fmt, out=codes))
        tad = timed(lambda: fl.amax(x[n], out=amax), dirty=True)
        tcd = timed(lambda: fl.scale_cast(x[n], bias, fmt, out=codes), dirty=True)
        per[n] = {"elements": elems, "amax_us": round(ta * 1e3, 2), "cast_us": round(tc * 1e3, 2),
                  "amax_gbs": round(2.0 * elems / (ta * 1e-3) / 1e9, 1),
                  "cast_gbs": round(3.0 * elems / (tc * 1e-3) / 1e9, 1),
                  "dirty_amax_gbs": round(2.0 * elems / (tad * 1e-3) / 1e9, 1),
                  "dirty_cast_gbs": round(3.0 * elems / (tcd * 1e-3) / 1e9, 1)}
        for k, t in (("amax_ms", ta), ("cast_ms", tc), ("dirty_amax_ms", tad), ("dirty_cast_ms", tcd)):
            tot[k] = tot.get(k, 0.0) + t
        tot["elems"] += elems
        if fmt == fl.E4M3 and e3m4:
            b3 = fl.compute_bias(amax, fl.E3M4, w.tensor(n).margin)
            c3 = torch.empty_like(codes)
            t3 = timed(lambda: fl.scale_cast(x[n], b3, fl.E3M4, out=c3))
            per[n]["e3m4_cast_gbs"] = round(3.0 * elems / (t3 * 1e-3) / 1e9, 1)
            tot["e3m4_ms"] += t3
            tot["e3m4_elems"] += elems
            del c3
    del scratch, clean
    if not per:
        return None
    gbs = lambda b, ms: 1.0 * b * tot["elems"] / (ms * 1e-3) / 1e9
    cast_gbs, amax_gbs = gbs(3, tot["cast_ms"]), gbs(2, tot["amax_ms"])
    return {"method": f"each kernel alone after a {COLD_FLUSH_BYTES >> 20} MiB scratch write and a "
                      f"{COLD_CLEAN_BYTES >> 20} MiB read of another buffer (dirty_*: the write alone), "
                      f"median of {reps}, HIP events",
            "cast_gbs": round(cast_gbs, 1), "cast_frac": round(cast_gbs / PEAK_HBM_GBS, 4),
            "amax_gbs": round(amax_gbs, 1), "amax_frac": round(amax_gbs / PEAK_HBM_GBS, 4),
            "dirty_cast_gbs": round(gbs(3, tot["dirty_cast_ms"]), 1),
            "dirty_amax_gbs": round(gbs(2, tot["dirty_amax_ms"]), 1),
            "e3m4_cast_gbs": round(3.0 * tot["e3m4_elems"] / (tot["e3m4_ms"] * 1e-3) / 1e9, 1)
            if tot["e3m4_ms"] > 0 else None,
            "e3m4_cast_frac": round(3.0 * tot["e3m4_elems"] / (tot["e3m4_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
            if tot["e3m4_ms"] > 0 else None,
            "per_tensor": per}


def copy_calibration():
    """A plain device-to-device copy of COPY_BYTES, twice: what FETCH_SIZE and
    WRITE_SIZE read for a known number of bytes moved."""
    import torch
    x = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(2):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 2}), flush=True)


def loop_gemm(args):
    """The workload's largest product, back to back for args.loop_gemm seconds
    (synchronising every 10 launches), on the workload's own quantised
    operands: the sustained rate, while amd-smi reads power and clocks."""
    import torch

    import fp8_precision_linear_amd as fl
    import synth
    w = synth.WORKLOADS[args.workload]
    _, l, which = max((i for i in plan_of(w) if i[0] == "gemm"), key=lambda i: i[1].M * i[1].N * i[1].K)
    an, bn, _ = gemm_operands(l, which)
    q = {}
    for n in (an, bn):
        t = w.tensor(n)
        codes, bias, _ = fl.quantize(synth.workload_tensor(w, n).cuda(), t.fmt, t.margin)
        q[n] = (codes, bias, t.fmt)
    (a8, ba, fa), (b8, bb, fb) = q[an], q[bn]
    op = {"fwd": fl.OP_FWD, "dgrad": fl.OP_DGRAD, "wgrad": fl.OP_WGRAD}[which]
    math = fl.MATH_EXACT if args.math == "exact" else fl.MATH_NATIVE_FP8
    out = fl.scaled_gemm(op, a8, fa, ba, b8, fb, bb, math=math)
    torch.cuda.synchronize()
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < args.loop_gemm:
        for _ in range(10):
            fl.scaled_gemm(op, a8, fa, ba, b8, fb, bb, math=math, out=out)
        torch.cuda.synchronize()
        n += 10
    dt = time.perf_counter() - t0
    flops = 2.0 * l.M * l.N * l.K
    print(json.dumps({"product": f"{l.name}:{which}:{l.M}x{l.N}x{l.K}", "math": args.math, "launches": n,
                      "seconds": round(dt, 2), "tflops": round(n * flops / dt / 1e12, 1)}), flush=True)


def record_traffic(d, out=None):
    """profiles/gemm_traffic.json from four rocprofv3 --pmc runs (CSV output):
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the bench's product
    kernels, and of the calibration copy.  Each counter is scaled by
    COPY_BYTES / (what it reads for the copy)."""
    import csv
    import glob

    def rows(sub):
        files = glob.glob(os.path.join(d, sub, "**", "*counter_collection.csv"), recursive=True)
        if len(files) != 1:
            raise SystemExit(f"expected one counter CSV under {sub}, found {files}")
        return list(csv.DictReader(open(files[0])))

    def per_dispatch(rs, counter, pick):
        vals = {}
        for r in rs:
            if r["Counter_Name"] == counter and pick(r["Kernel_Name"]):
                vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        return vals

    is_gemm = lambda k: "gemm_detail" in k and "gemm" in k
    is_copy = lambda k: "copyBuffer" in k or "elementwise" in k
    copy_f = max(per_dispatch(rows("copy_fetch"), "FETCH_SIZE", is_copy).values())
    copy_w = max(per_dispatch(rows("copy_write"), "WRITE_SIZE", is_copy).values())
    f_factor = COPY_BYTES / (copy_f * 1024.0)
    w_factor = COPY_BYTES / (copy_w * 1024.0)
    f = per_dispatch(rows("fetch"), "FETCH_SIZE", is_gemm)
    wr = per_dispatch(rows("write"), "WRITE_SIZE", is_gemm)
    fetch = sum(f.values()) / len(f) * 1024.0 * f_factor
    write = sum(wr.values()) / len(wr) * 1024.0 * w_factor
    import synth
    rec = {
        "workload": synth.WORKLOADS[5].name,
        "bytes_per_launch": round(fetch + write),
        "fetch_bytes_per_launch": round(fetch),
        "write_bytes_per_launch": round(write),
        "launches_fetch": len(f), "launches_write": len(wr),
        "fetch_factor": round(f_factor, 4), "write_factor": round(w_factor, 4),
        "source_sha256": sources_sha(GEMM_SOURCES),
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <DIR>/fetch -o run -- "
            "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-cold --no-epilogue-amax --no-graph "
            "--no-per-config --no-native",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <DIR>/write -o run -- "
            "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-cold --no-epilogue-amax --no-graph "
            "--no-per-config --no-native",
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <DIR>/copy_fetch -o run -- "
            "python3 bench.py --copy-calibration",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <DIR>/copy_write -o run -- "
            "python3 bench.py --copy-calibration",
            "python3 bench.py --record-traffic <DIR>",
        ],
    }
    out = out or os.path.join(ROOT, "profiles", "gemm_traffic.json")
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec), flush=True)
    table = hbm_table(rows("fetch"), rows("write"), f_factor, w_factor)
    with open(os.path.join(os.path.dirname(out), "quant_gemm_llama70b_infer_hbm_bytes.txt"), "w") as fh:
        fh.write(table)
    print(table, flush=True)


def hbm_table(fetch_rows, write_rows, f_factor, w_factor):
    """Per-kernel HBM bytes of the library's dispatches in the counter runs:
    median over the dispatches of one kernel and grid (the products one row
    per product of the step, by their order in it), scaled by the copy
    calibration."""
    import re
    import statistics

    def per_dispatch(rs, counter):
        vals = {}
        for r in rs:
            if r["Counter_Name"] == counter and "fp8lin" in r["Kernel_Name"]:
                v = vals.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], int(r["Grid_Size"]), 0.0])
                v[2] += float(r["Counter_Value"])
        return vals

    def short(k):
        m = re.search(r"(\w+)(<[^(]*>)?\(", k.replace("(anonymous namespace)::", ""))
        return (m.group(1) + (m.group(2) or "")) if m else k

    f, wr = per_dispatch(fetch_rows, "FETCH_SIZE"), per_dispatch(write_rows, "WRITE_SIZE")
    groups, order, nth_gemm = {}, [], 0
    products = ("qkv", "o", "gate", "up", "down")
    for d in sorted(f):
        name, grid, v = f[d]
        key = (short(name), grid)
        if "gemm_pp_kernel" in name or "gemm_quad_kernel" in name:
            key = (short(name) + " " + products[nth_gemm % 5], grid)
            nth_gemm += 1
        if key not in groups:
            groups[key] = []
            order.append(key)
        groups[key].append((v * 1024.0 * f_factor / 1e6, wr.get(d, [0, 0, float("nan")])[2] * 1024.0 * w_factor / 1e6))
    lines = [
        "HBM-side bytes per dispatch of the library's kernels (rocprofv3 FETCH_SIZE and WRITE_SIZE,",
        f"KiB per dispatch, scaled by the plain-copy calibration: x{f_factor:.4f} for FETCH_SIZE,",
        f"x{w_factor:.4f} for WRITE_SIZE), Llama-2-70B-shaped inference workload (8192 tokens): the",
        "timed steps (one fp8_quantize_multi + the five products), the separate-calls event pass",
        "(fp8_amax / fp8_compute_bias / fp8_scale_cast per tensor) and the delayed-scaling timings",
        "(fp8_quantize_delayed per tensor), and the weights' one-time quantisation at set-up.",
        "Median over the dispatches of each kernel and grid.",
        "One MI355X.",
        "",
        "Commands (from /tmp, TMPDIR=/tmp), then python3 bench.py --record-traffic <DIR>:",
        "  rocprofv3 --pmc FETCH_SIZE --output-format csv -d <DIR>/fetch -o run -- python3 bench.py --steps 2 "
        "--warmup 1 --no-cpu-baseline --no-cold --no-epilogue-amax --no-graph --no-per-config --no-native",
        "  rocprofv3 --pmc WRITE_SIZE --output-format csv -d <DIR>/write -o run -- (the same)",
        "  rocprofv3 --pmc FETCH_SIZE --output-format csv -d <DIR>/copy_fetch -o run -- python3 bench.py --copy-calibration",
        "  rocprofv3 --pmc WRITE_SIZE --output-format csv -d <DIR>/copy_write -o run -- python3 bench.py --copy-calibration",
        "",
        f"{'kernel':52s} {'grid':>9s} {'dispatches':>10s} {'read MB':>9s} {'written MB':>10s}",
    ]
    for key in order:
        v = groups[key]
        lines.append(f"{key[0][:52]:52s} {key[1]:9d} {len(v):10d} {statistics.median(a for a, _ in v):9.1f} "
                     f"{statistics.median(b for _, b in v):10.1f}")
    return "\n".join(lines) + "\n"


def cpu_baseline(w, host, rows, cols, results=None):
    """The oracle, as it stands, beside the GPU: amax + bias + cast of every
    quantised-in-step tensor at full size (the oracle's scalar loops, one
    thread), and a rows x cols block of every product (OpenMP over rows),
    extrapolated to the full product by its sampled fraction of the flops.
    results (a dict, optional) receives what the oracle computed, for
    parity(): "quant" name -> (amax bits, bias, codes), "gemm" (linear,
    pass) -> (output block, bound block)."""
    import numpy as np
    import oracle
    import synth

    plan = plan_of(w)
    codes, biases = {}, {}
    if results is not None:
        results.update(quant={}, gemm={})
    # static operands: quantised offline (untimed), like the GPU leg; only the
    # sampled rows are cast, with the bias of the whole tensor
    t_quant = t_gemm = 0.0
    step_quant_elems = 0
    sampled_quant_elems = 0
    for t in w.tensors:
        words = synth.bf16_words(host[t.name])
        if t.timed:
            step_quant_elems += words.size
            sampled_quant_elems += words.size
            t0 = time.perf_counter()
            a = oracle.amax_bits(words)
            b = oracle.compute_bias(a, t.fmt, t.margin)
            c = oracle.scale_cast(words, b, t.fmt)
            t_quant += time.perf_counter() - t0
            if results is not None:
                results["quant"][t.name] = (a, b, c)
            # the products below need every row their sample touches
            codes[t.name] = c
            biases[t.name] = b
        else:
            b = oracle.compute_bias(oracle.amax_bits(words), t.fmt, t.margin)
            biases[t.name] = b
            codes[t.name] = None  # cast on demand below (untimed)
    flops_sample = 0
    for item in plan:
        if item[0] != "gemm":
            continue
        _, l, which = item
        an, bn, (R, C) = gemm_operands(l, which)
        r, c = min(rows, R), min(cols, C)
        ta, tb = w.tensor(an), w.tensor(bn)
        wa, wb = synth.bf16_words(host[an]), synth.bf16_words(host[bn])
        # operands restricted to what the r x c block reads (untimed preparation)
        if which == "fwd":       # X[r, K], W[c, K]
            a8 = oracle.scale_cast(wa[:r], biases[an], ta.fmt)
            b8 = oracle.scale_cast(wb[:c], biases[bn], tb.fmt)
            fn = oracle.gemm_fwd
        elif which == "dgrad":   # dY[r, N], W[N, c]
            a8 = oracle.scale_cast(wa[:r], biases[an], ta.fmt)
            b8 = oracle.scale_cast(np.ascontiguousarray(wb[:, :c]), biases[bn], tb.fmt)
            fn = oracle.gemm_dgrad
        else:                    # dY[M, r], X[M, c]
            a8 = oracle.scale_cast(np.ascontiguousarray(wa[:, :r]), biases[an], ta.fmt)
            b8 = oracle.scale_cast(np.ascontiguousarray(wb[:, :c]), biases[bn], tb.fmt)
            fn = oracle.gemm_wgrad
        t0 = time.perf_counter()
        ref, bound = fn(a8, ta.fmt, biases[an], b8, tb.fmt, biases[bn])
        t_gemm += time.perf_counter() - t0
        contraction = {"fwd": l.K, "dgrad": l.N, "wgrad": l.M}[which]
        flops_sample += 2 * r * c * contraction
        if results is not None:
            results["gemm"][(l.name, which)] = (ref, bound)
    step_flops = w.flops()
    # extrapolate each part by its own sampled fraction
    t_step = t_quant * (step_quant_elems / max(sampled_quant_elems, 1)) + t_gemm * (step_flops / flops_sample)
    return {
        "value": step_flops / t_step / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.threads(),
        "host_cpu_count": os.cpu_count(),
        "host_affinity": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"every in-step quantisation at full size (amax+bias+cast, 1 thread, "
                   f"{t_quant:.1f} s) and "
                   + (f"the full output of every product (OpenMP over rows, {t_gemm:.1f} s)"
                      if flops_sample == step_flops else
                      f"a {rows}x{cols} output block of every product (OpenMP over rows, "
                      f"{t_gemm:.1f} s), the products extrapolated to their full size by the "
                      f"sampled fraction of the flops")),
        "seconds_sampled": round(t_quant + t_gemm, 3),
        "quant_seconds_full_size": round(t_quant, 3),
        "gemm_seconds_sampled": round(t_gemm, 3),
        "gemm_extrapolated": flops_sample != step_flops,
    }


def cpu_baseline_mlp(m, host, tokens):
    """The oracle, as it stands, on a bounded sample of the chained MLP's step:
    the first `tokens` tokens through the forward and backward (every
    quantisation, product and SwiGLU; the weights quantised whole, as each
    step does), scaled to the step: the quantisations of the weights are
    whole-step work, everything else scales with the tokens."""
    import numpy as np
    import oracle
    import synth

    T, d, f = m.tokens, m.d, m.f
    t = min(tokens, T)
    x = synth.bf16_words(host["X"])[:t]
    w1 = host["W1"].numpy().view(np.uint32)
    w2 = host["W2"].numpy().view(np.uint32)
    g = host["G"].numpy()[:t].copy().view(np.uint32)
    E4, E5 = 0, 1

    def bf16_words_of(v):
        import torch
        return synth.bf16_words(torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16))

    t0 = time.perf_counter()
    _, bw1, w1_8 = oracle.quantize(w1, E4)
    _, bw2, w2_8 = oracle.quantize(w2, E4)
    t_weights = time.perf_counter() - t0
    t0 = time.perf_counter()
    _, bx, x8 = oracle.quantize(x, E4)
    h, _ = oracle.gemm_fwd(x8, E4, bx, w1_8, E4, bw1)
    a = bf16_words_of(oracle.swiglu_fwd(h.astype(np.float32)))
    _, ba, a8 = oracle.quantize(a, E4)
    oracle.gemm_fwd(a8, E4, ba, w2_8, E4, bw2)
    _, bdy, dy8 = oracle.quantize(g, E5)
    da, _ = oracle.gemm_dgrad(dy8, E5, bdy, w2_8, E4, bw2)
    oracle.gemm_wgrad(dy8, E5, bdy, a8, E4, ba)
    dh = bf16_words_of(oracle.swiglu_bwd(h.astype(np.float32), da.astype(np.float32)))
    _, bdh, dh8 = oracle.quantize(dh, E5)
    oracle.gemm_dgrad(dh8, E5, bdh, w1_8, E4, bw1)
    oracle.gemm_wgrad(dh8, E5, bdh, x8, E4, bx)
    t_tokens = time.perf_counter() - t0
    t_step = t_weights + t_tokens * (T / t)
    return {"value": round(m.flops() / t_step / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"the first {t} of {T} tokens through the whole forward and backward "
                      f"(weights quantised whole); token work scaled by {T / t:.0f}",
            "seconds": round(t_weights + t_tokens, 2), "host_cpu_count": os.cpu_count(),
            "host_affinity": len(os.sched_getaffinity(0))}


def measure_mlp(args, m, light=False):
    """The chained FP8 MLP: x [T, d] bf16, fp32 master weights w1 [2F, d] and
    w2 [d, F], upstream gradient g [T, d] (the synthetic loss L = sum(y * g)).
    One step = FP8MLPFunction forward + backward through autograd; every
    product, quantisation and SwiGLU runs in libfp8lin (dx is computed and
    handed to autograd, which drops it: x is a leaf that needs no gradient).
    Weights are re-quantised every step, as training does.  No optimizer step
    in the timed region (the weight update is not part of the layer).
    Returns the bench line; light: only the step and per-kernel figures (no
    graph replay, bias history or CPU baseline)."""
    import torch

    import fp8_precision_linear_amd as fl
    from fp8_precision_linear_amd import mlp
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    host = {n: synth.chained_mlp_tensor(m, n) for n in m.ORDER}
    x = host["X"].cuda()
    w1 = host["W1"].cuda().requires_grad_()
    w2 = host["W2"].cuda().requires_grad_()
    g = host["G"].cuda()
    math = fl.MATH_EXACT if args.math == "exact" else fl.MATH_NATIVE_FP8
    cfg = mlp.MLPConfig(math=math)

    def step():
        w1.grad = None
        w2.grad = None
        y = mlp.FP8MLPFunction.apply(x, w1, w2, cfg)
        y.backward(g)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # per-kernel durations: K more steps with events around every launch group
    cfg.events = []
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    events, cfg.events = cfg.events, None
    if light:
        gc.enable()
        by = {}
        for kind, name, e0, e1 in events:
            by[(kind, name)] = by.get((kind, name), 0.0) + e0.elapsed_time(e1) / args.steps
        gemm_ms = sum(v for (k, _), v in by.items() if k == "gemm")
        gemm_tflops = m.flops() / (gemm_ms * 1e-3) / 1e12
        out = {"workload": m.name, "step_ms": round(ms_per_step, 4),
               "step_tflops": round(m.flops() / (ms_per_step * 1e-3) / 1e12, 2),
               "gemm_tflops": round(gemm_tflops, 2),
               "gemm_frac_of_fp8_peak": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
               "gemm_frac_of_mfma_used_peak": round(gemm_tflops / mfma_used_peak(args.math), 4),
               "step_breakdown_ms": {k: round(sum(v for (kk, _), v in by.items() if kk == k), 4)
                                     for k in ("gemm", "quant", "swiglu")},
               "parity": "every stage against the oracle in tests/test_gpu_mlp.py (not repeated here)"}
        del x, w1, w2, g, host
        torch.cuda.empty_cache()
        return out
    # the same step captured once into a HIP graph and replayed K times (no
    # host-side launch or autograd work per step); fresh leaf weights, so that
    # their gradient nodes are made on the warm-up stream, not the default one
    gw1 = w1.detach().clone().requires_grad_()
    gw2 = w2.detach().clone().requires_grad_()

    def gstep():
        gw1.grad = None
        gw2.grad = None
        mlp.FP8MLPFunction.apply(x, gw1, gw2, cfg).backward(g)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gstep()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        gstep()
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    del graph, gw1, gw2
    gc.enable()
    K = args.steps
    by = {}
    for kind, name, e0, e1 in events:
        by[(kind, name)] = by.get((kind, name), 0.0) + e0.elapsed_time(e1) / K
    T, d, f = m.tokens, m.d, m.f
    gemm_flops = {"fwd h": 2 * T * 2 * f * d, "fwd y": 2 * T * d * f, "dgrad da": 2 * T * d * f,
                  "wgrad dw2": 2 * T * d * f, "dgrad dx": 2 * T * 2 * f * d, "wgrad dw1": 2 * T * 2 * f * d}
    gemm_ms = sum(v for (k, _), v in by.items() if k == "gemm")
    gemm_tflops = sum(gemm_flops.values()) / (gemm_ms * 1e-3) / 1e12
    peak = PEAK_F16_TFLOPS if args.math == "exact" else PEAK_FP8_TFLOPS
    # HBM bytes per group: amax reads the input, the cast reads it again and
    # writes one byte per element; SwiGLU fwd reads g, u (fp32) and writes a
    # (bf16), bwd reads g, u, da and writes dg, du
    quant_bytes = {"x+w1+w2": (2 + 2 + 1) * T * d + (4 + 4 + 1) * 2 * f * d + (4 + 4 + 1) * d * f,
                   "a": (2 + 1) * T * f, "dy": (4 + 4 + 1) * T * d, "dh": (2 + 1) * T * 2 * f}
    sw_bytes = {"fwd": (8 + 2) * T * f, "bwd": (12 + 4) * T * f}
    gbs = lambda b, ms: b / (ms * 1e-3) / 1e9

    hist = None
    if args.bias_steps > 0:
        # untimed: Adam on a regression towards a fixed target, so that the
        # tensors (and with them the biases) move as in training
        log = mlp.BiasLog()
        tcfg = mlp.MLPConfig(math=math, log=log)
        p1 = w1.detach().clone().requires_grad_()
        p2 = w2.detach().clone().requires_grad_()
        with torch.no_grad():
            target = mlp.mlp_forward(x, w1.detach() * 3, w2.detach() * 3, mlp.MLPConfig(math=math))[0]
        opt = torch.optim.Adam([p1, p2], lr=1e-3)
        losses = []
        for _ in range(args.bias_steps):
            y = mlp.FP8MLPFunction.apply(x, p1, p2, tcfg)
            loss = ((y - target) ** 2).mean()
            opt.zero_grad()
            loss.backward()
            opt.step()
            losses.append(loss.detach())
        hist = {"per_tensor_bias": log.history(),
                "loss": [round(float(v), 6) for v in torch.stack(losses).cpu()],
                "method": f"{args.bias_steps} untimed Adam steps (lr 1e-3) on mean((y - y_t)^2), "
                          f"y_t the same MLP with weights x3"}
        del p1, p2, opt, target

    line = {
        "metric": "chained FP8 MLP fwd+bwd TFLOP/s (six FP8-AMAX products, quantisations and SwiGLU included)",
        "value": round(m.flops() / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {"workload": m.name, "tokens": T, "d": d, "f": f, "math": args.math,
                   "weights": "fp32 masters, re-quantised each step", "accumulate": "f32",
                   "input_sha256": {n: synth.sha256(host[n]) for n in m.ORDER},
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "kernel": "the six products (gemm_pp_kernel)",
                     "achieved": round(gemm_tflops, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
                     "mfma_used_peak": peak,
                     "frac_of_mfma_used_peak": round(gemm_tflops / peak, 4),
                     "traffic": None,
                     "per_product_us": {n: round(by[("gemm", n)] * 1e3, 1) for n in gemm_flops}},
        "swiglu": {n: {"us": round(by[("swiglu", n)] * 1e3, 1),
                       "gbs": round(gbs(b, by[("swiglu", n)]), 1),
                       "frac": round(gbs(b, by[("swiglu", n)]) / PEAK_HBM_GBS, 4)}
                   for n, b in sw_bytes.items()},
        "quantise": {n: {"us": round(by[("quant", n)] * 1e3, 1),
                         "gbs": round(gbs(b, by[("quant", n)]), 1),
                         "frac": round(gbs(b, by[("quant", n)]) / PEAK_HBM_GBS, 4)}
                     for n, b in quant_bytes.items()},
        "step_breakdown_ms": {k: round(sum(v for (kk, _), v in by.items() if kk == k), 4)
                              for k in ("gemm", "quant", "swiglu")},
        "hip_graph": {"ms_per_step": round(graph_ms, 4),
                      "value": round(m.flops() / (graph_ms * 1e-3) / 1e12, 2),
                      "method": "the same forward + backward captured once with torch.cuda.graph, "
                                f"{K} replays timed"},
        "bias_history": hist,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_mlp(m, host, args.cpu_tokens)
        line["cpu_baseline"]["vs_gpu"] = round(line["value"] / line["cpu_baseline"]["value"], 1)
    return line


def parity(fl, w, q, outs, results):
    """The GPU step's outputs against what cpu_baseline's oracle computed on
    the same inputs: codes, amax and bias of every in-step quantisation bit
    for bit, and the sampled output block of every product within
    1e-5 * 2^-(ba+bb) * sum |a||b| elementwise.  Reports the worst
    err / (2^-(ba+bb) * sum |a||b|) over the checked outputs."""
    import numpy as np
    import torch

    quant_ok, checked = True, 0
    for n, (a_bits, b, codes) in results["quant"].items():
        g_codes, g_bias, g_amax, _ = q[n]
        quant_ok &= (int(g_amax.view(torch.int32).item()) & 0xFFFFFFFF) == a_bits
        quant_ok &= int(g_bias.item()) == b
        quant_ok &= bool(np.array_equal(g_codes.cpu().numpy().reshape(-1), np.asarray(codes).reshape(-1)))
    worst, within = 0.0, True
    for key, (ref, bound) in results["gemm"].items():
        r, c = ref.shape
        got = outs[key][:r, :c].cpu().numpy().astype(np.float64)
        err = np.abs(got - ref)
        within &= bool(np.all(err <= 1e-5 * bound))
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
        worst = max(worst, float(ratio.max()) if ratio.size else 0.0)
        checked += ref.size
    return {"quantisation_bit_exact": bool(quant_ok),
            "quantised_tensors": sorted(results["quant"]),
            "gemm_within_tolerance": within, "gemm_worst_err_over_sum_ab": worst,
            "gemm_tolerance": 1e-5, "gemm_outputs_checked": checked,
            "method": "the last timed step's outputs against the oracle's (cpu_baseline's sample): "
                      "codes, amax and bias bit for bit; the product blocks elementwise"}


class Bench:
    """One workload set up on the GPU: its synthetic inputs (host and device),
    static weights quantised once, the step's output and workspace buffers,
    and the step itself (one pass of every in-step quantisation and every
    product, on torch's current stream)."""

    def __init__(self, fl, w, args):
        import torch
        import synth

        self.fl, self.w, self.args = fl, w, args
        dev = torch.device("cuda:0")
        self.plan = plan_of(w)
        self.host = {t.name: synth.workload_tensor(w, t.name) for t in w.tensors}
        self.x = {n: v.to(dev) for n, v in self.host.items()}
        self.q = {}   # name -> (codes, bias, amax, fmt)
        for t in w.tensors:
            codes = torch.empty(t.shape, dtype=torch.uint8, device=dev)
            bias = torch.empty(1, dtype=torch.int32, device=dev)
            amax = torch.empty(1, dtype=torch.float32, device=dev)
            self.q[t.name] = (codes, bias, amax, t.fmt)
            if not t.timed:   # static weights: quantised once, outside the timed step
                fl.amax(self.x[t.name], out=amax)
                fl.compute_bias(amax, t.fmt, t.margin, out=bias)
                fl.scale_cast(self.x[t.name], bias, t.fmt, out=codes)
        self.outs = {}
        for item in self.plan:
            if item[0] == "gemm":
                _, l, which = item
                self.outs[(l.name, which)] = torch.empty(gemm_operands(l, which)[2], dtype=torch.float32,
                                                         device=dev)
        self.math = fl.MATH_EXACT if args.math == "exact" else fl.MATH_NATIVE_FP8
        self.op_of = {"fwd": fl.OP_FWD, "dgrad": fl.OP_DGRAD, "wgrad": fl.OP_WGRAD}
        # products whose outputs have too few tiles to fill the chip run split
        # along the contraction in a workspace allocated here, once (the
        # library allocates nothing)
        self.ws_of, self.ws = {}, None
        if not args.no_split:
            for item in self.plan:
                if item[0] == "gemm":
                    _, l, which = item
                    self.ws_of[(l.name, which)] = fl.gemm_workspace_bytes(self.op_of[which], l.M, l.N, l.K)
            need = max(self.ws_of.values(), default=0)
            self.ws = torch.empty(need, dtype=torch.uint8, device=dev) if need > 0 else None
        self.split_products = [f"{k[0]}:{k[1]}" for k, v in self.ws_of.items() if v > 0]
        # the step's in-step quantisations as one call, and its products as one
        # grouped call, prepared once (descriptors and workspace)
        self.quant_names = [i[1] for i in self.plan if i[0] == "quant"]
        self.group = None
        if args.gemm == "grouped":
            prods, outs = [], []
            for item in self.plan:
                if item[0] == "gemm":
                    _, l, which = item
                    an, bn, _ = gemm_operands(l, which)
                    a8, ba, _, fa = self.q[an]
                    b8, bb, _, fb = self.q[bn]
                    prods.append((self.op_of[which], a8, fa, ba, b8, fb, bb))
                    outs.append(self.outs[(l.name, which)])
            self.group_math = self.math
            self.group = fl.GemmGroup(prods, outs=outs, math=self.math)
        names = self.quant_names
        self.qmulti = fl.QuantizeMulti([self.x[n] for n in names], [self.q[n][3] for n in names],
                                       [w.tensor(n).margin for n in names],
                                       outs=[self.q[n][:3] for n in names]) if names else None
        # --overlap: the first product's in-step operands, then that product,
        # on torch's stream; the other quantisations on a second stream
        # (default priority) meanwhile; the other products after its event
        self.overlap = None
        gemms = [i for i in self.plan if i[0] == "gemm"]
        if args.overlap and self.group is not None and names and gemms:
            first_ops = [n for n in gemm_operands(gemms[0][1], gemms[0][2])[:2] if n in names]
            rest = [n for n in names if n not in first_ops]
            if first_ops and rest and len(gemms) > 1:
                mk_q = lambda ns: fl.QuantizeMulti([self.x[n] for n in ns], [self.q[n][3] for n in ns],
                                                   [w.tensor(n).margin for n in ns],
                                                   outs=[self.q[n][:3] for n in ns])

                def mk_g(items):
                    prods, outs = [], []
                    for _, l, which in items:
                        an, bn, _ = gemm_operands(l, which)
                        a8, ba, _, fa = self.q[an]
                        b8, bb, _, fb = self.q[bn]
                        prods.append((self.op_of[which], a8, fa, ba, b8, fb, bb))
                        outs.append(self.outs[(l.name, which)])
                    return fl.GemmGroup(prods, outs=outs, math=self.math)
                self.overlap = {"q_first": mk_q(first_ops), "q_rest": mk_q(rest), "g_first": mk_g(gemms[:1]),
                                "g_rest": mk_g(gemms[1:]), "side": torch.cuda.Stream(),
                                "event": torch.cuda.Event(), "first": first_ops, "rest": rest}

    def event_calls(self):
        """The step as direct library calls (every argument prepared here, so
        that the HIP events around each call bracket only its launch): for
        each in-step tensor fp8_amax, fp8_compute_bias, fp8_scale_cast; then
        for each product fp8_scaled_gemm (fp8_scaled_gemm_ws when split).  As
        in the timed step, every quantisation comes before the products, so
        the products run back to back: with memory-bound quantisations
        between them (the plan's first-use order) the clock recovers under
        the power limit, and the 13B backward's products measured ~8% faster
        that way than they run in the step."""
        import ctypes

        import torch
        fl, w, q, x = self.fl, self.w, self.q, self.x
        P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        calls = []
        for item in self.plan:
            if item[0] == "quant":
                n = item[1]
                codes, bias, amax, fmt = q[n]
                dt = fl.BF16 if x[n].dtype == torch.bfloat16 else fl.FP32
                calls.append(("amax", n, fl.lib.fp8_amax, (P(x[n]), dt, x[n].numel(), P(amax), st)))
                calls.append(("bias", n, fl.lib.fp8_compute_bias, (P(amax), fmt, w.tensor(n).margin, P(bias), st)))
                calls.append(("cast", n, fl.lib.fp8_scale_cast,
                              (P(x[n]), dt, x[n].numel(), P(bias), fmt, P(codes), st)))
        for item in self.plan:
            if item[0] == "quant":
                continue
            _, l, which = item
            an, bn, _ = gemm_operands(l, which)
            a8, ba, _, fa = q[an]
            b8, bb, _, fb = q[bn]
            args = (self.op_of[which], self.math, P(a8), fa, P(ba), P(b8), fb, P(bb), l.M, l.N, l.K,
                    P(self.outs[(l.name, which)]))
            if self.ws_of.get((l.name, which), 0) > 0:
                calls.append(("gemm", (l.name, which), fl.lib.fp8_scaled_gemm_ws,
                              args + (P(self.ws), self.ws.numel(), st)))
            else:
                calls.append(("gemm", (l.name, which), fl.lib.fp8_scaled_gemm, args + (st,)))
        return calls

    def step_events(self, ev, calls):
        import torch
        for kind, key, fn, args in calls:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            status = fn(*args)
            e1.record()
            if status != 0:
                raise RuntimeError(f"{fn.__name__}: status {status}")
            ev.append((kind, key, e0, e1))

    def step(self):
        """One timed step: the in-step quantisations (one fp8_quantize_multi
        call, or per tensor), then the products (one fp8_scaled_gemm_group
        call, or per product), all on torch's current stream."""
        fl, w, q, x = self.fl, self.w, self.q, self.x
        if self.overlap is not None:
            import torch
            o, main = self.overlap, torch.cuda.current_stream()
            for g in (o["g_first"], o["g_rest"]):
                g.math = self.math
            # the side stream first waits for everything before (the previous
            # step's products read the codes it is about to rewrite)
            o["side"].wait_stream(main)
            with torch.cuda.stream(o["side"]):
                o["q_rest"].run()
                o["event"].record()
            o["q_first"].run()
            o["g_first"].run()
            main.wait_event(o["event"])
            o["g_rest"].run()
            return
        if self.args.quant == "multi":
            if self.qmulti is not None:
                self.qmulti.run()
        else:
            for n in self.quant_names:
                codes, bias, amax, fmt = q[n]
                if self.args.quant == "one-call":
                    fl.quantize(x[n], fmt, w.tensor(n).margin, out=codes, bias=bias, amax=amax)
                else:
                    fl.amax(x[n], out=amax)
                    fl.compute_bias(amax, fmt, w.tensor(n).margin, out=bias)
                    fl.scale_cast(x[n], bias, fmt, out=codes)
        if self.group is not None:
            if self.group_math != self.math:   # the arithmetic was switched after set-up
                self.group.math = self.math
                self.group_math = self.math
            self.group.run()
            return
        for item in self.plan:
            if item[0] != "gemm":
                continue
            _, l, which = item
            an, bn, _ = gemm_operands(l, which)
            a8, ba, _, fa = q[an]
            b8, bb, _, fb = q[bn]
            fl.scaled_gemm(self.op_of[which], a8, fa, ba, b8, fb, bb, math=self.math, out=self.outs[(l.name, which)],
                           workspace=self.ws if self.ws_of.get((l.name, which), 0) > 0 else None)

    def measure(self, steps, warmup):
        """K timed steps (wall clock, synchronised on both sides, no events and
        no Python garbage collection inside), then K more steps with HIP
        events around every launch (on the launch stream) for per-kernel
        durations.  Returns the step and per-kernel figures."""
        import statistics

        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        gc.collect()
        gc.disable()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
        ev, step_ev = [], []
        calls = self.event_calls()
        # Where the host takes longer to enqueue a step's calls than the GPU
        # to run them (small workloads), a spin kernel leads each event-timed
        # step for the difference, so that the step's launches and events are
        # queued before the GPU reaches them and each event pair brackets its
        # kernel alone rather than the gaps between launches; where the GPU is
        # the slower one (the queue runs ahead by itself) there is no spin.
        warm = []
        t0 = time.perf_counter()
        self.step_events(warm, calls)
        host_us = (time.perf_counter() - t0) * 1e6
        torch.cuda.synchronize()
        spin_us = max(0.0, 1.5 * host_us - ms_per_step * 1e3)
        spin_cycles = int(spin_us * 2500)  # >= spin_us at clocks up to 2.5 GHz
        for _ in range(steps):
            if spin_cycles:
                torch.cuda._sleep(spin_cycles)
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record()
            self.step_events(ev, calls)
            s1.record()
            step_ev.append((s0, s1))
        torch.cuda.synchronize()
        gc.enable()
        r = {"ms_per_step": ms_per_step, "event_step_spin_us": round(spin_us, 1),
             "step_median_ms": statistics.median(a.elapsed_time(b) for a, b in step_ev),
             "gemm_ms": 0.0, "amax_ms": 0.0, "bias_ms": 0.0, "cast_ms": 0.0,
             "cast_by": {}, "amax_by": {}, "steps": steps}
        for kind, key, e0, e1 in ev:
            t = e0.elapsed_time(e1)
            r[kind + "_ms"] += t
            if kind in ("amax", "cast"):
                r[kind + "_by"][key] = r[kind + "_by"].get(key, 0.0) + t
        K = steps
        w = self.w
        r["step_flops"] = w.flops()
        r["gemm_launches"] = sum(1 for i in self.plan if i[0] == "gemm")
        r["quant_elems"] = sum(self.x[i[1]].numel() for i in self.plan if i[0] == "quant")
        r["step_tflops"] = r["step_flops"] / (ms_per_step * 1e-3) / 1e12
        r["gemm_tflops"] = r["step_flops"] * K / (r["gemm_ms"] * 1e-3) / 1e12
        r["cast_gbs"] = 3.0 * r["quant_elems"] * K / (r["cast_ms"] * 1e-3) / 1e9 if r["cast_ms"] > 0 else None
        r["amax_gbs"] = 2.0 * r["quant_elems"] * K / (r["amax_ms"] * 1e-3) / 1e9 if r["amax_ms"] > 0 else None
        return r


# the peak of the MFMA each arithmetic runs its contraction on: the exact
# arithmetic the 16-bit MFMA (FP8 widened exactly), the native one the FP8 MFMA
def mfma_used_peak(math):
    return PEAK_F16_TFLOPS if math == "exact" else PEAK_FP8_TFLOPS


def per_config_line(fl, wl, args):
    """A shorter measurement of another workload in the same run: its step
    (wall clock), GEMM TFLOP/s (events) as a fraction of the dense FP8 peak
    and of the peak of the MFMA the arithmetic uses, amax / cast GB/s in the
    step and cold, and parity of the last timed step against the oracle
    (every output of workloads of at most 200 GFLOP a step, else a 64 x 1024
    block of every product)."""
    import torch
    import synth

    if wl in synth.CHAINED_MLPS:
        return measure_mlp(args, synth.CHAINED_MLPS[wl], light=True)
    w = synth.WORKLOADS[wl]
    b = Bench(fl, w, args)
    r = b.measure(args.steps, args.warmup)
    cold = None if args.no_cold else cold_quant(fl, w, b.plan, b.q, b.x, 3, e3m4=False)
    res = {}
    full = w.flops() <= 2e11
    cpu = cpu_baseline(w, b.host, 1 << 31 if full else 64, 1 << 31 if full else 1024, results=res)
    out = {
        "workload": w.name,
        "step_ms": round(r["ms_per_step"], 4),
        "separate_calls_step_ms_events": round(r["step_median_ms"], 4),
        "step_tflops": round(r["step_tflops"], 2),
        "gemm_tflops": round(r["gemm_tflops"], 2),
        "gemm_frac_of_fp8_peak": round(r["gemm_tflops"] / PEAK_FP8_TFLOPS, 4),
        "gemm_frac_of_mfma_used_peak": round(r["gemm_tflops"] / mfma_used_peak(args.math), 4),
        "gemm_avg_launch_us": round(r["gemm_ms"] * 1e3 / (r["steps"] * r["gemm_launches"]), 2),
        "cast_gbs_in_step": round(r["cast_gbs"], 1) if r["cast_gbs"] else None,
        "amax_gbs_in_step": round(r["amax_gbs"], 1) if r["amax_gbs"] else None,
        "cold_cast_gbs": cold["cast_gbs"] if cold else None,
        "cold_amax_gbs": cold["amax_gbs"] if cold else None,
        "split_along_contraction": b.split_products,
        "step_products_call": products_call(b, w.flops()),
        "parity": parity(fl, w, b.q, b.outs, res),
        "oracle_tflops": round(cpu["value"], 4),
    }
    if r["ms_per_step"] < 1.0 and not args.no_graph:
        # launch-bound: the same step replayed from a HIP graph
        g = graph_replay(b.step, b.q, b.outs, args.steps)
        g["tflops"] = round(w.flops() / (g["ms_per_step"] * 1e-3) / 1e12, 2)
        out["hip_graph"] = g
    if not args.no_native and args.math == "exact":
        b.math = fl.MATH_NATIVE_FP8
        rn = b.measure(args.steps, args.warmup)
        out["native_fp8"] = {"step_tflops": round(rn["step_tflops"], 2),
                             "gemm_tflops": round(rn["gemm_tflops"], 2),
                             "gemm_frac_of_fp8_peak": round(rn["gemm_tflops"] / PEAK_FP8_TFLOPS, 4),
                             "parity": parity(fl, w, b.q, b.outs, res)}
    del b
    gc.collect()
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(args.record_traffic)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU (no multi-GPU path); --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.loop_gemm:
        loop_gemm(args)
        return
    import torch

    import fp8_precision_linear_amd as fl
    import synth

    if args.workload in synth.CHAINED_MLPS:
        print(json.dumps(measure_mlp(args, synth.CHAINED_MLPS[args.workload])), flush=True)
        return
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = synth.WORKLOADS[args.workload]
    b = Bench(fl, w, args)
    plan, q, x, outs, host = b.plan, b.q, b.x, b.outs, b.host
    r = b.measure(args.steps, args.warmup)
    K = args.steps
    gemm_ms, amax_ms, bias_ms, cast_ms = r["gemm_ms"], r["amax_ms"], r["bias_ms"], r["cast_ms"]
    step_flops, gemm_tflops, quant_elems = r["step_flops"], r["gemm_tflops"], r["quant_elems"]
    cast_gbs, amax_gbs = r["cast_gbs"], r["amax_gbs"]

    graph_info = None if args.no_graph else graph_replay(b.step, q, outs, args.steps)
    cold = None if args.no_cold else cold_quant(fl, w, plan, q, x, args.cold_reps)
    epi = None if args.no_epilogue_amax else epilogue_amax(fl, w, plan, q, outs, b.math, b.op_of)
    acc = None if args.no_epilogue_amax else epilogue_accumulate(fl, w, plan, q, outs, b.math, b.op_of)
    small = None if args.no_epilogue_amax else small_batch_products(fl, w, plan, q, b.math, b.op_of)
    delayed = None if args.no_delayed else delayed_quant(fl, w, plan, q, x)
    one_call = None if args.no_delayed else one_call_quant(fl, w, plan, q, x)
    # the timed step's own quantisation call (one fp8_quantize_multi over every
    # in-step tensor), alone: median of 9, gpu_us
    step_call_us = None
    if b.qmulti is not None:
        import statistics
        step_call_us = statistics.median(gpu_us(b.qmulti.run) for _ in range(9))

    rec = traffic_record(w.name)
    traffic = rec["bytes_per_launch"] if rec else None
    n_quant = len([i for i in plan if i[0] == "quant"])

    line = {
        "metric": "FP8-AMAX scaled GEMM TFLOP/s incl. amax+cast; cast GB/s vs HBM peak",
        "value": round(r["step_tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "separate_calls_step_ms_events": round(r["step_median_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "tokens": w.linears[0].M,
            "products": [f"{l.name}:{p}:{l.M}x{l.N}x{l.K}" for l in w.linears for p in l.passes],
            "in_step_quantised": [i[1] for i in plan if i[0] == "quant"],
            "accumulate": "f32",
            "input_sha256": {t.name: synth.sha256(host[t.name]) for t in w.tensors},
            "math": args.math,
            "split_along_contraction": b.split_products,
            "quantisation": {"multi": "fp8_quantize_multi: every in-step tensor in one call (clear, amax "
                                      "and cast launches for all of them)",
                             "one-call": "fp8_quantize per tensor (one workgroup up to 256 KiB, else clear, "
                                         "amax and a cast deriving the bias)",
                             "three-calls": "fp8_amax -> fp8_compute_bias -> fp8_scale_cast per tensor"}[args.quant],
            "product_calls": ("fp8_scaled_gemm_group: every product in one call (the training-step products in "
                              "one launch, other format pairs a launch per layout; products of 1024 or more "
                              "tiles alone)" if args.gemm == "grouped"
                         else "fp8_scaled_gemm per product (fp8_scaled_gemm_ws when split)"),
            "products_grouped_ws_bytes": b.group.ws_bytes if b.group is not None else None,
            "overlapped_quantisation": ({"side_stream": b.overlap["rest"], "before_first_product": b.overlap["first"]}
                                        if b.overlap is not None else None),
            "parallelism": "single-gpu",
        },
        # the GEMM's bound is the dense FP8 MFMA peak (its operands are FP8);
        # the exact arithmetic issues the 16-bit MFMA, whose peak is half of it
        "roofline": {
            "bound": "mfma",
            "kernel": ("gemm_pp_kernel (256x256 tiles, ping-pong waves), exact math: FP8 codes "
                       "widened to fp16, 32x32x16 fp16 MFMA" if args.math == "exact" else
                       "gemm_pp_kernel (256x256 tiles, ping-pong waves), native 32x32x64 FP8 MFMA"),
            "achieved": round(gemm_tflops, 2),
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
            "traffic": traffic,
            "mfma_used_peak": mfma_used_peak(args.math),
            "frac_of_mfma_used_peak": round(gemm_tflops / mfma_used_peak(args.math), 4),
            "avg_launch_us": round(gemm_ms * 1e3 / (K * r["gemm_launches"]), 2),
            "flops_per_launch_avg": step_flops / r["gemm_launches"],
        },
        "cast": {
            "bound": "hbm", "unit": "GB/s", "peak": PEAK_HBM_GBS,
            "achieved": round(cast_gbs, 1) if cast_gbs else None,
            "frac": round(cast_gbs / PEAK_HBM_GBS, 4) if cast_gbs else None,
            "bytes_per_element": 3,
            "avg_launch_us": round(cast_ms * 1e3 / max(K * n_quant, 1), 2),
            "per_tensor": {n: {"elements": x[n].numel(), "us": round(t * 1e3 / K, 2),
                               "gbs": round(3.0 * x[n].numel() / (t * 1e-3 / K) / 1e9, 1)}
                           for n, t in r["cast_by"].items()},
        },
        "amax": {
            "bound": "hbm", "unit": "GB/s", "peak": PEAK_HBM_GBS,
            "achieved": round(amax_gbs, 1) if amax_gbs else None,
            "frac": round(amax_gbs / PEAK_HBM_GBS, 4) if amax_gbs else None,
            "bytes_per_element": 2,
            "per_tensor": {n: {"us": round(t * 1e3 / K, 2),
                               "gbs": round(2.0 * x[n].numel() / (t * 1e-3 / K) / 1e9, 1)}
                           for n, t in r["amax_by"].items()},
        },
        # the whole in-step quantisation: amax reads x, the cast reads it again
        # and writes the codes (5 bytes per bf16 element), clear and bias
        # launches included
        "quantise": {
            "bound": "hbm", "unit": "GB/s", "peak": PEAK_HBM_GBS,
            "achieved": round(5.0 * quant_elems * K / ((amax_ms + bias_ms + cast_ms) * 1e-3) / 1e9, 1)
            if cast_ms > 0 else None,
            "frac": round(5.0 * quant_elems * K / ((amax_ms + bias_ms + cast_ms) * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
            if cast_ms > 0 else None,
            "bytes_per_element": 5,
            "method": "separate calls per tensor (fp8_amax, fp8_compute_bias, fp8_scale_cast) with "
                      "events; step_call_*: the timed step's one fp8_quantize_multi call alone",
            "step_call_us": round(step_call_us, 1) if step_call_us else None,
            "step_call_gbs": round(5.0 * quant_elems / (step_call_us * 1e-6) / 1e9, 1) if step_call_us else None,
            "step_call_frac": round(5.0 * quant_elems / (step_call_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
            if step_call_us else None,
        },
        "cold": cold,
        "epilogue_amax": epi,
        "epilogue_accumulate": acc,
        "small_batch_products": small,
        "delayed_scaling": delayed,
        "one_call_quantisation": one_call,
        "step_products_call": products_call(b, step_flops),
        "hip_graph": None if graph_info is None else dict(
            graph_info, tflops=round(step_flops / (graph_info["ms_per_step"] * 1e-3) / 1e12, 2)),
        "step_breakdown_ms": {"gemm": round(gemm_ms / K, 4), "amax": round(amax_ms / K, 4),
                              "bias": round(bias_ms / K, 4), "cast": round(cast_ms / K, 4)},
    }
    res = None
    if not args.no_cpu_baseline:
        # small workloads (at most 200 GFLOP a step): the products' full outputs
        full = w.flops() <= 2e11
        res = {}
        line["cpu_baseline"] = cpu_baseline(w, host, 1 << 31 if full else args.cpu_rows,
                                            1 << 31 if full else args.cpu_cols, results=res)
        line["cpu_baseline"]["vs_gpu"] = round(line["value"] / line["cpu_baseline"]["value"], 1)
        line["parity"] = parity(fl, w, q, outs, res)
    if not args.no_native and args.math == "exact":
        # the same step with the products on the native FP8 MFMA (an opt-in
        # arithmetic whose error depends on the data), checked against the
        # same oracle sample
        b.math = fl.MATH_NATIVE_FP8
        rn = b.measure(args.steps, args.warmup)
        line["native_fp8"] = {
            "value": round(rn["step_tflops"], 2), "ms_per_step": round(rn["ms_per_step"], 4),
            "gemm_tflops": round(rn["gemm_tflops"], 2),
            "gemm_frac_of_fp8_peak": round(rn["gemm_tflops"] / PEAK_FP8_TFLOPS, 4),
            "parity": parity(fl, w, q, outs, res) if res is not None else None,
            "note": "fp8_scaled_gemm(FP8_GEMM_NATIVE_FP8): each 64-product instruction keeps 13 bits "
                    "below its largest product, so its error depends on the data; the library's "
                    "default products are exact (16-bit MFMA on exactly widened codes)"}
        b.math = fl.MATH_EXACT
    if not args.no_per_config:
        del b, plan, q, x, outs, host
        gc.collect()
        torch.cuda.empty_cache()
        others = [int(v) for v in args.per_config.split(",") if v and int(v) != args.workload]
        line["per_config"] = {str(wl): per_config_line(fl, wl, args) for wl in others}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
