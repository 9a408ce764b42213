"""Benchmark of the MoE decode layer on one MI355X.

A step is one call of moe_layer_decode on one batch of synthetic input: route,
group by expert, gate | up, SiLU-multiply, down, combine -- the whole hot path.
The default workload is the largest decode layer that fits one GPU: 16 tokens,
hidden 6144, 288 experts, top-8, intermediate 2048.  Inputs are resident in HBM
before the timed region starts.  To defeat the 256 MB last-level cache, every
step uses a fresh set of router logits (so it selects different experts), the
layer is replicated until the replicas hold >= 4 GiB, and a shared expert gets
its own copy per logit set (so it is re-read only after >= 1 GB of other
weights).  The K timed steps are captured once in a HIP graph; the graph is
replayed enough times to fill a window of >= 50 ms, and the figure is the
median of 5 such windows (GPU time, launch gaps between the graph's kernels
included).  The same K calls launched eagerly from Python are timed the same
way and reported as eager_ms_per_step.  The oracle runs on the host cores on a
bounded sample, on all threads and on one, and the last timed output is
compared with it (relative L2 and max relative error of the bf16 output).

Prints one JSON line.  --config picks another workload (toy_decode,
dense_gemv_e2m3, wide_decode, batched_decode, prefill).

HBM traffic.  `roofline.traffic` comes from two rocprofv3 counter runs of
`bench.py --profile-steps N` (FETCH_SIZE, then WRITE_SIZE).  Each such run
ends with an elementwise copy of COPY_BYTES, whose counters calibrate the
per-dispatch figures.  `bench.py --traffic-summary FETCH.csv WRITE.csv` turns
the two counter files into a text summary under profiles/, stamped with a hash
of the kernel sources; the JSON line carries the traffic only while that hash
matches the sources it was built from, and null otherwise.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_FP8_PEAK_TFLOPS = 5000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak
DEFAULT_CONFIG = "batched_decode"
COPY_BYTES = 512 << 20           # calibration copy: reads and writes this many bytes
PROFILES = os.path.join(ROOT, "profiles")


def kernel_of(workload, batch=1):
    """The dominant kernel of a workload (the one the roofline is quoted for)."""
    if workload == "dense_gemv_e2m3":
        return "gemv_reg_kernel" if batch == 1 else "gemv_mfma_kernel"
    return {"wide_decode": "decode1_kernel", "toy_decode": "decode1_kernel",
            "batched_decode": "decodeT_kernel", "prefill": "layer_step",
            "wide_block": "block_step", "batched_block": "block_step"}.get(workload, "kernel")


ARITH = {"bf16": "low-bit weights decoded exactly, bf16 activations, fp32 accumulate, bf16 output",
         "mxfp8": "activations quantised to MX e4m3 + UE8M0/32; MX weights on the scaled fp8 x fp6/fp4 matrix "
                  "cores (many-token path), otherwise decoded exactly against the dequantised activations; "
                  "fp32 accumulate, bf16 output"}
FMT_NAMES = {1: "e2m1+e4m3/16", 2: "e2m3+ue8m0/128", 3: "e2m1+ue8m0/32", 4: "int4+fp16/64", 5: "e2m3+e4m3/16"}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default=DEFAULT_CONFIG)
    p.add_argument("--batch", type=int, default=1, help="GEMV tokens (dense_gemv_e2m3 only)")
    p.add_argument("--fmt", type=int, default=0,
                   help="weight format of the workload (1..5; 0: the workload's own): measures the format variants")
    p.add_argument("--act", choices=("bf16", "mxfp8"), default="bf16",
                   help="activations entering gate|up: bf16, or MX e4m3 + UE8M0/32 (MOE_ACT_MXFP8)")
    p.add_argument("--replicas", type=int, default=0, help="weight replicas (0: enough for >= 4x the MALL)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--profile-steps", type=int, default=0,
                   help="only run this many eager steps after warmup, then the calibration copy "
                        "(for rocprofv3 counter runs)")
    p.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="write the HBM traffic summary of two counter runs to profiles/ and exit")
    p.add_argument("--command", default="", help="command line recorded in the traffic summary")
    return p.parse_args()


def sources_hash():
    """Hash of the HIP sources: a traffic summary is valid only for the kernels it measured."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "block_scaled_bit_moe_amd", "csrc", "*"))):
        if f.endswith((".h", ".hip", ".cpp")):
            h.update(os.path.basename(f).encode())
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_file(workload, batch, fmt=0, act="bf16"):
    """Summary file of one workload; a format or activation other than the
    workload's own gets a file of its own (its kernels and bytes differ)."""
    tag = workload if workload != "dense_gemv_e2m3" else "%s_b%d" % (workload, batch)
    if fmt:
        tag += "_fmt%d" % fmt
    if act != "bf16":
        tag += "_" + act
    return os.path.join(PROFILES, "traffic_%s_%s.txt" % (kernel_of(workload, batch), tag))


def copy_calibration(torch):
    """An elementwise copy of known size (reads COPY_BYTES, writes COPY_BYTES)."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()


def read_counters(path, counter):
    """{kernel name: [per-dispatch values of `counter`]} from a rocprofv3 counter CSV."""
    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return out


def traffic_summary(a):
    cfg_name, batch = a.config, a.batch
    want = kernel_of(cfg_name, batch)
    fetch = read_counters(a.traffic_summary[0], "FETCH_SIZE")
    write = read_counters(a.traffic_summary[1], "WRITE_SIZE")

    def pick(d, key):
        names = [n for n in d if key in n]
        if not names:
            raise SystemExit("no kernel matching %r in the counter file" % key)
        vals = [v for n in names for v in d[n]]
        return names, vals
    if want in ("layer_step", "block_step"):
        # a step of several launches (the many-token layer: route, group, gate|up,
        # down, combine; the block: norm, router scores, layer): sum them, per step
        if want == "layer_step":
            keys, first = ("pf_", "route_kernel", "mx_quant_kernel"), "pf_combine"
        else:
            keys, first = ("rmsnorm_kernel", "router_kernel", "decode1_kernel", "decodeT_kernel"), "rmsnorm_kernel"

        def step(d):
            names = [n for n in d if any(k in n for k in keys)]
            steps = sum(len(d[n]) for n in names if first in n)
            if not steps:
                raise SystemExit("no %s in the counter file" % want)
            return names, [sum(v for n in names for v in d[n]) / steps] * steps
        kn, kf = step(fetch)
        _, kw = step(write)
    else:
        kn, kf = pick(fetch, want)
        _, kw = pick(write, want)
    ckey = "neg_kernel" if any("neg_kernel" in n for n in fetch) else "elementwise_kernel"
    _, cf = pick(fetch, ckey)
    _, cw = pick(write, ckey)
    copy_kib = COPY_BYTES / 1024.0
    ff = copy_kib / cf[-1]
    wf = copy_kib / cw[-1]
    mf, mw = sum(kf) / len(kf), sum(kw) / len(kw)
    traffic = (mf * ff + mw * wf) * 1024.0
    os.makedirs(PROFILES, exist_ok=True)
    path = traffic_file(cfg_name, batch, a.fmt, a.act)
    with open(path, "w") as f:
        f.write("# HBM traffic per dispatch of %s on %s (rocprofv3 --pmc, one counter per run)\n" % (want, cfg_name))
        f.write("# command: %s\n" % a.command)
        f.write("kernel: %s\n" % (" + ".join(sorted(kn)) if want in ("layer_step", "block_step") else kn[0]))
        f.write("dispatches: %d\n" % len(kf))
        f.write("fetch_kib_per_dispatch: %.1f\n" % mf)
        f.write("write_kib_per_dispatch: %.1f\n" % mw)
        f.write("copy_bytes: %d\n" % COPY_BYTES)
        f.write("copy_fetch_kib: %.1f\n" % cf[-1])
        f.write("copy_write_kib: %.1f\n" % cw[-1])
        f.write("fetch_factor: %.4f\n" % ff)
        f.write("write_factor: %.4f\n" % wf)
        f.write("traffic_bytes_per_dispatch: %.0f\n" % traffic)
        f.write("sources_sha256_16: %s\n" % sources_hash())
    print(open(path).read())


def measured_traffic(workload, batch, fmt=0, act="bf16"):
    """Calibrated HBM bytes per dispatch from the committed summary, or None when
    there is none or the kernels changed since it was taken."""
    path = traffic_file(workload, batch, fmt, act)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("sources_sha256_16") != sources_hash():
        return None
    return float(kv["traffic_bytes_per_dispatch"])


def bytes_per_expert(cfg, inter):
    import synth
    f = cfg.fmt
    H = cfg.hidden
    return (2 * inter * (synth.code_row_bytes(f, H) + synth.scale_row_bytes(f, H))
            + H * (synth.code_row_bytes(f, inter) + synth.scale_row_bytes(f, inter)))


def topk_sets(logits, k):
    """Distinct experts selected per call (bookkeeping for the byte count)."""
    order = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :k]
    return np.unique(order)


class Timer:
    def __init__(self, torch):
        self.torch = torch
        self.e0 = torch.cuda.Event(enable_timing=True)
        self.e1 = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.torch.cuda.synchronize()
        self.e0.record()

    def stop(self):
        self.e1.record()
        self.torch.cuda.synchronize()
        return self.e0.elapsed_time(self.e1) * 1e-3      # seconds


WINDOW_S = 0.05     # each timed window lasts at least this long
WINDOWS = 5         # windows per figure; the median is reported


def _windows(torch, run_once, per_run_guess):
    """Median over WINDOWS windows of the time of one `run_once()`; each window
    repeats it enough times to last >= WINDOW_S.  Returns (median seconds per
    run, repeats per window)."""
    reps = max(1, int(np.ceil(WINDOW_S / max(per_run_guess, 1e-7))))
    t = Timer(torch)
    per = []
    for _ in range(WINDOWS):
        t.start()
        for _ in range(reps):
            run_once()
        per.append(t.stop() / reps)
    return float(np.median(per)), reps


def run_steps(torch, calls, steps, warmup):
    """Per-step seconds of `steps` calls (cycling through `calls`) after
    `warmup` untimed ones, two ways: the `steps` calls captured once in a HIP
    graph and replayed (GPU time, launch gaps inside the graph included), and
    the same calls launched eagerly from Python (adds the binding's per-call
    host cost).  Each figure is the median of WINDOWS windows of >= WINDOW_S."""
    n = len(calls)
    for i in range(warmup):
        calls[i % n]()
    torch.cuda.synchronize()
    seq = [calls[(warmup + i) % n] for i in range(steps)]

    def eager():
        for c in seq:
            c()

    t = Timer(torch)
    t.start()
    eager()
    guess = t.stop()
    eager_s, eager_reps = _windows(torch, eager, guess)

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            eager()
    torch.cuda.synchronize()
    g.replay()                      # one untimed replay
    t.start()
    g.replay()
    guess = t.stop()
    graph_s, graph_reps = _windows(torch, g.replay, guess)
    return {"per_step": graph_s / steps, "eager_per_step": eager_s / steps, "graph_replays_per_window": graph_reps,
            "eager_repeats_per_window": eager_reps, "windows": WINDOWS}


def err_figures(got_bf16_bits, ref):
    """S13(iii)-style figures of a bf16 output against the double oracle: the
    relative L2 error and the unadjusted max relative error (informational;
    the parity bar is on the fp32 output, in the tests)."""
    import oracle
    got = np.array([oracle.bf16_value(int(b)) for b in np.asarray(got_bf16_bits).ravel()]).reshape(ref.shape)
    rel_l2 = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    nz = np.abs(ref) > 0
    max_rel = float(np.max(np.abs(got - ref)[nz] / np.abs(ref)[nz])) if nz.any() else 0.0
    return {"rel_l2": rel_l2, "max_rel_unadjusted": max_rel, "elements": int(ref.size)}


def cpu_baseline_moe(cfg, seconds, logits_list, x, slice_tokens=None):
    """The oracle on the host cores, call after call of the same workload, until
    ~`seconds` of oracle time.  With slice_tokens, each call takes the next
    slice of that many tokens of the workload (for workloads whose full call
    would take the oracle minutes).  Generating the selected experts' bytes on
    the host is not timed.  Returns (tokens done, oracle seconds)."""
    import oracle
    import synth
    cache = {}
    sh = synth.expert_weights(cfg, cfg.experts) if cfg.shared_inter else None
    spent, done, tokens = 0.0, 0, 0
    T = x.shape[0]
    while spent < seconds:
        l = logits_list[done % len(logits_list)]
        xs = x
        if slice_tokens:
            t0 = (done * slice_tokens) % T
            l, xs = l[t0:t0 + slice_tokens], x[t0:t0 + slice_tokens]
        idx, _ = oracle.route(l, cfg.top_k)
        ex = {}
        for e in np.unique(idx):
            e = int(e)
            if e not in cache:
                cache[e] = synth.expert_weights(cfg, e)
            ex[e] = cache[e]
        t1 = time.perf_counter()
        oracle.layer(cfg.fmt, cfg.hidden, cfg.inter, cfg.experts, cfg.top_k, ex, xs, l, shared=sh,
                     shared_inter=cfg.shared_inter)
        spent += time.perf_counter() - t1
        done += 1
        tokens += xs.shape[0]
    return tokens, spent


def oracle_bf16_rmsnorm(x, gamma, eps):
    """The block's normalised activation as the oracle computes it (bookkeeping
    of which experts a block call selects)."""
    import oracle
    return oracle.bf16_round(oracle.rmsnorm(x, gamma, eps))


def router_scores(xn, wr):
    import oracle
    return oracle.router_logits(xn, wr).astype(np.float32)


def cpu_figures(run_sample, seconds, cores):
    """The oracle timed on all `cores` threads (~`seconds`) and on one thread
    (~seconds / 2).  run_sample(budget) returns (work units done, seconds,
    sample text).  Returns the cpu_baseline dict's parts."""
    import oracle
    oracle.set_threads(cores)
    n_all, el_all, what_all = run_sample(seconds)
    oracle.set_threads(1)
    n_one, el_one, what_one = run_sample(seconds / 2)
    oracle.set_threads(cores)
    return (n_all / el_all, what_all), (n_one / el_one, what_one)


def cpu_baseline_block(cfg, seconds, xs_host):
    """The oracle's whole block (norm, scores, routing, layer, residual) call
    after call on the host cores until ~`seconds` of oracle time.  Returns
    (tokens, seconds, sample text)."""
    import oracle
    import synth
    g, wr = synth.norm_gamma(cfg), synth.router_weights(cfg)
    sh = synth.expert_weights(cfg, cfg.experts) if cfg.shared_inter else None
    cache, spent, done, tokens = {}, 0.0, 0, 0
    while spent < seconds:
        x = xs_host[done % len(xs_host)]
        lg = router_scores(oracle_bf16_rmsnorm(x, g, cfg.norm_eps), wr)
        ex = {}
        for e in np.unique(oracle.route(lg, cfg.top_k)[0]):
            e = int(e)
            if e not in cache:
                cache[e] = synth.expert_weights(cfg, e)
            ex[e] = cache[e]
        t1 = time.perf_counter()
        oracle.block(cfg.fmt, cfg.hidden, cfg.inter, cfg.experts, cfg.top_k, ex, x, g, wr, cfg.norm_eps, shared=sh,
                     shared_inter=cfg.shared_inter)
        spent += time.perf_counter() - t1
        done += 1
        tokens += x.shape[0]
    return tokens, spent, "%d token(s) of the workload (whole blocks, fresh inputs); %.1f s of oracle time" % (
        tokens, spent)


def main():
    a = parse()
    if a.traffic_summary:
        traffic_summary(a)
        return
    if a.gpus != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(expert sharding over RCCL is a design note, not code)", file=sys.stderr)
        sys.exit(2)
    import torch
    import block_scaled_bit_moe_amd as moeq
    import synth
    from synth import configs
    from synth.device import dev_bf16, dev_u8, upload_layer_tensors

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    moeq.load_library()
    cfg = configs.ALL[a.config]
    if a.fmt:
        import dataclasses
        cfg = dataclasses.replace(cfg, fmt=a.fmt)
    cores = len(os.sched_getaffinity(0))
    omp = int(os.environ.get("OMP_NUM_THREADS", cores))
    errs = None

    if isinstance(cfg, configs.GemvConfig):
        if a.act != "bf16":
            sys.exit("--act mxfp8 applies to the layer workloads")
        B = a.batch
        c, s = synth.gemv_weights(cfg)
        wbytes = c.nbytes + s.nbytes
        R = a.replicas or max(1, -(-(1 << 30) // wbytes))
        Ws = []
        base_c, base_s = dev_u8(c), dev_u8(s)
        for r in range(R):
            cc, ss = (base_c, base_s) if r == 0 else (base_c.clone(), base_s.clone())
            Ws.append(moeq.QMat(cfg.fmt, cfg.rows, cfg.cols, cc, ss))
        xg = synth.gemv_x(cfg, B)
        x = dev_bf16(xg)
        y = torch.empty((B, cfg.rows), dtype=torch.bfloat16, device="cuda")
        calls = [(lambda W=W: moeq.dense_gemv_q(W, x, y=y)) for W in Ws]
        if a.profile_steps:
            for i in range(a.warmup + a.profile_steps):
                calls[i % len(calls)]()
            torch.cuda.synchronize()
            copy_calibration(torch)
            return
        tm = run_steps(torch, calls, a.steps, a.warmup)
        per = tm["per_step"]
        tokens_per_s = B / per
        achieved = wbytes / per / 1e9
        metric_value = tokens_per_s
        workload = {"workload": cfg.name, "rows": cfg.rows, "cols": cfg.cols, "batch": B, "fmt": FMT_NAMES[cfg.fmt],
                    "replicas": R}
        kernel = kernel_of(cfg.name, B)
        import oracle
        rows = np.arange(0, cfg.rows, 97)
        yb = y.view(torch.int16).cpu().numpy().view(np.uint16)[:, rows]
        errs = err_figures(yb, oracle.gemv(cfg.fmt, cfg.rows, cfg.cols, c, s, xg, row_list=rows))
        errs["sample"] = "every 97th row of the last timed call"
        cpu = None
        if not a.no_cpu_baseline:
            n_rows = 256

            def sample(budget):
                t0, reps = time.perf_counter(), 0
                while time.perf_counter() - t0 < budget:
                    oracle.gemv(cfg.fmt, cfg.rows, cfg.cols, c, s, xg, row_list=np.arange(n_rows) + reps)
                    reps += 1
                el = time.perf_counter() - t0
                frac = reps * n_rows / cfg.rows
                return B * frac, el, "%d row blocks of %d rows (%.4f of the matrix) x B=%d, scaled to whole GEMVs" % (
                    reps, n_rows, frac, B)
    else:
        T = cfg.tokens
        many = T > moeq.MAX_DECODE_TOKENS
        per_expert = bytes_per_expert(cfg, cfg.inter)
        layer_bytes = cfg.experts * per_expert
        R = a.replicas or max(1, min(32, -(-(4 << 30) // layer_bytes)))
        devs, shared = upload_layer_tensors(cfg)
        names = ("w13_codes", "w13_scales", "w2_codes", "w2_scales")
        routed = [[devs[n] for n in names]]
        for r in range(1, R):
            routed.append([t.clone() for t in routed[0]])
        NL = 64 if not many else 4
        # one copy of the shared expert per logit set: a call re-reads its
        # shared expert only NL calls later (>= 1 GB of other weights between)
        n_sh = NL if cfg.shared_inter else 0
        shared_copies = [shared] + [{n: shared[n].clone() for n in names} for _ in range(n_sh - 1)] if n_sh else []
        n = max(R, NL)
        layers = [moeq.Layer(cfg.fmt, cfg.hidden, cfg.inter, cfg.experts, cfg.top_k, *routed[i % R],
                             shared_inter=cfg.shared_inter, shared=shared_copies[i % n_sh] if n_sh else None)
                  for i in range(n)]
        is_block = cfg.name.endswith("_block")
        act_flag = moeq.MOE_ACT_MXFP8 if a.act == "mxfp8" else 0
        if act_flag and is_block:
            sys.exit("--act mxfp8 applies to the layer workloads")
        xh = synth.hidden_states(cfg)
        x = dev_bf16(xh)
        out = torch.empty((T, cfg.hidden), dtype=torch.bfloat16, device="cuda")
        if is_block:
            # the whole block: every call gets another residual-stream input (so
            # other experts) and the router weights are read each call
            gamma, wr = dev_bf16(synth.norm_gamma(cfg)), dev_bf16(synth.router_weights(cfg))
            blocks = [moeq.Block(Lr, gamma, wr, cfg.norm_eps) for Lr in layers]
            xs_host = [synth.hidden_states(cfg, sub=i) for i in range(NL)]
            xs = [dev_bf16(v) for v in xs_host]
            ws = moeq.block_workspace(blocks[0], T)
            calls = [(lambda i=i: moeq.moe_block_decode(blocks[i], xs[i % NL], out=out, flags=act_flag, ws=ws))
                     for i in range(n)]
            logits_host = []
            for v in xs_host:
                xn = oracle_bf16_rmsnorm(v, synth.norm_gamma(cfg), cfg.norm_eps)
                logits_host.append(router_scores(xn, synth.router_weights(cfg)))
        else:
            logits_host = [synth.router_logits(cfg, sub=i) for i in range(NL)]
            logits = [torch.from_numpy(l).cuda() for l in logits_host]
            ws = moeq.workspace(layers[0], T)
            calls = [(lambda i=i: moeq.moe_layer_decode(layers[i], x, logits[i % NL], out=out, flags=act_flag, ws=ws))
                     for i in range(n)]
        if a.profile_steps:
            for i in range(a.warmup + a.profile_steps):
                calls[i % len(calls)]()
            torch.cuda.synchronize()
            moeq.moe_workspace_status(ws)
            copy_calibration(torch)
            return
        tm = run_steps(torch, calls, a.steps, a.warmup)
        moeq.moe_workspace_status(ws)
        per = tm["per_step"]
        # algorithmic bytes: the packed codes + scales of every expert the call uses, read once
        used = [len(topk_sets(logits_host[(a.warmup + i) % NL], cfg.top_k)) + (1 if cfg.shared_inter else 0)
                for i in range(a.steps)]
        wbytes = float(np.mean(used)) * per_expert if not cfg.shared_inter else \
            float(np.mean([u - 1 for u in used])) * per_expert + bytes_per_expert(cfg, cfg.shared_inter)
        if is_block:
            wbytes += cfg.experts * cfg.hidden * 2 + cfg.hidden * 2     # router weights and norm gains
        tokens_per_s = T / per
        achieved = wbytes / per / 1e9
        metric_value = tokens_per_s
        workload = {"workload": cfg.name, "tokens": T, "hidden": cfg.hidden, "experts": cfg.experts,
                    "top_k": cfg.top_k, "inter": cfg.inter, "shared_inter": cfg.shared_inter,
                    "fmt": FMT_NAMES[cfg.fmt], "replicas": R, "logit_sets": NL, "shared_copies": n_sh,
                    "experts_read_per_call": float(np.mean(used)), "weight_bytes_per_call": wbytes}
        kernel = kernel_of(cfg.name)
        if many:
            # the matrix-core work of the step: 2 flops per multiply-add of gate, up and down
            pairs = T * (cfg.top_k + (1 if cfg.shared_inter else 0))
            flops = 2.0 * T * cfg.top_k * 3 * cfg.hidden * cfg.inter
            if cfg.shared_inter:
                flops += 2.0 * T * 3 * cfg.hidden * cfg.shared_inter
            workload["pairs"] = pairs
            workload["mfma_tflops_algorithmic"] = flops / per / 1e12
            workload["mfma_frac_of_bf16_dense_peak"] = flops / per / 1e12 / MFMA_BF16_PEAK_TFLOPS
            if act_flag:
                workload["mfma_frac_of_fp8_dense_peak"] = flops / per / 1e12 / MFMA_FP8_PEAK_TFLOPS
        # error figures of the last timed call's bf16 output against the oracle
        # (all tokens; the first 16 of a many-token call)
        last = (a.warmup + a.steps - 1) % n
        outb = out.view(torch.int16).cpu().numpy().view(np.uint16)
        nt = min(T, 16)
        import oracle
        lg = logits_host[last % NL][:nt]
        idx, _ = oracle.route(lg, cfg.top_k)
        ex = {int(e): synth.expert_weights(cfg, int(e)) for e in np.unique(idx)}
        sh = synth.expert_weights(cfg, cfg.experts) if cfg.shared_inter else None
        if is_block:
            _, _, ref, _, _ = oracle.block(cfg.fmt, cfg.hidden, cfg.inter, cfg.experts, cfg.top_k, ex,
                                           xs_host[last % NL][:nt], synth.norm_gamma(cfg), synth.router_weights(cfg),
                                           cfg.norm_eps, shared=sh, shared_inter=cfg.shared_inter)
        else:
            xr = xh[:nt]
            if act_flag:    # the reference layer on the oracle's quantised-then-dequantised activations
                xr = oracle.bf16_round(oracle.dequantize_mx_e4m3(*oracle.quantize_mx_e4m3(xr)))
            _, _, ref = oracle.layer(cfg.fmt, cfg.hidden, cfg.inter, cfg.experts, cfg.top_k, ex, xr, lg,
                                     shared=sh, shared_inter=cfg.shared_inter)
        errs = err_figures(outb[:nt], ref)
        errs["sample"] = "%d token(s) of the last timed call" % nt
        cpu = None
        if not a.no_cpu_baseline:
            def sample(budget):
                if is_block:
                    return cpu_baseline_block(cfg, budget, xs_host)
                tok, el = cpu_baseline_moe(cfg, budget, logits_host, xh, slice_tokens=16 if many else None)
                return tok, el, "%d token(s) of the workload (%s, fresh logits); %.1f s of oracle time" % (
                    tok, "slices of 16 tokens of the chunk" if many else "whole calls", el)

    if not a.no_cpu_baseline:
        (v_all, s_all), (v_one, s_one) = cpu_figures(sample, a.cpu_seconds, omp)
        cpu = {"value": v_all, "unit": "tokens/s", "cores": omp, "kind": "oracle", "sample": s_all,
               "single_thread": {"value": v_one, "unit": "tokens/s", "cores": 1, "sample": s_one}}

    traffic = measured_traffic(cfg.name, a.batch, a.fmt, a.act)
    line = {
        "metric": "MoE decode layer tokens/s and effective weight GB/s (% of 8 TB/s HBM)",
        "value": metric_value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": per * 1e3,
        "eager_ms_per_step": tm["eager_per_step"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if a.act == "bf16" else "e4m3 activations",
        "data": "synthetic (seeded generator; random-init weights of the workload's shapes)",
        "config": dict(workload, launch="hipgraph", arithmetic=ARITH[a.act], graph_replays_per_window=tm["graph_replays_per_window"],
                       eager_repeats_per_window=tm["eager_repeats_per_window"], windows=tm["windows"],
                       window_min_ms=WINDOW_S * 1e3, statistic="median of windows"),
        "effective_weight_GBps": achieved,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": kernel},
        "cpu_baseline": cpu,
        "output_error_vs_oracle": errs,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
