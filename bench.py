"""Benchmark of the joint video-audio attention hot path on one MI355X.

One step = the whole hot path of one dual-stream block on the 480p-latent
layer (21 x 30 x 52 video tokens + one conditioning frame at t = -1, 218
audio tokens, 512 text tokens, 24 heads x 128): video->text cross-attention
(unrotated video queries), time-shifted 3D RoPE of Q and K, joint
self-attention over all 35050 tokens, and both directions of the
audio<->video cross-attention.  Inputs are seeded synthetic bf16 tensors
already resident in HBM.

The JSON line reports the step's attention throughput (4 * Nq * Nk * d per
head summed over the step's attention calls, over the step time), the
joint-attention call against the bf16 matrix-core peak, the block-sparse vs
dense comparison on the 172032-token video grid, and the fp64 oracle timed on
the host over a bounded sample.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0
PEAK_CLOCK_MHZ = 2400.0         # the clock the published peaks assume


def attn_flops(nq, nk, heads, d):
    return 4.0 * nq * nk * heads * d


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-sparse", action="store_true", help="skip the block-sparse leg")
    ap.add_argument("--no-train", action="store_true",
                    help="skip the training leg (joint attention forward with lse + backward)")
    ap.add_argument("--sparse-reps", type=int, default=3)
    ap.add_argument("--no-adaptive", action="store_true", help="skip the content-adaptive block-shape leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip sampling the GPU clock and socket power under sustained joint and sparse attention")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="query rows of the oracle sample (all heads, all keys)")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run a 1 GiB device copy (counter calibration) and three joint-attention "
                         "calls on the 480p-latent layer, then exit (profile with rocprofv3 --pmc)")
    ap.add_argument("--summarize", nargs="+", metavar="CSV",
                    help="print markdown summaries of rocprofv3 csv output (kernel_trace.csv, "
                         "or FETCH_SIZE and WRITE_SIZE counter_collection.csv), then exit")
    ap.add_argument("--traffic-out", metavar="JSON",
                    help="with --summarize over the two counter files of a --traffic-probe run: "
                         "write the copy-calibrated HBM bytes per joint-attention call here")
    ap.add_argument("--probe", action="store_true",
                    help="run every kernel of the library a few times on the bench's workloads (a 1 GiB copy for "
                         "counter calibration, the 480p-latent step and training pair, the block-sparse call and "
                         "its training pair), then exit (profile with rocprofv3 --kernel-trace or --pmc)")
    ap.add_argument("--kernel-table", nargs="+", metavar="CSV",
                    help="join rocprofv3 csv files of --probe runs (kernel_trace.csv and the counter_collection.csv "
                         "of FETCH_SIZE, WRITE_SIZE, MfmaUtil passes) into one markdown table per kernel and grid: "
                         "mean duration, copy-calibrated HBM bytes and GB/s, matrix-core utilisation; then exit")
    ap.add_argument("--oracle-times", action="store_true",
                    help="time the fp64 oracle on the host cores for every workload (no GPU used): the "
                         "88-token, 5850-token and 480p-latent workloads in full, the 720p-latent and "
                         "block-sparse ones on one head, scaled to 24 heads; print a markdown table, then exit")
    return ap.parse_args()


KERNEL_SOURCES = ("attn.hip", "attn_core.hpp", "internal.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "joint_attn_480p_traffic.json")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "joint_video_audio_rope_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per joint-attention launch from the committed counter summary,
    or None when the kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


COPY_BYTES = 1 << 30            # the probe's device copy: 1 GiB read + 1 GiB written


def parse_smi_metrics(text):
    """Mean gfx clock (MHz, over the XCDs) and socket power (W) from the JSON of
    `amd-smi metric -c -p --json`; None for a value the text does not hold."""
    try:
        doc = json.loads(text)
    except ValueError:
        return None, None
    clocks, power = [], []

    def walk(o, path):
        if isinstance(o, dict):
            for key, val in o.items():
                walk(val, path + (str(key),))
        elif isinstance(o, list):
            for val in o:
                walk(val, path)
        elif isinstance(o, (int, float)) and path[-1:] == ("value",):
            if len(path) >= 4 and path[-2] == "clk" and path[-3].startswith("gfx_") and path[-4] == "clock":
                clocks.append(float(o))
            elif len(path) >= 3 and path[-2] == "socket_power" and path[-3] == "power":
                power.append(float(o))

    walk(doc, ())
    return (sum(clocks) / len(clocks) if clocks else None), (power[0] if power else None)


def clock_under(torch, fn, seconds=3.0):
    """Run fn back to back for about `seconds` while a host thread samples the
    gfx clock and socket power through amd-smi (a child process); returns the
    means over the samples taken while the GPU was busy, or None without amd-smi."""
    import shutil
    import subprocess
    import threading
    import time
    smi = shutil.which("amd-smi")
    if smi is None:
        return None
    samples, busy, stop = [], [False], [False]

    def sampler():
        while not stop[0]:
            try:
                txt = subprocess.run([smi, "metric", "-c", "-p", "--json"], capture_output=True, text=True,
                                     timeout=20).stdout
            except (OSError, subprocess.SubprocessError):
                return
            if busy[0]:
                samples.append(parse_smi_metrics(txt))
            time.sleep(0.2)

    fn()
    torch.cuda.synchronize()
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.time()
    while time.time() - t0 < seconds:
        if time.time() - t0 > 0.5:
            busy[0] = True                   # let the clock settle first
        fn()
        torch.cuda.synchronize()
    busy[0] = False
    stop[0] = True
    th.join(timeout=30)
    mhz = [c for c, _ in samples if c is not None]
    watts = [p for _, p in samples if p is not None]
    if not mhz:
        return None
    return {"gfx_mhz": round(sum(mhz) / len(mhz)), "socket_w": round(sum(watts) / len(watts)) if watts else None,
            "samples": len(mhz)}


def traffic_from_counters(means):
    """HBM bytes of one joint-attention call (V prescale, V^T staging and the
    attention kernel)
    from mean FETCH_SIZE / WRITE_SIZE KiB per dispatch, each scaled by what the
    counter reads for the 1 GiB copy."""
    def mean(part, counter):
        v = [x for (k, c), x in means.items() if part in k and c == counter]
        if len(v) != 1:
            raise SystemExit("expected one %s entry for %s, found %d" % (counter, part, len(v)))
        return v[0]

    f_scale = COPY_BYTES / (mean("copyBuffer", "FETCH_SIZE") * 1024.0)
    w_scale = COPY_BYTES / (mean("copyBuffer", "WRITE_SIZE") * 1024.0)
    out = {"fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4), "kernels": {}}
    total = 0.0
    for part in ("v_absmax_kernel", "vt_dense_kernel", "attn_bf16_kernel"):
        fb = mean(part, "FETCH_SIZE") * 1024.0 * f_scale
        wb = mean(part, "WRITE_SIZE") * 1024.0 * w_scale
        out["kernels"][part] = {"fetch_bytes": round(fb), "write_bytes": round(wb)}
        total += fb + wb
    out["bytes_per_launch"] = round(total)
    out["source_sha256"] = kernel_source_hash()
    return out


def summarize(paths, traffic_out=None):
    import collections
    import csv

    def short(name):
        name = name.replace("(anonymous namespace)::", "").replace("void ", "")
        return name.split("(")[0][:64]

    means = {}
    for path in paths:
        rows = list(csv.DictReader(open(path)))
        print("### %s\n" % os.path.basename(path))
        if rows and "Counter_Name" in rows[0]:
            g = collections.defaultdict(list)
            for r in rows:
                g[(short(r["Kernel_Name"]), r["Grid_Size"], r["Counter_Name"])].append(float(r["Counter_Value"]))
            print("| kernel | grid (threads) | counter | dispatches | mean KiB per dispatch |")
            print("|---|---|---|---|---|")
            for (k, gs, c), v in sorted(g.items()):
                print("| %s | %s | %s | %d | %.0f |" % (k, gs, c, len(v), sum(v) / len(v)))
                means[(k, c)] = sum(v) / len(v)
        else:
            g = collections.defaultdict(list)
            for r in rows:
                g[(short(r["Kernel_Name"]), r["Grid_Size_X"], r["Workgroup_Size_X"])].append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6)
            print("| kernel | grid x (threads) | workgroup | calls | avg ms | min ms | max ms |")
            print("|---|---|---|---|---|---|---|")
            for (k, gs, wg), v in sorted(g.items(), key=lambda kv: -sum(kv[1])):
                if sum(v) >= 0.05:
                    print("| %s | %s | %s | %d | %.3f | %.3f | %.3f |" % (k, gs, wg, len(v), sum(v) / len(v), min(v), max(v)))
        print()
    if traffic_out:
        t = traffic_from_counters(means)
        with open(traffic_out, "w") as f:
            json.dump(t, f, indent=1)
        print("traffic per joint-attention call: %.4g bytes (%s)" % (t["bytes_per_launch"], traffic_out))


def kernel_table(paths):
    """One markdown row per (kernel, grid) from --probe runs: mean duration
    (kernel trace), FETCH_SIZE and WRITE_SIZE scaled by what they read for the
    1 GiB copy, the GB/s they imply over that duration, and MfmaUtil."""
    import collections
    import csv

    def short(name):
        name = name.replace("(anonymous namespace)::", "").replace("void ", "")
        if name.startswith("_ZN5mmdit12_GLOBAL__N_1"):     # mangled: keep the kernel's own name
            rest = name[len("_ZN5mmdit12_GLOBAL__N_1"):]
            i = 0
            while rest[i].isdigit():
                i += 1
            name = "mmdit::" + rest[i:i + int(rest[:i])]
        return name.split("(")[0][:60]

    dur = collections.defaultdict(list)
    ctr = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in paths:
        for r in csv.DictReader(open(path)):
            if "Counter_Name" in r:
                key = (short(r["Kernel_Name"]), int(r["Grid_Size"]))
                ctr[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
            else:
                g = int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y", 1) or 1) * int(r.get("Grid_Size_Z", 1) or 1)
                dur[(short(r["Kernel_Name"]), g)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6)

    def mean(x):
        return sum(x) / len(x) if x else None

    # the 1 GiB copy is the largest copy the probe makes: its dispatch reads
    # the largest FETCH_SIZE and WRITE_SIZE of all copyBuffer dispatches
    def copy_max(counter):
        v = [x for k, c in ctr.items() if "copyBuffer" in k[0] for x in c.get(counter, [])]
        return max(v) if v else None
    f_scale = COPY_BYTES / (copy_max("FETCH_SIZE") * 1024.0) if copy_max("FETCH_SIZE") else None
    w_scale = COPY_BYTES / (copy_max("WRITE_SIZE") * 1024.0) if copy_max("WRITE_SIZE") else None
    print("Copy calibration (1 GiB copy): fetch x %s, write x %s\n" % (
        "%.4f" % f_scale if f_scale else "-", "%.4f" % w_scale if w_scale else "-"))
    print("| kernel | grid (threads) | calls | avg ms | fetch GB | write GB | GB/s | % of 8 TB/s | MfmaUtil % |")
    print("|---|---|---|---|---|---|---|---|---|")
    keys = sorted((k for k in set(dur) | set(ctr) if "mmdit" in k[0]), key=lambda k: -(sum(dur.get(k, [0])) or 0))
    for k in keys:
        d = mean(dur.get(k, []))
        c = ctr.get(k, {})
        fb = mean(c.get("FETCH_SIZE", [])) * 1024.0 * f_scale / 1e9 if c.get("FETCH_SIZE") and f_scale else None
        wb = mean(c.get("WRITE_SIZE", [])) * 1024.0 * w_scale / 1e9 if c.get("WRITE_SIZE") and w_scale else None
        mu = mean(c.get("MfmaUtil", []))
        gbs = (fb or 0) + (wb or 0)
        rate = gbs / (d * 1e-3) if d and (fb is not None or wb is not None) else None
        f = lambda x, fmt: "-" if x is None else fmt % x
        print("| %s | %d | %d | %s | %s | %s | %s | %s | %s |" % (
            k[0], k[1], len(dur.get(k, [])), f(d, "%.3f"), f(fb, "%.3f"), f(wb, "%.3f"), f(rate, "%.0f"),
            f(None if rate is None else 100 * rate / PEAK_HBM_GBS, "%.0f"), f(mu, "%.1f")))


def probe():
    """Every kernel of the library on the bench's workloads, a few calls each,
    for rocprofv3 (kernel trace or one counter pass per run)."""
    import torch

    import joint_video_audio_rope_amd as J
    from synth import WORKLOADS, joint_inputs, sparse_inputs, upstream_grad

    dev = "cuda"
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
    dst = torch.empty_like(src)
    src.fill_(1.0)
    for _ in range(2):
        dst.copy_(src)
    del src, dst
    w = WORKLOADS["480p"]
    x = joint_inputs(w, dev)
    q, k, v = x["q"], x["k"], x["v"]
    n, h, d = q.shape
    frame = w["H"] * w["W"]
    n_vs = (w["n_cond_frames"] + w["T"]) * frame
    a0, t0 = n_vs, n_vs + w["n_audio"]
    spec = J.rope_spec_for(w)
    for _ in range(2):
        J.mmdit_joint_attn(q[:n_vs], k[t0:], v[t0:])
        q2, k2 = q.clone(), k.clone()
        J.mmdit_rope3d(spec, q2, k2)
        J.mmdit_joint_attn(q2, k2, v)
        J.mmdit_av_cross_attn(q2[:n_vs], k2[:n_vs], v[:n_vs], q2[a0:t0], k2[a0:t0], v[a0:t0])
        J.mmdit_joint_attn_rope(spec, q, k, v)
    g = upstream_grad(w, dev)
    o, lse = J.mmdit_joint_attn_fwd(q2, k2, v)
    J.mmdit_joint_attn_bwd(q2, k2, v, o, lse, g)
    torch.cuda.synchronize()
    del o, lse, g, q2, k2, x, q, k, v
    ws = WORKLOADS["sparse2k"]
    xs = sparse_inputs(ws, dev)
    T, H, W = ws["T"], ws["H"], ws["W"]
    args = (xs["q"], xs["k"], xs["v"], T, H, W, ws["zone"], ws["block"], ws["top_k"], ws["top_p"])
    for _ in range(2):
        J.mmdit_block_sparse_attn(*args)
    o, lse, mask, _ = J.mmdit_block_sparse_attn_fwd(*args)
    gs = torch.randn(xs["q"].shape, device=dev).to(torch.bfloat16)
    J.mmdit_block_sparse_attn_bwd(xs["q"], xs["k"], xs["v"], o, lse, gs, mask, T, H, W, ws["zone"], ws["block"])
    torch.cuda.synchronize()
    print("probe done", flush=True)


def traffic_probe():
    import torch

    import joint_video_audio_rope_amd as J
    from synth import WORKLOADS, joint_inputs

    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
    dst = torch.empty_like(src)
    src.fill_(1.0)
    torch.cuda.synchronize()
    for _ in range(2):
        dst.copy_(src)
    x = joint_inputs(WORKLOADS["480p"], "cuda")
    n = x["q"].shape[0]
    o = torch.empty((n, 24, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(J.mmdit_workspace_bytes(J.MMDIT_OP_JOINT_ATTN, n, n, 24, 128, J.MMDIT_BF16),
                     dtype=torch.uint8, device="cuda")
    for _ in range(3):
        J.mmdit_joint_attn(x["q"], x["k"], x["v"], o=o, ws=ws)
    torch.cuda.synchronize()
    print("traffic probe done: 1 GiB copy x2, joint attention x3", flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def host_workers():
    """Oracle worker processes: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


_SHARED = {}


def _oracle_task(task):
    """Worker side of the oracle timing: one oracle call on arrays the parent
    set up before forking (shared copy-on-write, nothing pickled)."""
    kind, a = task
    if kind == "attn":
        from oracle import attention as A
        qn, kn, vn, hd, r0, r1 = a
        q, k, v = _SHARED[qn], _SHARED[kn], _SHARED[vn]
        return A.attention(q[r0:r1, hd:hd + 1], k[:, hd:hd + 1], v[:, hd:hd + 1], chunk=128).shape
    from oracle import block_sparse as B
    b0, b1 = a
    S = _SHARED
    return len(B.block_sparse_attention(S["q"], S["k"], S["v"], S["idx"], S["mask"], query_blocks=range(b0, b1)))


def oracle_times():
    """The fp64 oracle (numpy, as it stands) timed on the host cores for each
    workload, split over heads and query slices into single-threaded worker
    processes (numpy's exp is single-threaded).  Inputs are the workloads'
    seeded tensors drawn on the host (same distributions and shapes as on the
    GPU; the bytes differ, which does not matter for timing).  This mode never
    touches the GPU, so the workers are forked and share the inputs."""
    import multiprocessing as mp

    import numpy as np
    import torch

    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)            # no BLAS threads exist when the workers fork
    except Exception:
        pass
    from oracle import attention as A
    from oracle import block_sparse as B
    from oracle import rope as R
    from synth import WORKLOADS, joint_inputs, n_tokens, shrink, sparse_inputs

    nw = host_workers()

    def f32(t):
        return t.to(torch.float32).numpy()

    def run(tasks):
        with mp.get_context("fork").Pool(nw) as pool:
            t0 = time.perf_counter()
            pool.map(_oracle_task, tasks, chunksize=1)
            return time.perf_counter() - t0

    def attn_tasks(qn, kn, vn, per_head):
        nq, h = _SHARED[qn].shape[0], _SHARED[qn].shape[1]
        step = -(-nq // per_head)
        return [("attn", (qn, kn, vn, hd, r0, min(nq, r0 + step))) for hd in range(h) for r0 in range(0, nq, step)]

    rows = []

    def joint_layer(name, heads=None):
        w = WORKLOADS[name] if heads is None else shrink(name, heads=heads)
        x = joint_inputs(w, "cpu")
        q, k, v = f32(x["q"]), f32(x["k"]), f32(x["v"])
        pos, rot = R.token_positions(w)
        t0 = time.perf_counter()
        rq = R.apply_rope(q, pos, rot, w["split"], w["theta"])
        rk = R.apply_rope(k, pos, rot, w["split"], w["theta"])
        t_rope = time.perf_counter() - t0
        seg = A.joint_segments(w)
        (v0, v1), (a0, a1), (s0, s1) = seg["video_stream"], seg["audio"], seg["text"]
        _SHARED.clear()
        _SHARED.update(q=q, rq=rq, rk=rk, v=v, qv=rq[v0:v1], kv=rk[v0:v1], vv=v[v0:v1], qa=rq[a0:a1],
                       ka=rk[a0:a1], va=v[a0:a1], qs=q[v0:v1], ks=k[s0:s1], vs=v[s0:s1])
        per_head = max(1, -(-4 * nw // w["heads"]))
        t_joint = run(attn_tasks("rq", "rk", "v", per_head))
        t_av = run(attn_tasks("qv", "ka", "va", per_head) + attn_tasks("qa", "kv", "vv", 1))
        t_vt = run(attn_tasks("qs", "ks", "vs", per_head)) if name == "480p" else None
        return t_rope, t_joint, t_av, t_vt

    for name, label in (("tiny", "88-token fp32 (2 x 64)"), ("block", "5850-token joint block"),
                        ("480p", "480p-latent layer (35050 tokens)")):
        t_rope, t_joint, t_av, t_vt = joint_layer(name)
        rows.append((label, "in full", t_rope, t_joint, t_av, t_vt))
        print("[oracle] %s: rope %.2f s, joint %.2f s, A<->V %.2f s%s" % (
            label, t_rope, t_joint, t_av, "" if t_vt is None else ", video->text %.2f s" % t_vt),
            file=sys.stderr, flush=True)
    h = WORKLOADS["720p"]["heads"]
    t_rope, t_joint, t_av, _ = joint_layer("720p", heads=1)
    rows.append(("720p-latent layer (76330 tokens)", "one head x %d (extrapolated)" % h,
                 t_rope * h, t_joint * h, t_av * h, None))
    print("[oracle] 720p one head: joint %.2f s, A<->V %.2f s" % (t_joint, t_av), file=sys.stderr, flush=True)

    w = shrink("sparse2k", heads=1)
    T, H, W = w["T"], w["H"], w["W"]
    x = sparse_inputs(w, "cpu")
    q, k, v = f32(x["q"]), f32(x["k"]), f32(x["v"])
    t0 = time.perf_counter()
    idx = B.block_token_index(T, H, W, w["zone"], w["block"])
    P = B.block_probs(B.block_means(q, idx), B.block_means(k, idx))
    mask, counts, _ = B.select_blocks(P, w["top_k"], w["top_p"])
    t_sel = time.perf_counter() - t0
    nb = idx.shape[0]
    _SHARED.clear()
    _SHARED.update(q=q, k=k, v=v, idx=idx, mask=mask)
    step = -(-nb // (4 * nw))
    t_sparse = run([("sparse", (b0, min(nb, b0 + step))) for b0 in range(0, nb, step)])
    t_dense = run(attn_tasks("q", "k", "v", 4 * nw))
    _SHARED.clear()
    hs = WORKLOADS["sparse2k"]["heads"]
    dens = float(counts.mean()) / nb
    rows.append(("block-sparse 24x64x112 (172032 tokens), dense", "one head x %d (extrapolated)" % hs,
                 None, t_dense * hs, None, None))
    rows.append(("block-sparse 24x64x112 (172032 tokens), sparse", "one head x %d (extrapolated)" % hs,
                 None, (t_sel + t_sparse) * hs, None, None))
    print("[oracle] sparse2k one head: selection %.2f s, sparse attention %.2f s (density %.3f), dense %.2f s" % (
        t_sel, t_sparse, dens, t_dense), file=sys.stderr, flush=True)

    print("CPU: %s; os.cpu_count() = %s; %d single-threaded worker processes (numpy %s)\n" % (
        cpu_model(), os.cpu_count(), nw, np.__version__))
    print("| workload | coverage | RoPE s | joint (or dense / sparse) attention s | A<->V s | video->text s |")
    print("|---|---|---|---|---|---|")
    fmt = lambda t: "-" if t is None else "%.1f" % t
    for label, cov, a, b, c, d in rows:
        print("| %s | %s | %s | %s | %s | %s |" % (label, cov, fmt(a), fmt(b), fmt(c), fmt(d)))
    print("\nblock-sparse, one head: selection (pooling, scores, top-k/top-p) %.1f s, sparse attention over "
          "all %d query blocks %.1f s at density %.3f, dense %.1f s" % (t_sel, nb, t_sparse, dens, t_dense))


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize, args.traffic_out)
        return
    if args.oracle_times:
        oracle_times()
        return
    if args.kernel_table:
        kernel_table(args.kernel_table)
        return
    if args.probe:
        if args.gpus != 1:
            sys.exit(2)
        probe()
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.traffic_probe:
        traffic_probe()
        return
    import torch

    import joint_video_audio_rope_amd as J
    from synth import WORKLOADS, joint_inputs, n_tokens, sparse_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WORKLOADS["480p"]
    n = n_tokens(w)
    h, d = w["heads"], w["head_dim"]
    frame = w["H"] * w["W"]
    n_vs = (w["n_cond_frames"] + w["T"]) * frame           # video stream incl. cond frame
    n_a, n_t = w["n_audio"], w["n_text"]
    a0, t0 = n_vs, n_vs + n_a

    x = joint_inputs(w, dev)
    q, k, v = x["q"], x["k"], x["v"]
    qv, kv, vv = q[:n_vs], k[:n_vs], v[:n_vs]              # contiguous views (leading rows)
    qa, ka, va = (t[a0:a0 + n_a] for t in (q, k, v))
    kt, vt = k[t0:t0 + n_t], v[t0:t0 + n_t]
    spec = J.rope_spec_for(w)
    spec.device_table(dev)

    f32 = dict(dtype=torch.float32, device=dev)
    o_joint = torch.empty((n, h, d), **f32)
    o_vt = torch.empty((n_vs, h, d), **f32)
    o_va = torch.empty((n_vs, h, d), **f32)
    o_av = torch.empty((n_a, h, d), **f32)
    ws_joint = torch.empty(J.mmdit_workspace_bytes(J.MMDIT_OP_JOINT_ATTN, n, n, h, d, J.MMDIT_BF16),
                           dtype=torch.uint8, device=dev)
    ws_vt = torch.empty(J.mmdit_workspace_bytes(J.MMDIT_OP_JOINT_ATTN, n_vs, n_t, h, d, J.MMDIT_BF16),
                        dtype=torch.uint8, device=dev)
    ws_av = torch.empty(J.mmdit_workspace_bytes(J.MMDIT_OP_AV_CROSS_ATTN, n_vs, n_a, h, d, J.MMDIT_BF16),
                        dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    ev_joint = []

    def step(record=False):
        J.mmdit_joint_attn(qv, kt, vt, o=o_vt, ws=ws_vt, stream=stream)
        J.mmdit_rope3d(spec, q, k, stream=stream)
        if record:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        J.mmdit_joint_attn(q, k, v, o=o_joint, ws=ws_joint, stream=stream)
        if record:
            e1.record(stream)
            ev_joint.append((e0, e1))
        J.mmdit_av_cross_attn(qv, kv, vv, qa, ka, va, o_video=o_va, o_audio=o_av, ws=ws_av,
                              stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for _ in range(args.steps):
        step(record=True)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    joint_ms = sum(a.elapsed_time(b) for a, b in ev_joint) / len(ev_joint)

    fl_joint = attn_flops(n, n, h, d)
    fl_step = fl_joint + attn_flops(n_vs, n_t, h, d) + 2 * attn_flops(n_vs, n_a, h, d)
    value = fl_step / (ms_step * 1e-3) / 1e12
    joint_tflops = fl_joint / (joint_ms * 1e-3) / 1e12
    print("[bench] step %.3f ms, joint call %.3f ms (%.1f TFLOP/s)" % (ms_step, joint_ms, joint_tflops),
          file=sys.stderr, flush=True)

    out = {
        "metric": "MMDiT joint-attn fwd TFLOP/s (480p-latent, 21f+218 audio) + % bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "pv_dtype": "fp16 (P in (0, 256]; V prescaled per head by a power of two, exact)",
        "data": "synthetic (seeded N(0,1) Q/K/V, bf16, resident in HBM)",
        "config": {"workload": "480p-latent layer: video 21x30x52 + 1 cond frame (t=-1), 218 audio, "
                               "512 text; 35050 tokens, 24 heads x 128; step = video->text + RoPE + "
                               "joint self-attn + audio<->video cross-attn",
                   "tokens": n, "heads": h, "head_dim": d, "step_flop": fl_step,
                   "value_is": "TFLOP/s of the whole step: 4*Nq*Nk*d*h summed over its four attention calls, "
                               "over the step time; the joint self-attention call alone (the metric's "
                               "kernel) is roofline.achieved / joint_attn.tflops"},
        "joint_attn": {"ms": round(joint_ms, 4), "tflops": round(joint_tflops, 2),
                       "pct_bf16_peak": round(100.0 * joint_tflops / PEAK_BF16_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(joint_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(joint_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "joint attention call (V prescale + V^T staging + attn_bf16_kernel<128>), "
                               "4*N^2*d*h = %.4g FLOP per call" % fl_joint},
    }

    out["fused_rope"] = fused_rope_leg(args, torch, J, spec, x, step, o_joint, o_vt, o_va, o_av, ws_vt, ws_av,
                                       n_vs, a0, t0, dev, stream)
    print("[bench] RoPE fused into the joint attention: %s" % out["fused_rope"], file=sys.stderr, flush=True)

    if not args.no_clock:
        clk = clock_under(torch, lambda: J.mmdit_joint_attn(q, k, v, o=o_joint, ws=ws_joint, stream=stream))
        out["joint_attn"]["clock"] = clk
        if clk:
            out["joint_attn"]["pct_peak_at_clock"] = round(
                100.0 * joint_tflops / (PEAK_BF16_TFLOPS * clk["gfx_mhz"] / PEAK_CLOCK_MHZ), 2)
        print("[bench] under sustained joint attention: %s" % clk, file=sys.stderr, flush=True)

    del o_vt, o_va, o_av, ws_vt, ws_av
    if not args.no_train:
        out["train"] = train_leg(args, torch, J, w, q, k, v, dev)
        print("[bench] training leg: %s" % out["train"], file=sys.stderr, flush=True)
    if not args.no_sparse:
        out["block_sparse"] = sparse_leg(args, torch, J, WORKLOADS["sparse2k"], sparse_inputs, dev)
        print("[bench] block sparse: %s" % out["block_sparse"], file=sys.stderr, flush=True)

    if not args.no_adaptive:
        out["adaptive_sparse"] = adaptive_leg(args, torch, J, WORKLOADS["adaptive2k"], dev)
        print("[bench] adaptive block shapes: %s" % out["adaptive_sparse"], file=sys.stderr, flush=True)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args, torch, q, k, v)
        print("[bench] cpu baseline: %s" % out["cpu_baseline"], file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


def fused_rope_leg(args, torch, J, spec, x, step, o_joint, o_vt, o_va, o_av, ws_vt, ws_av, n_vs, a0, t0, dev,
                   stream):
    """The same step with the RoPE fused into the joint attention
    (mmdit_joint_attn_rope: K rotated in the V staging pass, Q in registers,
    both written out for the cross-attentions): video->text, fused joint
    attention, audio<->video on the rotated tensors.  The separate-call step
    and the fused one are timed alternately, twice each, and the faster run
    of each is kept, so that both see the same clock."""
    n_a = o_av.shape[0]
    v = x["v"]
    n, h, d = v.shape
    from synth import WORKLOADS, joint_inputs
    fresh = joint_inputs(WORKLOADS["480p"], dev)     # unrotated Q, K (the step rotates its own in place)
    qu, ku = fresh["q"], fresh["k"]
    q_rot, k_rot = torch.empty_like(qu), torch.empty_like(ku)
    ws_f = torch.empty(J.mmdit_workspace_bytes(J.MMDIT_OP_JOINT_ATTN_ROPE, n, n, h, d, J.MMDIT_BF16),
                       dtype=torch.uint8, device=dev)
    qv = qu[:n_vs]
    kt, vt = ku[t0:], v[t0:]

    def fused_step():
        J.mmdit_joint_attn(qv, kt, vt, o=o_vt, ws=ws_vt, stream=stream)
        J.mmdit_joint_attn_rope(spec, qu, ku, v, o=o_joint, q_rot=q_rot, k_rot=k_rot, ws=ws_f, stream=stream)
        J.mmdit_av_cross_attn(q_rot[:n_vs], k_rot[:n_vs], v[:n_vs], q_rot[a0:a0 + n_a], k_rot[a0:a0 + n_a],
                              v[a0:a0 + n_a], o_video=o_va, o_audio=o_av, ws=ws_av, stream=stream)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    sep, fus = [], []
    for _ in range(2):
        sep.append(timed(step))
        fus.append(timed(fused_step))
    del ws_f, q_rot, k_rot, fresh
    return {"step_ms_fused": round(min(fus), 4), "step_ms_separate": round(min(sep), 4),
            "saved_ms": round(min(sep) - min(fus), 4)}


def train_leg(args, torch, J, w, q, k, v, dev):
    """Joint attention of a training step on the same 480p-latent tensors:
    forward with the log-sum-exp, then the backward for a seeded dO."""
    from synth import upstream_grad

    n, h, d = q.shape
    g = upstream_grad(w, dev)
    o = torch.empty((n, h, d), dtype=torch.float32, device=dev)
    lse = torch.empty((h, n), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty((n, h, d), dtype=torch.float32, device=dev) for _ in range(3))
    ws_f = torch.empty(J.mmdit_workspace_bytes(J.MMDIT_OP_JOINT_ATTN, n, n, h, d, J.MMDIT_BF16),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty(J.mmdit_workspace_bytes(J.MMDIT_OP_JOINT_ATTN_BWD, n, n, h, d, J.MMDIT_BF16),
                       dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def fwd():
        J.mmdit_joint_attn_fwd(q, k, v, o=o, lse=lse, ws=ws_f, stream=stream)

    def bwd():
        J.mmdit_joint_attn_bwd(q, k, v, o, lse, g, dq=dq, dk=dk, dv=dv, ws=ws_b, stream=stream)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    t_f = timed(fwd, 5)
    t_b = timed(bwd, 5)
    fl_f = attn_flops(n, n, h, d)
    fl_b = 2.5 * fl_f          # five products of 2*N^2*d per head
    return {"workload": "joint self-attention of the 480p-latent layer (35050 tokens, 24 x 128), "
                        "seeded N(0,1) dO",
            "fwd_lse_ms": round(t_f, 3), "bwd_ms": round(t_b, 3),
            "bwd_tflops": round(fl_b / t_b * 1e-9, 1),
            "fwd_bwd_tflops": round((fl_f + fl_b) / (t_f + t_b) * 1e-9, 1),
            "flop_convention": "fwd 4*N^2*d*h, bwd 10*N^2*d*h"}


def sparse_leg(args, torch, J, w, sparse_inputs, dev):
    """Dense vs block-sparse self-attention on the 24 x 64 x 112 video grid."""
    T, H, W = w["T"], w["H"], w["W"]
    h, d = w["heads"], w["head_dim"]
    n = T * H * W
    x = sparse_inputs(w, dev)
    q, k, v = x["q"], x["k"], x["v"]
    o = torch.empty((n, h, d), dtype=torch.float32, device=dev)
    ws_d = torch.empty(J.mmdit_workspace_bytes(J.MMDIT_OP_JOINT_ATTN, n, n, h, d, J.MMDIT_BF16),
                       dtype=torch.uint8, device=dev)
    sd = J.sparse_desc(w["zone"], w["block"], w["top_k"], w["top_p"])
    ws_s = torch.empty(J.mmdit_workspace_bytes(J.MMDIT_OP_BLOCK_SPARSE_ATTN, n, n, h, d, J.MMDIT_BF16, sd),
                       dtype=torch.uint8, device=dev)
    nb = n // 64
    mask = torch.empty((h, nb, (nb + 31) // 32), dtype=torch.int32, device=dev)
    cnt = torch.empty((h, nb), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def dense():
        J.mmdit_joint_attn(q, k, v, o=o, ws=ws_d, stream=stream)

    def sparse():
        J.mmdit_block_sparse_attn(q, k, v, T, H, W, w["zone"], w["block"], w["top_k"], w["top_p"],
                                  o=o, sel_mask=mask, sel_count=cnt, ws=ws_s, stream=stream)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.sparse_reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.sparse_reps

    t_dense = timed(dense)
    t_sparse = timed(sparse)
    counts = cnt.to(torch.float64)
    density = float(counts.mean().item() / nb)
    fl_dense = attn_flops(n, n, h, d)
    fl_sparse = 4.0 * 64 * 64 * d * float(counts.sum().item())
    out = {"workload": "video 24x64x112 (172032 tokens), 24 heads x 128, zones 8x8x8, blocks 4x4x4, "
                       "top-k 32 + top-p 0.9, smooth-field Q/K/V",
           "dense_ms": round(t_dense, 3), "sparse_ms": round(t_sparse, 3),
           "speedup": round(t_dense / t_sparse, 3), "density": round(density, 4),
           "dense_tflops": round(fl_dense / t_dense * 1e-9, 1),
           "sparse_attn_tflops_incl_selection": round(fl_sparse / t_sparse * 1e-9, 1)}
    if not args.no_clock:
        out["clock_sparse"] = clock_under(torch, sparse)
    if not args.no_train:
        out.update(sparse_train_leg(args, torch, J, w, q, k, v, o, ws_d, ws_s, mask, cnt, timed, stream))
    return out


def adaptive_leg(args, torch, J, w, dev):
    """Dense vs block-sparse self-attention with content-adaptive block shapes
    on the 24 x 64 x 112 grid (foreground blob in V, pulsing audio norms)."""
    from synth import adaptive_inputs

    T, H, W = w["T"], w["H"], w["W"]
    h, d = w["heads"], w["head_dim"]
    n = T * H * W
    x = adaptive_inputs(w, dev)
    q, k, v, a = x["q"], x["k"], x["v"], x["a"]
    o = torch.empty((n, h, d), dtype=torch.float32, device=dev)
    ws_d = torch.empty(J.mmdit_workspace_bytes(J.MMDIT_OP_JOINT_ATTN, n, n, h, d, J.MMDIT_BF16),
                       dtype=torch.uint8, device=dev)
    ws_a = torch.empty(J.mmdit_workspace_bytes(J.MMDIT_OP_BLOCK_SPARSE_ATTN_ADAPTIVE, n, 0, h, d, J.MMDIT_BF16),
                       dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    res = {}

    def dense():
        J.mmdit_joint_attn(q, k, v, o=o, ws=ws_d, stream=stream)

    def adaptive():
        res.update(J.mmdit_block_sparse_attn_adaptive(q, k, v, T, H, W, a_norm=a, top_k=w["top_k"],
                                                      top_p=w["top_p"], o=o, ws=ws_a, stream=stream))

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.sparse_reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.sparse_reps

    t_dense = timed(dense)
    t_ad = timed(adaptive)
    train = {}
    if not args.no_train:
        from synth import normal_tensors

        g = normal_tensors([(n, h, d)], seed=int(w["seed"]) + 7919, device=dev)[0]
        lse = torch.empty((h, n), dtype=torch.float32, device=dev)
        dq, dk, dv = (torch.empty((n, h, d), dtype=torch.float32, device=dev) for _ in range(3))
        ws_db = torch.empty(J.mmdit_workspace_bytes(J.MMDIT_OP_JOINT_ATTN_BWD, n, n, h, d, J.MMDIT_BF16),
                            dtype=torch.uint8, device=dev)
        ws_ab = torch.empty(J.mmdit_workspace_bytes(J.MMDIT_OP_BLOCK_SPARSE_ATTN_ADAPTIVE_BWD, n, 0, h, d,
                                                    J.MMDIT_BF16), dtype=torch.uint8, device=dev)
        fwd = {}

        def dense_step():
            J.mmdit_joint_attn_fwd(q, k, v, o=o, lse=lse, ws=ws_d, stream=stream)
            J.mmdit_joint_attn_bwd(q, k, v, o, lse, g, dq=dq, dk=dk, dv=dv, ws=ws_db, stream=stream)

        def adaptive_step():
            fwd.update(J.mmdit_block_sparse_attn_adaptive(q, k, v, T, H, W, a_norm=a, top_k=w["top_k"],
                                                          top_p=w["top_p"], o=o, lse=lse, ws=ws_a, stream=stream))
            J.mmdit_block_sparse_attn_adaptive_bwd(q, k, v, fwd, g, T, H, W, dq=dq, dk=dk, dv=dv, ws=ws_ab,
                                                   stream=stream)

        t_dt, t_at = timed(dense_step), timed(adaptive_step)
        train = {"train_dense_ms": round(t_dt, 3), "train_adaptive_ms": round(t_at, 3),
                 "train_speedup": round(t_dt / t_at, 3)}
        del ws_db, ws_ab, dq, dk, dv
    nt = n // 64
    words = res["sel_mask"].view(torch.uint8).cpu()
    pairs = int(torch.bitwise_and(words[..., None] >> torch.arange(8, dtype=torch.uint8), 1).sum().item())
    vols = torch.bincount(res["zone_shape"].long().cpu(), minlength=16)
    by_vol = {64: int(vols[:7].sum()), 128: int(vols[7:13].sum()), 256: int(vols[13:].sum())}
    fl_sparse = 4.0 * 64 * 64 * d * pairs
    return {"workload": "video 24x64x112 (172032 tokens), 24 heads x 128, zones 8x8x8, content-adaptive "
                        "blocks (16 shapes, 64/128/256 tokens), top-k 32 + top-p 0.9, foreground blob in V, "
                        "pulsing audio norms",
            "zones_by_volume": by_vol, "shapes_used": int((vols > 0).sum()),
            "blocks": int(res["n_blocks"].item()),
            "dense_ms": round(t_dense, 3), "adaptive_ms": round(t_ad, 3),
            "speedup": round(t_dense / t_ad, 3), "density": round(pairs / (h * nt * nt), 4),
            "sparse_attn_tflops_incl_selection": round(fl_sparse / t_ad * 1e-9, 1), **train}


def sparse_train_leg(args, torch, J, w, q, k, v, o, ws_d, ws_s, mask, cnt, timed, stream):
    """Attention of a training step at the same shape: forward with the
    log-sum-exp plus backward, dense against block-sparse."""
    from synth import normal_tensors

    T, H, W = w["T"], w["H"], w["W"]
    n, h, d = q.shape
    dev = q.device
    g = normal_tensors([(n, h, d)], seed=int(w["seed"]) + 7919, device=dev)[0]
    lse = torch.empty((h, n), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty((n, h, d), dtype=torch.float32, device=dev) for _ in range(3))
    ws_db = torch.empty(J.mmdit_workspace_bytes(J.MMDIT_OP_JOINT_ATTN_BWD, n, n, h, d, J.MMDIT_BF16),
                        dtype=torch.uint8, device=dev)
    sd = J.sparse_desc(w["zone"], w["block"], w["top_k"], w["top_p"])
    ws_sb = torch.empty(J.mmdit_workspace_bytes(J.MMDIT_OP_BLOCK_SPARSE_ATTN_BWD, n, n, h, d, J.MMDIT_BF16, sd),
                        dtype=torch.uint8, device=dev)

    def dense_step():
        J.mmdit_joint_attn_fwd(q, k, v, o=o, lse=lse, ws=ws_d, stream=stream)
        J.mmdit_joint_attn_bwd(q, k, v, o, lse, g, dq=dq, dk=dk, dv=dv, ws=ws_db, stream=stream)

    def sparse_step():
        J.mmdit_block_sparse_attn_fwd(q, k, v, T, H, W, w["zone"], w["block"], w["top_k"], w["top_p"], o=o,
                                      lse=lse, sel_mask=mask, sel_count=cnt, ws=ws_s, stream=stream)
        J.mmdit_block_sparse_attn_bwd(q, k, v, o, lse, g, mask, T, H, W, w["zone"], w["block"], dq=dq, dk=dk,
                                      dv=dv, ws=ws_sb, stream=stream)

    t_dense = timed(dense_step)
    t_sparse = timed(sparse_step)
    del ws_db, ws_sb, dq, dk, dv, g
    return {"train_dense_ms": round(t_dense, 3), "train_sparse_ms": round(t_sparse, 3),
            "train_speedup": round(t_dense / t_sparse, 3)}


def cpu_baseline(args, torch, q, k, v):
    """The fp64 oracle on host cores over a bounded sample of the joint attention."""
    import numpy as np

    from oracle import attention as A

    rows = np.linspace(0, q.shape[0] - 1, args.cpu_rows).astype(np.int64)
    qh = q[torch.from_numpy(rows).to(q.device)].to("cpu", torch.float64).numpy()
    kh = k.to("cpu", torch.float64).numpy()
    vh = v.to("cpu", torch.float64).numpy()
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    t0 = time.perf_counter()
    A.attention(qh, kh, vh, chunk=256)
    dt = time.perf_counter() - t0
    fl = attn_flops(len(rows), k.shape[0], q.shape[1], q.shape[2])
    return {"value": round(fl / dt / 1e12, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "cpu_count": os.cpu_count(),
            "sample": "joint attention of %d evenly spaced query rows x all 24 heads against all %d "
                      "keys (numpy fp64, BLAS threads for the products, exp single-threaded), "
                      "%.1f s" % (len(rows), k.shape[0], dt)}


if __name__ == "__main__":
    main()
