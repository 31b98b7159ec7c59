#!/usr/bin/env python3
"""Benchmark of the Tail-Replay state rebuild on one MI355X.

A step is one pass of the replay hot path over one batch of synthetic inputs that are
already resident in HBM: tail selection for every hit (k = ceil(r m)), then the
library call(s) that rebuild the states.  Workloads:

  group        12 groups x 3 LA layers, d_model 2048, 16 qk / 32 v heads, dk = dv = 128,
               m = 32,768, r = 0.05 -> 1,639 tail tokens per group (tr_group_replay:
               RMSNorm + projections, GDN recurrence, output projection + residual)
  batched_r05  36 (group, layer) instances x 32 v-heads (16 qk), m = 32,768, r = 0.05
  batched      the same at r = 0.10 (3,277 tokens)
  single_hit   1 layer, 16 heads, m = 32,768, r = 0.05
  varlen       64 hits, m ~ U{4096..131072}, r = 0.05, 16 heads

Prints ONE JSON line.  The roofline entry covers the dominant kernel: its algorithmic
bytes (or FLOPs) per launch divided by its average launch time, measured with HIP
events on the stream the kernel runs on.
"""
from __future__ import annotations

import argparse
import gc
import json
import re
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(HERE, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = {
    "gemm_tn_kernel": "linear_attention_state_amd/csrc/la_layer.hip",
    "rmsnorm_kernel": "linear_attention_state_amd/csrc/la_layer.hip",
    "gdn_chunk_bf16_kernel": "linear_attention_state_amd/csrc/gdn_chunk_bf16.hip",
    "gdn_scan_split_kernel": "linear_attention_state_amd/csrc/gdn_scan_split.hip",
    "gdn_decode_kernel": "linear_attention_state_amd/csrc/state_ops.hip",
}
# the split schedule's two kernels, whose traffic adds up to one tr_gdn_replay call
SPLIT_KERNELS = ("gdn_chunk_bf16_kernel<{dk},{dv}> prep", "gdn_scan_split_kernel<{dk},{dv}>")
COPY_BYTES = 1 << 30
BF16_PEAK_TFLOPS = 2500.0
METRIC = "replayed token-heads/sec (GDN state rebuild)"


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="group",
                   choices=["group", "batched_r05", "batched", "single_hit", "varlen",
                            "fidelity", "full_prefix", "decode", "overlap"])
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--schedule", default="auto", choices=["auto", "fused", "split"],
                   help="schedule of the bf16 recurrence (tr_gdn_set_schedule)")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum CPU-baseline sample time")
    p.add_argument("--flush-cache", action="store_true",
                   help="write 512 MiB between steps so no input is cache-resident (timed per launch)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy (the reference kernel for the "
                        "FETCH_SIZE / WRITE_SIZE counter scale) and exit")
    return p.parse_args()


# ---------------------------------------------------------------- HBM traffic
def kernel_digest(path):
    """sha256 of a kernel source with its // comments and blank lines removed: edits to the
    comments do not change the kernel the counts were taken on."""
    import hashlib
    import re
    with open(os.path.join(HERE, path), encoding="utf-8") as f:
        text = f.read()
    lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.split("\n")]
    code = "\n".join(ln for ln in lines if ln.strip())
    return hashlib.sha256(code.encode("utf-8")).hexdigest()


def measured_traffic(kernel_name, workload):
    """HBM bytes per launch of a kernel from rocprofv3 FETCH_SIZE and WRITE_SIZE counts
    (profiles/hbm_traffic.json), each scaled by the factor that turns the same counter's
    reading for a plain copy of known size into that size.  None when no count exists, or
    when the kernel's source has changed since the counts were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    m = re.match(r"gdn split schedule <(\d+),(\d+)>", kernel_name)
    if m:
        parts = [measured_traffic(k.format(dk=m.group(1), dv=m.group(2)), workload) for k in SPLIT_KERNELS]
        return None if None in parts else sum(parts)
    key = kernel_name.split(" (")[0] + "@" + workload
    ent = table.get("kernels", {}).get(key)
    if not ent:
        return None
    src = KERNEL_SOURCES.get(key.split("<")[0].split("@")[0])
    if src is None or ent.get("source_digest") != kernel_digest(src):
        return None
    return ent.get("hbm_bytes_per_launch")


def copy_calibration():
    import torch
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "launches": 3}), flush=True)


# ---------------------------------------------------------------- counting rules
def gdn_bytes(T, B, Hqk, Hv, dk, dv, with_o=True, with_state_in=False, elt=2):
    """Algorithmic HBM bytes of one tr_gdn_replay launch: every input read once, every
    output written once (q and k once per query/key head; a state-only launch reads no q)."""
    per_tok = Hqk * (2 if with_o else 1) * dk * elt + Hv * dv * elt + Hv * 8 + (Hv * dv * elt if with_o else 0)
    state = B * Hv * dv * dk * 4 * (2 if with_state_in else 1)
    return T * per_tok + state


def gdn_useful_flops(lengths, Hv, dk, dv, C=64, with_o=True):
    """Useful chunked-form FLOPs: per chunk of n tokens and value head, the dense products
    K K^T, W = A(..)K, U = A(..)V, W S^T, the state update, and with outputs Q K^T, Q S^T, P U'."""
    total = 0.0
    for L in lengths:
        full, rem = divmod(int(L), C)
        for n in [C] * full + ([rem] if rem else []):
            f = 2 * n * n * dk + 2 * n * n * dk + 2 * n * n * dv + 2 * n * dk * dv + 2 * dv * n * dk
            if with_o:
                f += 2 * n * n * dk + 2 * n * dk * dv + 2 * n * n * dv
            total += f
    return total * Hv


def group_gemm_flops(G, L, n, d, Hqk, Hv, dk, dv):
    proj = 2 * n * d * (2 * Hqk * dk + Hv * dv + 2 * Hv)
    oproj = 2 * n * Hv * dv * d
    return G * (L * proj + (L - 1) * oproj)


# ---------------------------------------------------------------- workloads
def build_workload(name, seed):
    import torch
    import synthetic
    from linear_attention_state_amd import tail_seqlens

    spec = dict(synthetic.WORKLOADS[name])
    rn, rd = spec["r"]
    if "G" in spec:
        G, L = spec["G"], spec["L"]
        ms = [spec["m"]] * G
        cu, _ = tail_seqlens(ms, rn, rd)
        n = int(cu[1])
        gi = synthetic.group_inputs(G, L, n, spec["d_model"], spec["Hqk"], spec["Hv"], spec["dk"], spec["dv"],
                                    seed=seed, backend="torch", device="cuda")
        return dict(kind="group", spec=spec, ms=ms, r=(rn, rd), n=n, inputs=gi)
    if name == "varlen":
        ms = synthetic.prefix_lengths(spec["n_hits"], seed=5 + seed)
    else:
        ms = [spec["m"]] * spec["B"]
    cu, _ = tail_seqlens(ms, rn, rd)
    lens = np.diff(cu.numpy()).tolist()
    inp = synthetic.gdn_inputs(lens, spec["Hqk"], spec["Hv"], spec["dk"], spec["dv"], seed=seed,
                               backend="torch", device="cuda")
    return dict(kind="gdn", spec=spec, ms=ms, r=(rn, rd), lens=lens, inputs=inp,
                cu_dev=cu.to("cuda"))


def make_step(w):
    """Returns step() that runs tail selection + the replay call(s) on the current stream."""
    import torch
    from linear_attention_state_amd import GroupReplay, gdn_replay, gdn_replay_workspace_size, tail_seqlens

    rn, rd = w["r"]
    if w["kind"] == "gdn":
        inp, spec = w["inputs"], w["spec"]
        B, Hv, dk, dv = len(w["lens"]), spec["Hv"], spec["dk"], spec["dv"]
        S = torch.empty((B, Hv, dv, dk), dtype=torch.float32, device="cuda")
        o = torch.empty((inp.q.shape[0], Hv, dv), dtype=torch.bfloat16, device="cuda")
        # the split schedule's workspace, allocated once outside the timed steps
        cu0, _ = tail_seqlens(w["ms"], rn, rd)
        nws = gdn_replay_workspace_size(cu0, spec["Hqk"], Hv, dk, dv, torch.bfloat16)
        w["workspace"] = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None

        def step():
            cu, _ = tail_seqlens(w["ms"], rn, rd)
            gdn_replay(inp.q, inp.k, inp.v, inp.g, inp.beta, cu, cu_seqlens_dev=w["cu_dev"], state_out=S, o=o,
                       workspace=w["workspace"])
        return step, (S, o)
    spec, gi = w["spec"], w["inputs"]
    runner = GroupReplay(gi.weights, w["n"], spec["d_model"], spec["Hqk"], spec["Hv"], spec["dk"], spec["dv"])
    states = torch.empty((spec["G"], spec["L"], spec["Hv"], spec["dv"], spec["dk"]), dtype=torch.float32,
                         device="cuda")

    def step():
        tail_seqlens(w["ms"], rn, rd)
        runner(gi.h_tail, states_out=states)
    return step, (states,)


def time_steps(step, steps, warmup, flush):
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") if flush else None
    if not flush:
        gc.collect()
        gc.disable()
        try:
            t_host = time.perf_counter()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                step()
            e1.record(stream)
            torch.cuda.synchronize()
            host_ms = (time.perf_counter() - t_host) * 1e3
        finally:
            gc.enable()
        return e0.elapsed_time(e1) / steps, host_ms / steps, None
    per = []
    for _ in range(steps):
        scratch.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b))
    return float(np.mean(per)), None, per


def step_stats(step, steps, warmup):
    """Per-step mean, median and min (ms) with HIP events around each step: warm (inputs
    resident in HBM, steps back to back) and with the 256 MB MALL flushed before each step by a
    512 MiB fill of a scratch buffer (the fill is outside the events)."""
    import torch
    out = {}
    mean, med, mn = time_launches(step, steps, warmup)
    out["warm"] = dict(mean_ms=mean, median_ms=med, min_ms=mn, reps=steps)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    per = []
    for _ in range(steps):
        scratch.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b))
    del scratch
    out["flushed"] = dict(mean_ms=float(np.mean(per)), median_ms=float(np.median(per)), min_ms=float(np.min(per)),
                          reps=steps)
    return out


def fused_kernel_name(dk, dv, schedule):
    """The kernel a fused-schedule tr_gdn_replay launch runs."""
    return "gdn_chunk_bf16_kernel<%d,%d>" % (dk, dv)


def time_launches(fn, steps, warmup):
    """Average duration of one launch of fn() with HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    # The GPU is kept busy while the launches are enqueued (a spin kernel first, and no
    # garbage collection meanwhile), so no event pair spans a host-side pause on an idle stream.
    gc.collect()
    gc.disable()
    try:
        _busy_gpu(torch, 0.05)
        fn()
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
    finally:
        gc.enable()
    d = [a.elapsed_time(b) for a, b in ev]
    return float(np.mean(d)), float(np.median(d)), float(np.min(d))


def time_sequence(fns, steps, warmup):
    """Average launch duration of each fn when the sequence fns[0], fns[1], ... is repeated
    `steps` times, every launch bracketed by its own HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        for fn in fns:
            fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
          for _ in range(steps)]
    gc.collect()
    gc.disable()
    try:
        _busy_gpu(torch, 0.05)
        for row in ev:
            for fn, (a, b) in zip(fns, row):
                a.record(stream)
                fn()
                b.record(stream)
        torch.cuda.synchronize()
    finally:
        gc.enable()
    out = []
    for i in range(len(fns)):
        d = [row[i][0].elapsed_time(row[i][1]) for row in ev]
        out.append((float(np.mean(d)), float(np.median(d)), float(np.min(d))))
    return out


def _busy_gpu(torch, seconds):
    """Enqueue about `seconds` of GPU spinning on the current stream."""
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(int(seconds * 2.4e9))


# ---------------------------------------------------------------- CPU baseline
def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


_ONE_CORE = r"""
import json, sys, time
import numpy as np
sys.path.insert(0, sys.argv[1])
import oracle
z = np.load(sys.argv[2])
kind, min_s = sys.argv[3], float(sys.argv[4])
done, elapsed, units = 0, 0.0, 0
while elapsed < min_s or units == 0:
    t0 = time.perf_counter()
    if kind == "gdn":
        oracle.gdn(z["q"], z["k"], z["v"], z["g"], z["beta"], z["cu"])
    else:
        L = int(z["L"])
        ws = [[{k: z["%s_%d" % (k, l)] for k in ("w_qk", "w_v", "w_a", "w_b", "w_o")} for l in range(L)]]
        oracle.group(z["h"], ws, int(z["Hqk"]), int(z["Hv"]), int(z["dk"]), int(z["dv"]))
    elapsed += time.perf_counter() - t0
    done += int(z["token_heads"])
    units += 1
print(json.dumps(dict(value=done / elapsed, seconds=elapsed, units=units, threads=oracle.num_threads())))
"""


def cpu_one_core(arrays, kind, min_seconds, unit_desc):
    """The same oracle on one core (OpenMP and BLAS limited to one thread, in a child process
    that loads one unit of the workload from a temporary file), repeated until min_seconds."""
    import subprocess
    import tempfile
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "unit.npz")
        np.savez(path, **arrays)
        env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
        res = subprocess.run([sys.executable, "-c", _ONE_CORE, HERE, path, kind, str(min_seconds)],
                             capture_output=True, text=True, env=env, timeout=600)
    if res.returncode != 0:
        return dict(error=res.stderr[-500:])
    out = json.loads(res.stdout.strip().splitlines()[-1])
    out["sample"] = "%d repetition(s) of %s" % (out.pop("units"), unit_desc)
    out["seconds"] = round(out["seconds"], 2)
    out["cores"] = out.pop("threads")
    return out


def cpu_baseline(w, min_seconds):
    """The fp64 oracle on whole (sequence, all heads) units of the same workload until at
    least min_seconds of CPU time has accumulated."""
    import oracle

    def np64(t):
        return t.detach().to("cpu").double().numpy()

    if w["kind"] == "gdn":
        inp, spec = w["inputs"], w["spec"]
        cu = np.concatenate([[0], np.cumsum(w["lens"])])
        order = list(range(len(w["lens"])))
        done_th, elapsed, units = 0, 0.0, 0
        for b in order:
            sl = slice(int(cu[b]), int(cu[b + 1]))
            args = [np64(t[sl]) for t in (inp.q, inp.k, inp.v, inp.g, inp.beta)]
            t0 = time.perf_counter()
            oracle.gdn(*args, [0, sl.stop - sl.start])
            elapsed += time.perf_counter() - t0
            done_th += (sl.stop - sl.start) * spec["Hv"]
            units += 1
            if elapsed >= min_seconds:
                break
        sample = "%d of %d sequences x %d heads (%d token-heads), fp64 token loop" % (
            units, len(order), spec["Hv"], done_th)
        n0 = int(w["lens"][0])
        unit = {k: np64(t[:n0]) for k, t in (("q", inp.q), ("k", inp.k), ("v", inp.v), ("g", inp.g),
                                              ("beta", inp.beta))}
        unit.update(cu=np.array([0, n0], dtype=np.int32), token_heads=n0 * spec["Hv"])
        one = cpu_one_core(unit, "gdn", min_seconds / 4,
                           "sequence 0 (%d tokens x %d heads), fp64 token loop" % (n0, spec["Hv"]))
        return dict(value=done_th / elapsed, unit="token-heads/s", cores=oracle.num_threads(), kind="oracle",
                    sample=sample, seconds=round(elapsed, 2), cpu_model=cpu_model(), one_core=one)
    # group: whole groups (all layers) through the chain oracle
    spec, gi = w["spec"], w["inputs"]
    done_th, elapsed, units = 0, 0.0, 0
    n_cpu = min(w["n"], 1639)       # a token prefix of each group is a whole replay of its own
    for g in range(spec["G"]):
        h = np64(gi.h_tail[g:g + 1, :n_cpu])
        ws = [[{k: np64(t) for k, t in d.items()} for d in gi.weights[g]]]
        t0 = time.perf_counter()
        oracle.group(h, ws, spec["Hqk"], spec["Hv"], spec["dk"], spec["dv"])
        elapsed += time.perf_counter() - t0
        done_th += n_cpu * spec["Hv"] * spec["L"]
        units += 1
        if elapsed >= min_seconds:
            break
    sample = "%d of %d groups x %d layers x %d heads x %d tokens, fp64" % (
        units, spec["G"], spec["L"], spec["Hv"], n_cpu)
    unit = dict(h=np64(gi.h_tail[0:1, :n_cpu]), L=spec["L"], Hqk=spec["Hqk"], Hv=spec["Hv"], dk=spec["dk"],
                dv=spec["dv"], token_heads=n_cpu * spec["Hv"] * spec["L"])
    for li in range(spec["L"]):
        for k, t in gi.weights[0][li].items():
            unit["%s_%d" % (k, li)] = np64(t)
    one = cpu_one_core(unit, "group", min_seconds / 4,
                       "group 0 (%d layers x %d heads x %d tokens), fp64" % (spec["L"], spec["Hv"], n_cpu))
    return dict(value=done_th / elapsed, unit="token-heads/s", cores=oracle.num_threads(), kind="oracle",
                sample=sample, seconds=round(elapsed, 2), cpu_model=cpu_model(), one_core=one)


# ---------------------------------------------------------------- next-row modes
def _line(args, value, ms, config, roof, extra):
    line = {"metric": METRIC, "value": value, "unit": "token-heads/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": config, "roofline": roof}
    line.update(extra)
    print(json.dumps(line), flush=True)


def run_fidelity(args):
    """One 32,768-token sequence: the full recurrence from zero, the tail replays at each r,
    and the transition products; reports |S_m - S_hat_m| / |S_m| and the exact truncation
    |S_a Phi| / |S_m| (both from the GPU path), and the times."""
    import torch
    import synthetic
    from linear_attention_state_amd import (gdn_replay, gdn_replay_workspace_size, gdn_transition,
                                            gdn_transition_workspace_size, state_compose, tail_seqlens)
    spec = synthetic.WORKLOADS["fidelity"]
    m, H, d = spec["m"], spec["Hv"], spec["dk"]
    inp = synthetic.gdn_inputs([m], spec["Hqk"], H, d, d, seed=args.seed, backend="torch", device="cuda")
    cu_m = torch.tensor([0, m], dtype=torch.int32)
    cu_m_dev = cu_m.cuda()
    S_m = torch.empty((1, H, d, d), dtype=torch.float32, device="cuda")

    def workspace(cu):
        n = gdn_replay_workspace_size(cu, spec["Hqk"], H, d, d, torch.bfloat16)
        return torch.empty(n, dtype=torch.uint8, device="cuda") if n else None
    ws_m = workspace(cu_m)

    def full():
        gdn_replay(inp.q, inp.k, inp.v, inp.g, inp.beta, cu_m, cu_seqlens_dev=cu_m_dev, state_out=S_m, want_o=False,
                   workspace=ws_m)
    t_full = time_launches(full, max(args.steps, 5), 1)[0]
    res = {}
    for rn, rd in spec["rs"]:
        k = int(tail_seqlens([m], rn, rd)[0][1])
        a = m - k
        head = [t[:a].contiguous() for t in (inp.q, inp.k, inp.v, inp.g, inp.beta)]
        tail = [t[a:].contiguous() for t in (inp.q, inp.k, inp.v, inp.g, inp.beta)]
        cu_k = torch.tensor([0, k], dtype=torch.int32)
        cu_k_dev = cu_k.cuda()
        S_hat = torch.empty_like(S_m)
        ws_k = workspace(cu_k)

        def replay():
            gdn_replay(*tail, cu_k, cu_seqlens_dev=cu_k_dev, state_out=S_hat, want_o=False, workspace=ws_k)
        t_rep = time_launches(replay, max(args.steps, 5), 1)[0]
        # the fp32-input build of the same replay (token-serial fp32 recurrence)
        tail32 = [t.float() for t in tail[:3]] + tail[3:]
        S_hat32 = torch.empty_like(S_m)

        def replay_fp32():
            gdn_replay(*tail32, cu_k, cu_seqlens_dev=cu_k_dev, state_out=S_hat32, want_o=False)
        t_rep32 = time_launches(replay_fp32, 3, 1)[0]
        psi = torch.empty_like(S_m)
        n_ws = gdn_transition_workspace_size(cu_k, spec["Hqk"], H, d, torch.bfloat16)
        ws_phi = torch.empty(n_ws, dtype=torch.uint8, device="cuda") if n_ws else None

        def transition():
            return gdn_transition(tail[1], tail[3], tail[4], cu_k, cu_seqlens_dev=cu_k_dev, phi_out=psi,
                                  separate_decay=True, workspace=ws_phi)
        t_phi = time_launches(transition, max(args.steps, 5), 1)[0]
        _, ls = transition()
        S_a, _ = gdn_replay(*head, torch.tensor([0, a], dtype=torch.int32), want_o=False)
        E = state_compose(S_a, psi)                       # S_a psi; Phi = exp(ls) psi
        torch.cuda.synchronize()
        nm = torch.linalg.matrix_norm(S_m[0].double())
        measured = (torch.linalg.matrix_norm((S_m[0] - S_hat[0]).double()) / nm).cpu().numpy()
        log10_exact = ((ls[0].double() + torch.log(torch.linalg.matrix_norm(E[0].double())) - torch.log(nm))
                       / np.log(10)).cpu().numpy()
        res["r=%d/%d" % (rn, rd)] = dict(
            tail_tokens=k, replay_us=t_rep * 1e3, replay_fp32_inputs_us=t_rep32 * 1e3, transition_us=t_phi * 1e3,
            rel_state_error_max=float(measured.max()), rel_state_error_mean=float(measured.mean()),
            log10_exact_truncation_max=float(log10_exact.max()))
    nbytes = gdn_bytes(m, 1, spec["Hqk"], H, d, d, with_o=False)
    kname = ("gdn split schedule <128,128> (state only, one 32768-token sequence)" if ws_m is not None
             else "gdn_chunk_bf16_kernel<128,128> (state only, one 32768-token sequence)")
    roof = dict(bound="hbm", achieved=nbytes / (t_full * 1e-3) / 1e9, peak=HBM_PEAK_GBS, unit="GB/s",
                traffic=None, kernel=kname,
                algorithmic_bytes=nbytes, avg_launch_us=t_full * 1e3)
    roof["frac"] = roof["achieved"] / roof["peak"]
    config = dict(workload="fidelity", tokens=m, Hqk=spec["Hqk"], Hv=H, dk=d, dv=d, chunk=64,
                  rs=["%d/%d" % r for r in spec["rs"]])
    _line(args, m * H / (t_full * 1e-3), t_full, config, roof,
          {"fidelity": res, "note": "value: the full-prefix recurrence of the sequence (state only); "
           "rel_state_error = |S_m - S_hat_m|_F / |S_m|_F per head, GPU path; the exact truncation "
           "|S_a Phi|_F / |S_m|_F from tr_gdn_transition and tr_state_compose, in log10"})


def run_decode(args):
    import torch
    import synthetic
    from linear_attention_state_amd import gdn_decode
    spec = synthetic.WORKLOADS["decode"]
    B, Hqk, Hv, dk, dv = spec["B"], spec["Hqk"], spec["Hv"], spec["dk"], spec["dv"]
    inp = synthetic.gdn_inputs([1] * B, Hqk, Hv, dk, dv, seed=args.seed, backend="torch", device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(args.seed + 1)
    state = torch.randn((B, Hv, dv, dk), generator=gen, device="cuda") * 0.1
    o = torch.empty((B, Hv, dv), dtype=torch.bfloat16, device="cuda")

    def step():
        gdn_decode(inp.q, inp.k, inp.v, inp.g, inp.beta, state, o=o)
    ms, _, _ = time_steps(step, args.steps, args.warmup, False)
    t_mean, t_med, t_min = time_launches(step, max(args.steps, 10), 2)
    nbytes = B * Hv * dv * dk * 4 * 2 + B * (Hqk * dk * 2 * 2 + Hv * dv * 2 * 2 + Hv * 8)
    roof = dict(bound="hbm", achieved=nbytes / (t_mean * 1e-3) / 1e9, peak=HBM_PEAK_GBS, unit="GB/s",
                traffic=measured_traffic("gdn_decode_kernel<128,true>", "decode"),
                kernel="gdn_decode_kernel<128,true>", algorithmic_bytes=nbytes, avg_launch_us=t_mean * 1e3,
                median_launch_us=t_med * 1e3, min_launch_us=t_min * 1e3)
    roof["frac"] = roof["achieved"] / roof["peak"]
    config = dict(workload="decode", sequences=B, Hqk=Hqk, Hv=Hv, dk=dk, dv=dv)
    _line(args, B * Hv / (ms * 1e-3), ms, config, roof,
          {"note": "value: one token per (sequence, value head) per step, state read and written in place"})


def run_full_prefix(args):
    """The group workload at r = 1, and the 5% tail replay of the same groups for the ratio."""
    import torch
    from linear_attention_state_amd import GroupReplay, tail_seqlens
    w = build_workload("full_prefix", args.seed)
    step, _ = make_step(w)
    ms, host_ms, _ = time_steps(step, args.steps, args.warmup, False)
    spec, gi = w["spec"], w["inputs"]
    k = int(tail_seqlens([spec["m"]], 5, 100)[0][1])
    h_tail = gi.h_tail[:, spec["m"] - k:].contiguous()
    runner = GroupReplay(gi.weights, k, spec["d_model"], spec["Hqk"], spec["Hv"], spec["dk"], spec["dv"])
    states = torch.empty((spec["G"], spec["L"], spec["Hv"], spec["dv"], spec["dk"]), dtype=torch.float32,
                         device="cuda")
    ms_tail, _, _ = time_steps(lambda: runner(h_tail, states_out=states), args.steps, args.warmup, False)
    roof = group_roofline(w, args)
    G, L, n = spec["G"], spec["L"], w["n"]
    config = dict(workload="full_prefix", groups=G, layers_per_group=L, tokens_per_group=n, d_model=spec["d_model"],
                  Hqk=spec["Hqk"], Hv=spec["Hv"], dk=spec["dk"], dv=spec["dv"], r="1", chunk=64)
    _line(args, G * L * n * spec["Hv"] / (ms * 1e-3), ms, config, roof,
          {"replay_5pct_ms_per_step": ms_tail, "full_over_replay": ms / ms_tail,
           "note": "LA share of a full prefill of the 32768-token prefix versus its 5% tail replay"})


def run_overlap(args):
    """Host-to-device copy of the matched prefix's full-attention KV (pinned host memory, second
    stream) beside the group replay: serial, overlapped, and the max(T_kv, T_replay) model."""
    import torch
    import synthetic
    spec = synthetic.WORKLOADS["overlap"]
    w = build_workload("group", args.seed)
    step, _ = make_step(w)
    kv_bytes = spec["kv_layers"] * 2 * spec["m"] * spec["kv_heads"] * spec["kv_head_dim"] * 2
    host = torch.empty(kv_bytes, dtype=torch.uint8, pin_memory=True)
    host.fill_(1)
    dev = torch.empty(kv_bytes, dtype=torch.uint8, device="cuda")
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()                        # default priority

    def copy(stream):
        with torch.cuda.stream(stream):
            dev.copy_(host, non_blocking=True)

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(main)
            fn()
            e1.record(main)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1))
        return float(np.mean(out))

    def overlapped():
        side.wait_stream(main)
        copy(side)
        step()
        main.wait_stream(side)

    reps = max(3, min(args.steps, 10))
    t_kv = timed(lambda: copy(main), reps)
    t_rep = timed(step, reps)
    t_serial = timed(lambda: (copy(main), step()), reps)
    t_ovl = timed(overlapped, reps)
    G, L, n, Hv = spec["G"], spec["L"], w["n"], spec["Hv"]
    config = dict(workload="overlap", groups=G, layers_per_group=L, tokens_per_group=n, Hv=Hv,
                  kv_bytes=kv_bytes, kv_layers=spec["kv_layers"], kv_heads=spec["kv_heads"],
                  kv_head_dim=spec["kv_head_dim"], prefix_tokens=spec["m"])
    roof = dict(bound="pcie", achieved=kv_bytes / (t_kv * 1e-3) / 1e9, peak=None, unit="GB/s", frac=None,
                traffic=None, kernel="host-to-device copy of the prefix KV")
    _line(args, G * L * n * Hv / (t_ovl * 1e-3), t_ovl, config, roof,
          {"overlap": dict(t_kv_ms=t_kv, t_replay_ms=t_rep, t_serial_ms=t_serial, t_overlap_ms=t_ovl,
                           model_max_ms=max(t_kv, t_rep), saved_vs_serial=1 - t_ovl / t_serial),
           "note": "value: replayed token-heads/s with the KV copy running beside the replay"})


# ---------------------------------------------------------------- main
def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only (the replay would shard over heads and hits with no "
              "exchange step); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    import linear_attention_state_amd as tr
    tr.lib()   # fails loudly if the HIP library is not built
    tr.set_gdn_schedule(args.schedule)
    special = {"fidelity": run_fidelity, "decode": run_decode, "full_prefix": run_full_prefix,
               "overlap": run_overlap}
    if args.workload in special:
        special[args.workload](args)
        return

    w = build_workload(args.workload, args.seed)
    step, outs = make_step(w)
    ms, host_ms, per = time_steps(step, args.steps, args.warmup, args.flush_cache)
    spec = w["spec"]

    if w["kind"] == "gdn":
        B, T = len(w["lens"]), int(sum(w["lens"]))
        token_heads = T * spec["Hv"]
        flops = gdn_useful_flops(w["lens"], spec["Hv"], spec["dk"], spec["dv"])
        nbytes = gdn_bytes(T, B, spec["Hqk"], spec["Hv"], spec["dk"], spec["dv"])
        inp = w["inputs"]
        S, o = outs
        from linear_attention_state_amd import gdn_replay
        cu_host = torch.from_numpy(np.concatenate([[0], np.cumsum(w["lens"])]).astype(np.int32))

        def kern():
            gdn_replay(inp.q, inp.k, inp.v, inp.g, inp.beta, cu_host, cu_seqlens_dev=w["cu_dev"], state_out=S, o=o,
                       workspace=w["workspace"])
        k_mean, k_med, k_min = time_launches(kern, max(args.steps, 10), 2)
        if w["workspace"] is None:
            kname = fused_kernel_name(spec["dk"], spec["dv"], args.schedule)
        else:
            # split schedule: one tr_gdn_replay call is the prep kernel then the state scan
            kname = "gdn split schedule <%d,%d> (gdn_chunk_bf16_kernel prep + gdn_scan_split_kernel)" % (
                spec["dk"], spec["dv"])
        roof = dict(bound="hbm", achieved=nbytes / (k_mean * 1e-3) / 1e9, peak=HBM_PEAK_GBS, unit="GB/s",
                    traffic=measured_traffic(kname, args.workload), kernel=kname,
                    algorithmic_bytes=nbytes, avg_launch_us=k_mean * 1e3, median_launch_us=k_med * 1e3,
                    min_launch_us=k_min * 1e3)
        roof["frac"] = roof["achieved"] / roof["peak"]
        config = dict(workload=args.workload, hits=B, tokens_per_hit=(w["lens"][0] if len(set(w["lens"])) == 1
                                                                   else "varlen"),
                      total_tokens=T, Hqk=spec["Hqk"], Hv=spec["Hv"], dk=spec["dk"], dv=spec["dv"],
                      r="%d/%d" % w["r"], chunk=64)
        mfma = dict(useful_tflops=flops / (ms * 1e-3) / 1e12,
                    frac_of_bf16_peak=flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS)
    else:
        G, L, n = spec["G"], spec["L"], w["n"]
        token_heads = G * L * n * spec["Hv"]
        gemm = group_gemm_flops(G, L, n, spec["d_model"], spec["Hqk"], spec["Hv"], spec["dk"], spec["dv"])
        # the last layer of a group is state-only: no Q K^T, Q S^T or P U'
        gdn_f = G * ((L - 1) * gdn_useful_flops([n], spec["Hv"], spec["dk"], spec["dv"])
                     + gdn_useful_flops([n], spec["Hv"], spec["dk"], spec["dv"], with_o=False))
        flops = gemm + gdn_f
        roof = group_roofline(w, args)
        config = dict(workload=args.workload, groups=G, layers_per_group=L, tokens_per_group=n,
                      d_model=spec["d_model"], Hqk=spec["Hqk"], Hv=spec["Hv"], dk=spec["dk"], dv=spec["dv"],
                      r="%d/%d" % w["r"], chunk=64)
        mfma = dict(useful_tflops=flops / (ms * 1e-3) / 1e12,
                    frac_of_bf16_peak=flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS)

    line = {
        "metric": METRIC,
        "value": token_heads / (ms * 1e-3),
        "unit": "token-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": config,
        "roofline": roof,
        "mfma": mfma,
        "cache": "flushed before each step" if args.flush_cache else "warm (inputs resident in HBM)",
    }
    if host_ms is not None:
        line["host_ms_per_step"] = host_ms
    line["timing"] = step_stats(step, args.steps, 2)
    line["timing"]["note"] = ("per-step HIP events: warm = inputs resident, steps back to back; flushed = "
                              "a 512 MiB scratch fill before each step evicts the 256 MB MALL")
    if args.workload == "group":
        line["target_shape"] = target_shape(args)
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, args.cpu_seconds)
        cb["gpu_speedup"] = line["value"] / cb["value"]
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)


def target_shape(args):
    """The recurrence alone at the batched 5% shape (36 instances x 32 value heads sharing 16
    query/key heads, 1,639 tail tokens of a 32,768-token prefix): one tr_gdn_replay launch,
    timed warm and with the MALL flushed, against the HBM roofline of its compulsory bytes."""
    import torch
    from linear_attention_state_amd import gdn_replay
    w = build_workload("batched_r05", args.seed)
    spec, inp = w["spec"], w["inputs"]
    B, T = len(w["lens"]), int(sum(w["lens"]))
    S = torch.empty((B, spec["Hv"], spec["dv"], spec["dk"]), dtype=torch.float32, device="cuda")
    o = torch.empty((T, spec["Hv"], spec["dv"]), dtype=torch.bfloat16, device="cuda")
    cu_host = torch.from_numpy(np.concatenate([[0], np.cumsum(w["lens"])]).astype(np.int32))

    def launch():
        gdn_replay(inp.q, inp.k, inp.v, inp.g, inp.beta, cu_host, cu_seqlens_dev=w["cu_dev"], state_out=S, o=o)
    st = step_stats(launch, max(args.steps, 10), 2)
    nbytes = gdn_bytes(T, B, spec["Hqk"], spec["Hv"], spec["dk"], spec["dv"])
    kname = fused_kernel_name(spec["dk"], spec["dv"], args.schedule)
    t = st["warm"]["mean_ms"] * 1e-3
    out = dict(workload="batched_r05", hits=B, tokens_per_hit=w["lens"][0], Hqk=spec["Hqk"], Hv=spec["Hv"],
               dk=spec["dk"], dv=spec["dv"], token_heads=T * spec["Hv"], kernel=kname,
               value=T * spec["Hv"] / t, unit="token-heads/s", avg_launch_us=st["warm"]["mean_ms"] * 1e3,
               timing=st, roofline=dict(bound="hbm", achieved=nbytes / t / 1e9, peak=HBM_PEAK_GBS, unit="GB/s",
                                        frac=nbytes / t / 1e9 / HBM_PEAK_GBS, algorithmic_bytes=nbytes,
                                        traffic=measured_traffic(kname, "batched_r05")))
    tf = st["flushed"]["mean_ms"] * 1e-3
    out["roofline"]["frac_flushed"] = nbytes / tf / 1e9 / HBM_PEAK_GBS
    del w, inp, S, o
    torch.cuda.empty_cache()
    return out


def group_roofline(w, args):
    """Time every kernel of the group step through its own entry point, in the step's launch
    configuration, and return the roofline entry of the one with the largest per-step time."""
    import torch
    from linear_attention_state_amd import gdn_replay, la_output_residual, la_project, rmsnorm

    spec, gi = w["spec"], w["inputs"]
    G, L, n, d = spec["G"], spec["L"], w["n"], spec["d_model"]
    Hqk, Hv, dk, dv = spec["Hqk"], spec["Hv"], spec["dk"], spec["dv"]
    reps = max(args.steps, 10)
    ws0 = [gi.weights[g][0] for g in range(G)]
    x = gi.h_tail
    y = torch.empty_like(x)
    out = la_project(y, ws0, Hqk, Hv, dk, dv)
    q, k, v, g, beta = out
    cu = torch.arange(G + 1, dtype=torch.int32) * n
    cu_dev = cu.to("cuda")
    S = torch.empty((G, Hv, dv, dk), dtype=torch.float32, device="cuda")
    o = torch.empty((G * n, Hv, dv), dtype=torch.bfloat16, device="cuda")
    xo = torch.empty_like(x)
    o2 = o.view(G * n, Hv * dv)
    # The kernels run in the step's order (the MFMA-heavy GEMMs between memory-bound kernels,
    # as in the step: back to back they run hotter and clock lower), each launch timed alone.
    t_norm, t_proj, t_gdn_o, t_out, t_gdn_s = time_sequence([
        lambda: rmsnorm(x, [None] * G, y=y),
        lambda: la_project(y, ws0, Hqk, Hv, dk, dv, out=out),
        lambda: gdn_replay(q, k, v, g, beta, cu, cu_seqlens_dev=cu_dev, state_out=S, o=o),
        lambda: la_output_residual(x, o2, ws0, Hv, dv, x_out=xo),
        lambda: gdn_replay(q, k, v, g, beta, cu, cu_seqlens_dev=cu_dev, state_out=S, want_o=False),
    ], reps, 2)

    proj_flops = 2.0 * G * n * d * (2 * Hqk * dk + Hv * dv + 2 * Hv)
    out_flops = 2.0 * G * n * Hv * dv * d
    gdn_o_bytes = gdn_bytes(G * n, G, Hqk, Hv, dk, dv, with_o=True)
    gdn_s_bytes = gdn_bytes(G * n, G, Hqk, Hv, dk, dv, with_o=False)
    norm_bytes = 2.0 * G * n * d * 2
    kernels = {
        "gemm_tn_kernel<layer_in> (RMSNorm'd hidden x [W_qk|W_v|W_a|W_b]^T, fused L2 norm / gates)":
            dict(avg_us=t_proj[0] * 1e3, per_step=L, bound="mfma", work=proj_flops),
        fused_kernel_name(dk, dv, args.schedule) + " (with outputs)":
            dict(avg_us=t_gdn_o[0] * 1e3, per_step=L - 1, bound="hbm", work=gdn_o_bytes),
        fused_kernel_name(dk, dv, args.schedule) + " (state only)":
            dict(avg_us=t_gdn_s[0] * 1e3, per_step=1, bound="hbm", work=gdn_s_bytes),
        "gemm_tn_kernel<residual> (o W_o^T + x)":
            dict(avg_us=t_out[0] * 1e3, per_step=L - 1, bound="mfma", work=out_flops),
        "rmsnorm_kernel":
            dict(avg_us=t_norm[0] * 1e3, per_step=L, bound="hbm", work=norm_bytes),
    }
    for kd in kernels.values():
        kd["us_per_step"] = kd["avg_us"] * kd["per_step"]
        if kd["bound"] == "mfma":
            kd["achieved_tflops"] = kd["work"] / (kd["avg_us"] * 1e-6) / 1e12
        else:
            kd["achieved_gbs"] = kd["work"] / (kd["avg_us"] * 1e-6) / 1e9
    name, top = max(kernels.items(), key=lambda kv: kv[1]["us_per_step"])
    if top["bound"] == "mfma":
        roof = dict(bound="mfma", achieved=top["achieved_tflops"], peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    algorithmic_flops=top["work"])
    else:
        roof = dict(bound="hbm", achieved=top["achieved_gbs"], peak=HBM_PEAK_GBS, unit="GB/s",
                    algorithmic_bytes=top["work"])
    roof.update(frac=roof["achieved"] / roof["peak"], traffic=measured_traffic(name, args.workload),
                kernel=name, avg_launch_us=top["avg_us"],
                kernels={k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()
                             if kk != "work"} for k, v in kernels.items()})
    return roof


if __name__ == "__main__":
    main()
