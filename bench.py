#!/usr/bin/env python3
"""Throughput of the packed-weight product path on one MI355X.

A step is one pass of the hot path over one batch of synthetic input:
  * the q8 decode layer frame at one position (hidden 4096: QKV 4096->6144,
    residual add + RMSNorm, up 4096->14336 with relu^2, down 14336->4096,
    residual add + RMSNorm, head 4096->32000), and
  * the same frame as one prefill pass over 64 positions.
Eight weight copies (8 x 342 MB, more than ten times the 256 MB Infinity
Cache) rotate between steps so the weights stream from HBM.  `value` is the decode frame's
weight-stream rate (weight bytes per frame / frame time, GB/s); the prefill
rate (positions/s) is reported beside it.  After the timed steps (not part of
ms_per_step) the other workloads are measured: the HBM read ceiling
(pg_stream_read over 2 GiB), the 1024x1024 GEMV + add +
RMSNorm, the 4096x4096 f16 GEMV over 64 rotated copies, the 420-position
prompt as 6 x 64 + 36, the decode frame as one persistent launch, the
routed-MoE pass, the q8_2f GEMVs and prefill products and the q4tp GEMVs on
the frame's shapes, the per-position argmax, and causal GQA prefill
attention at context 64 and 4096.

Prints ONE JSON line on stdout; progress goes to stderr.
    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-components", action="store_true", help="only the timed steps")
    ap.add_argument("--moe-only", action="store_true",
                    help="run only the routed-MoE pass component (for profiling its kernels)")
    ap.add_argument("--formats-only", action="store_true",
                    help="run only the q8_2f, q4tp/argmax and attention components (for profiling their kernels)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of known size (counter calibration)")
    return ap.parse_args()


# ----------------------------------------------------------------- helpers

class Timer:
    """Pairs of HIP events on torch's current stream (the stream libpg launches on)."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, s):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append((s, e))

    def total_ms(self):
        return sum(s.elapsed_time(e) for s, e in self.pairs)


def file_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def recorded_traffic(profile, key, sources):
    """HBM bytes per launch recorded in a committed counter summary under profiles/
    (the line "<key>: `<bytes>`"), or None if the summary is missing, has no such line,
    or was taken on kernel sources other than the current ones (every
    "`<sha256[:16]>` (`<file>`)" pair it lists must match)."""
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    hashes = dict((f, h) for h, f in re.findall(r"`([0-9a-f]{16})` \(`([^`]+)`\)", text))
    if not hashes or set(hashes) != set(sources):
        return None
    for f in sources:
        if hashes[f] != file_hash(os.path.join(ROOT, "prefill_gemm_amd", "csrc", f)):
            return None
    t = re.search(re.escape(key) + r":\s*`?([0-9.eE+]+)", text)
    return float(t.group(1)) if t else None


def hbm_entry(kernel, nbytes, us, traffic=None, ceiling=None, **extra):
    """A roofline entry for an HBM-bound kernel: algorithmic bytes per launch over the
    average launch duration, against the published 8 TB/s (and the measured read ceiling)."""
    gbs = nbytes / (us * 1e-6) / 1e9
    e = {"kernel": kernel, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "avg_launch_us": round(us, 3),
         "algorithmic_bytes_per_launch": int(nbytes)}
    if ceiling:
        e["frac_of_read_ceiling"] = round(gbs / ceiling, 4)
    e.update(extra)
    return e


def to_dev(torch, a):
    import numpy as np
    return torch.as_tensor(np.ascontiguousarray(a)).to("cuda")


def q8_dev(torch, pg, m):
    return pg.Q8Weight(to_dev(torch, m.q), to_dev(torch, m.scale), to_dev(torch, m.bias))


# Weight copies a streaming measurement rotates through: two drawn on the host,
# the rest device clones at other addresses.  8 x 342 MB (2.7 GB) is more than ten
# times the 256 MB Infinity Cache, so a copy's lines are gone before it comes round
# again (with two copies, 5% of a frame's time was the cache's).
COPIES = 8


def q8_clone(torch, pg, W):
    return pg.Q8Weight(W.q.clone(), W.scale.clone(), W.bias.clone())


def make_frames(torch, pg, synth, n_list, copies=COPIES, host_copies=2):
    frames = {n: [] for n in n_list}
    nbytes = None
    host = []
    for c in range(host_copies):
        f = synth.frame_weights(seed=c)
        host.append(({k: q8_dev(torch, pg, f[k]) for k in ("qkv", "up", "down", "head")},
                     to_dev(torch, f["w1"]), to_dev(torch, f["w2"]), f["eps"]))
        del f
    for c in range(copies):
        W0, w1, w2, eps = host[c % host_copies]
        W = W0 if c < host_copies else {k: q8_clone(torch, pg, v) for k, v in W0.items()}
        for n in n_list:
            frames[n].append(pg.Frame(W["qkv"], W["up"], W["down"], W["head"], w1, w2, eps, n=n))
        nbytes = sum(w.nbytes() for w in W.values())
    return frames, nbytes


# ----------------------------------------------------------------- timed step

def capture_steps(torch, frames, inp):
    """Per weight copy, the decode frame (four GEMV launches) and the prefill pass
    (one prefill_frame_q8 call, five launches) each captured into a HIP graph, so
    that the timed replays measure the GPU's work and not the host's launch rate."""
    s = torch.cuda.Stream()
    graphs = []
    for dec, pre in zip(frames[1], frames[64]):
        inp["h1"].copy_(inp["h1_0"])
        inp["h64"].copy_(inp["h64_0"])
        for st in dec.stages(inp["x1"], inp["h1"]):   # eager once: kernel attributes, buffers
            st()
        pre.run(inp["x64"], inp["h64"])
        torch.cuda.synchronize()
        gd, gp = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(gd, stream=s):
            for st in dec.stages(inp["x1"], inp["h1"]):
                st()
        with torch.cuda.graph(gp, stream=s):
            pre.run(inp["x64"], inp["h64"])
        graphs.append((gd, gp))
    torch.cuda.synchronize()
    return graphs


def time_replays(torch, graphs, which, K):
    """K graph replays back to back (the weight copies in rotation) between one pair
    of HIP events on torch's current stream: the steady-state time per replay."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(K):
        graphs[i % len(graphs)][which].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / K


# ----------------------------------------------------------------- components

def one_graph(torch, fns):
    """All callables, in order, captured into ONE HIP graph (each run once eagerly first),
    so that a replay pays one launch for many kernels."""
    for f in fns:
        f()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return g


def time_graphs(torch, gs, K, tries=3):
    """Best of ``tries`` runs of K replays back to back (graphs in rotation): ms per replay."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = float("inf")
    for _ in range(tries):
        e0.record()
        for i in range(K):
            gs[i % len(gs)].replay()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / K)
    return best


def component_f16(torch, pg, synth, reps=100, copies=64, host_copies=16):
    """The f16 GEMV over 64 rotated copies (so that the weights come from HBM), the 64
    launches captured in one graph and replayed back to back (steady state); also one
    eager call at a time between events."""
    rng = synth.streams(7, host_copies + 1)
    Ws = [to_dev(torch, synth.f16(rng[i], 4096, 4096)) for i in range(host_copies)]
    Ws += [Ws[i % host_copies].clone() for i in range(host_copies, copies)]
    x = to_dev(torch, synth.normal(rng[host_copies], 4096))
    y = torch.empty(4096, device="cuda")
    best = time_graphs(torch, [one_graph(torch, [lambda i=i: pg.gemv_f16(Ws[i], x, y) for i in range(copies)])],
                       max(1, reps // copies)) / copies
    t = Timer(torch)
    for r in range(reps):
        s = t.start()
        pg.gemv_f16(Ws[r % copies], x, y)
        t.stop(s)
    torch.cuda.synchronize()
    single = t.total_ms() / reps
    nbytes = 4096 * 4096 * 2
    return {"workload": "f16 GEMV 4096x4096, 64 launches over 64 rotated copies (2.1 GB) in one graph, replayed back to back",
            "us_per_gemv": round(best * 1e3, 3), "GB_s": round(nbytes / (best * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (best * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "us_per_isolated_call": round(single * 1e3, 3)}


def component_q82(torch, pg, synth, reps=20, copies=COPIES, host_copies=2):
    """The pages' own int8 format (q8_2f) on the decode frame's four shapes: the four
    GEMVs (and, separately, the four prefill products at 64 positions) for each of 8
    weight copies (2.2 GB) captured in one graph, replayed back to back."""
    shapes = [(6144, 4096), (14336, 4096), (4096, 14336), (32000, 4096)]
    rng = synth.streams(11, host_copies * len(shapes) + len(shapes))
    Ws = []
    for c in range(host_copies):
        row = []
        for i, (r, k) in enumerate(shapes):
            m = synth.q82(rng[c * len(shapes) + i], r, k)
            row.append(pg.Q82Weight(to_dev(torch, m.q), torch.as_tensor(m.rs).cuda(), torch.as_tensor(m.cf).cuda()))
        Ws.append(row)
    for c in range(host_copies, copies):
        Ws.append([pg.Q82Weight(W.q.clone(), W.rs.clone(), W.cf.clone()) for W in Ws[c % host_copies]])
    xs = [to_dev(torch, synth.normal(rng[host_copies * len(shapes) + i], k)) for i, (r, k) in enumerate(shapes)]
    ys = [torch.empty(r, device="cuda") for r, k in shapes]

    def chain(c):
        for W, x, y in zip(Ws[c], xs, ys):
            pg.gemv_q82(W, x, y)
    best = time_graphs(torch, [one_graph(torch, [lambda c=c: chain(c) for c in range(copies)])], reps) / copies
    nbytes = sum(W.nbytes() for W in Ws[0])

    # The same four products over a pass of 64 positions (prefill_gemm_q82).
    n = 64
    Xs = [to_dev(torch, synth.normal(rng[host_copies * len(shapes) + i], (n, k))) for i, (r, k) in enumerate(shapes)]
    Ys = [torch.empty(n, r, device="cuda") for r, k in shapes]
    wss = [torch.empty(pg.prefill_gemm_q8_workspace_bytes(r, k, n), dtype=torch.uint8, device="cuda")
           for r, k in shapes]

    def pchain(c):
        for W, X, Y, ws in zip(Ws[c], Xs, Ys, wss):
            pg.prefill_gemm_q82(W, X, Y, workspace=ws)
    pbest = time_graphs(torch, [one_graph(torch, [lambda c=c: pchain(c) for c in range(copies)])], reps) / copies
    flops = 2.0 * n * sum(r * k for r, k in shapes)
    return {"workload": "q8_2f GEMVs on the decode frame's shapes (QKV, up, down, head), back to back",
            "us_per_frame": round(best * 1e3, 2), "weight_bytes": nbytes,
            "GB_s": round(nbytes / (best * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (best * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "prefill64_us_per_frame": round(pbest * 1e3, 2),
            "prefill64_weight_GB_s": round(nbytes / (pbest * 1e-3) / 1e9, 1),
            "prefill64_TFLOP_s": round(flops / (pbest * 1e-3) / 1e12, 1)}


def component_q4tp_argmax(torch, pg, synth, reps=20, copies=COPIES, host_copies=2):
    """The pages' 4-bit format (q4tp) on the decode frame's four shapes for each of eight
    weight copies, captured in one graph and replayed back to back (the GEMVs, and separately
    the prefill products at 64 positions); and the per-position argmax over a 64 x 32000 head
    output (50 launches in one graph)."""
    import numpy as np
    shapes = [(6144, 4096), (14336, 4096), (4096, 14336), (32000, 4096)]
    rng = synth.streams(13, host_copies * len(shapes) + len(shapes) + 1)
    dev = lambda m: pg.Q4TPWeight(to_dev(torch, m.nib), to_dev(torch, m.params.view(np.int32)),
                                  to_dev(torch, m.codes))
    Ws = [[dev(synth.q4tp(rng[c * len(shapes) + i], r, k)) for i, (r, k) in enumerate(shapes)]
          for c in range(host_copies)]
    for c in range(host_copies, copies):
        Ws.append([pg.Q4TPWeight(W.nib.clone(), W.params.clone(), W.codes.clone()) for W in Ws[c % host_copies]])
    xs = [to_dev(torch, synth.normal(rng[host_copies * len(shapes) + i], k)) for i, (r, k) in enumerate(shapes)]
    ys = [torch.empty(r, device="cuda") for r, k in shapes]

    def chain(c):
        for W, x, y in zip(Ws[c], xs, ys):
            pg.gemv_q4tp(W, x, y)
    best = time_graphs(torch, [one_graph(torch, [lambda c=c: chain(c) for c in range(copies)])], reps) / copies
    nbytes = sum(W.nbytes() for W in Ws[0])

    # The same four products over a pass of 64 positions (prefill_gemm_q4tp).
    n = 64
    Xs = [to_dev(torch, synth.normal(rng[host_copies * len(shapes) + i], (n, k))) for i, (r, k) in enumerate(shapes)]
    Ys = [torch.empty(n, r, device="cuda") for r, k in shapes]
    wss = [torch.empty(pg.prefill_gemm_q8_workspace_bytes(r, k, n), dtype=torch.uint8, device="cuda")
           for r, k in shapes]

    def pchain(c):
        for W, X, Y, ws in zip(Ws[c], Xs, Ys, wss):
            pg.prefill_gemm_q4tp(W, X, Y, workspace=ws)
    pbest = time_graphs(torch, [one_graph(torch, [lambda c=c: pchain(c) for c in range(copies)])], reps) / copies
    flops = 2.0 * n * sum(r * k for r, k in shapes)

    L = to_dev(torch, synth.logits(rng[-1], 64, 32000))
    ids = torch.empty(64, dtype=torch.int32, device="cuda")
    am = time_graphs(torch, [one_graph(torch, [lambda: pg.argmax_rows(L, ids)] * 50)], 10) / 50
    return {"workload": "q4tp GEMVs on the decode frame's shapes (QKV, up, down, head), back to back",
            "us_per_frame": round(best * 1e3, 2), "weight_bytes": nbytes,
            "GB_s": round(nbytes / (best * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (best * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "prefill64_us_per_frame": round(pbest * 1e3, 2),
            "prefill64_weight_GB_s": round(nbytes / (pbest * 1e-3) / 1e9, 1),
            "prefill64_TFLOP_s": round(flops / (pbest * 1e-3) / 1e12, 1),
            "argmax_64x32000_us": round(am * 1e3, 2),
            "argmax_GB_s": round(64 * 32000 * 4 / (am * 1e-3) / 1e9, 1)}


def component_q82_bank(torch, pg, synth, reps=10, host_experts=16):
    """The q8_2f expert bank at the MoE pass's up shape: 128 experts of 1856 x 2688, the
    top 6 of the MoE component's router logits at 64 positions, relu^2; the experts are 16
    drawn on the host and device copies at other addresses."""
    import numpy as np
    c = synth.moe(0)
    E, n, k, H, I = 128, 64, c["top_k"], 2688, 1856
    rng = synth.streams(23, host_experts)
    ms = [synth.q82(rng[i], I, H) for i in range(host_experts)]
    q = torch.empty(E, I, H, dtype=torch.int8, device="cuda")
    rs = torch.empty(E, I, dtype=torch.float16, device="cuda")
    cf = torch.empty(E, H, dtype=torch.float16, device="cuda")
    for e in range(E):
        m = ms[e % host_experts]
        q[e].copy_(torch.as_tensor(m.q))
        rs[e].copy_(torch.as_tensor(m.rs))
        cf[e].copy_(torch.as_tensor(m.cf))
    X = to_dev(torch, c["X"])
    logits = X @ to_dev(torch, c["Wr"]).t()
    sel = torch.topk(logits, k, dim=1).indices.to(torch.int32).cpu().numpy()
    counts = np.bincount(sel.reshape(-1), minlength=E).astype(np.int32)
    lists = np.zeros((E, n), np.int32)
    fill = np.zeros(E, np.int64)
    for j, e in enumerate(sel.reshape(-1)):
        lists[e, fill[e]] = j
        fill[e] += 1
    cnt, lst = to_dev(torch, counts), to_dev(torch, lists)
    out = torch.empty(n * k, I, device="cuda")
    t = time_graphs(torch, [one_graph(torch, [lambda: pg.expert_bank_q82(q, rs, cf, X, cnt, lst, src_div=k, act=1,
                                                                          out=out)] * reps)], 3) / reps
    active = int((counts > 0).sum())
    nbytes = active * (I * H + 2 * I + 2 * H)
    return {"workload": "q8_2f expert bank, MoE up shape: 128 experts 2688->1856, 64 positions top-6, relu^2",
            "active_experts": active, "us": round(t * 1e3, 2), "bytes": int(nbytes), "GB_s": round(nbytes / (t * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def component_q4tp_bank(torch, pg, synth, reps=10, host_experts=16):
    """The q4tp expert bank at the MoE pass's up shape: 128 experts of 1856 x 2688, the top 6
    of the MoE component's router logits at 64 positions, relu^2; 16 experts drawn on the host,
    the rest device copies at other addresses."""
    import numpy as np
    c = synth.moe(0)
    E, n, k, H, I = 128, 64, c["top_k"], 2688, 1856
    rng = synth.streams(29, host_experts)
    ms = [synth.q4tp(rng[i], I, H) for i in range(host_experts)]
    nib = torch.empty(E, I, H // 2, dtype=torch.uint8, device="cuda")
    params = torch.empty(E, I, dtype=torch.int32, device="cuda")
    codes = torch.empty(E, I, ms[0].codes.shape[1], dtype=torch.uint8, device="cuda")
    for e in range(E):
        m = ms[e % host_experts]
        nib[e].copy_(torch.as_tensor(m.nib))
        params[e].copy_(torch.as_tensor(m.params.view(np.int32)))
        codes[e].copy_(torch.as_tensor(m.codes))
    X = to_dev(torch, c["X"])
    logits = X @ to_dev(torch, c["Wr"]).t()
    sel = torch.topk(logits, k, dim=1).indices.to(torch.int32).cpu().numpy()
    counts = np.bincount(sel.reshape(-1), minlength=E).astype(np.int32)
    lists = np.zeros((E, n), np.int32)
    fill = np.zeros(E, np.int64)
    for j, e in enumerate(sel.reshape(-1)):
        lists[e, fill[e]] = j
        fill[e] += 1
    cnt, lst = to_dev(torch, counts), to_dev(torch, lists)
    out = torch.empty(n * k, I, device="cuda")
    t = time_graphs(torch, [one_graph(torch, [lambda: pg.expert_bank_q4tp(nib, params, codes, X, cnt, lst, src_div=k,
                                                                           act=1, out=out)] * reps)], 3) / reps
    active = int((counts > 0).sum())
    nbytes = active * (I * H // 2 + I * 4 + I * ms[0].codes.shape[1])
    return {"workload": "q4tp expert bank, MoE up shape: 128 experts 2688->1856, 64 positions top-6, relu^2",
            "active_experts": active, "us": round(t * 1e3, 2), "bytes": int(nbytes),
            "GB_s": round(nbytes / (t * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def component_attn(torch, pg, synth, reps=20):
    """Causal GQA prefill attention (32 query heads, 8 KV heads of 128) over a 64-position
    pass, first in its context and last in a 4096-position one: the KV append plus the
    attention, 20 launches of each in one graph."""
    out = {"workload": "causal GQA prefill attention, 64 positions, 32 q / 8 kv heads of 128"}
    for pos0 in (0, 4032):
        c = synth.attn_pass(17, 64, pos0)
        kc, vc = to_dev(torch, c["kc"]), to_dev(torch, c["vc"])
        k, v, q = to_dev(torch, c["k"]), to_dev(torch, c["v"]), to_dev(torch, c["q"])
        o = torch.empty_like(q)
        ws = torch.empty(max(4, pg.lib().attn_prefill_workspace_bytes(64, pos0, 32, 8, 128)), dtype=torch.uint8,
                         device="cuda")

        def step():
            pg.attn_kv_append(k, v, kc, vc, pos0)
            pg.attn_prefill(q, kc, vc, pos0, c["scale"], o=o, workspace=ws)
        t = time_graphs(torch, [one_graph(torch, [step] * reps)], 3) / reps
        keys = sum(pos0 + b + 1 for b in range(64))
        flops = 4.0 * keys * 32 * 128
        out[f"ctx{pos0 + 64}_us"] = round(t * 1e3, 2)
        out[f"ctx{pos0 + 64}_TFLOP_s"] = round(flops / (t * 1e-3) / 1e12, 2)
        out[f"ctx{pos0 + 64}_kv_MB"] = round((pos0 + 64) * 8 * 128 * 8 / 1e6, 2)
    return out


def component_gemv_norm(torch, pg, synth, reps=200):
    """The small q8 GEMV followed by add + RMSNorm: 50 pairs captured in one graph and
    replayed (steady state; the 1.3 MB of weights stay in cache), and one eager pair at
    a time."""
    c = synth.gemv_add_norm(0)
    W = q8_dev(torch, pg, c["W"])
    x, w = to_dev(torch, c["x"]), to_dev(torch, c["w"])
    h = to_dev(torch, c["h"]).view(1, -1)
    y = torch.empty(1024, device="cuda")
    out = torch.empty(1, 1024, device="cuda")
    def pair():
        pg.gemv_q8(W, x, y)
        pg.add_rmsnorm(h, y.view(1, -1), w, c["eps"], out=out)
    back_to_back = time_graphs(torch, [one_graph(torch, [pair] * 50)], max(1, reps // 50)) / 50
    t = Timer(torch)
    for _ in range(reps):
        s = t.start()
        pg.gemv_q8(W, x, y)
        pg.add_rmsnorm(h, y.view(1, -1), w, c["eps"], out=out)
        t.stop(s)
    torch.cuda.synchronize()
    return {"workload": "q8 GEMV 1024x1024 + add + RMSNorm (cache resident)",
            "us_per_pair": round(back_to_back * 1e3, 3),
            "us_per_isolated_pair": round(t.total_ms() / reps * 1e3, 3)}


def component_prompt(torch, pg, frames, inp, reps=3):
    """420 positions as 6 passes of 64 and one of 36 from ONE captured graph per weight
    copy: prefill_frame_q8_meta reads each pass's {n, pos0} from a device buffer, set
    before each replay; the passes rotate over the weight copies so that every pass
    streams its weights from HBM."""
    R = 420
    X0 = torch.cat([inp["x64"]] * 7)[:R].contiguous()
    H0 = torch.cat([inp["h64_0"]] * 7)[:R].contiguous()
    H = H0.clone()
    prompts = []
    for fr in frames[64]:
        pr = pg.Prompt(fr.W["qkv"], fr.W["up"], fr.W["down"], fr.W["head"], fr.w1, fr.w2, fr.eps, X0, H)
        pr.capture()
        prompts.append(pr)
    npass = len(prompts[0].passes)
    for i in range(npass):
        prompts[i % len(prompts)].run_pass(i)
    torch.cuda.synchronize()
    t = Timer(torch)
    for r in range(reps):
        s = t.start()
        for i in range(npass):
            prompts[(7 * r + i) % len(prompts)].run_pass(i)
        t.stop(s)
    torch.cuda.synchronize()
    ms = t.total_ms() / reps
    return {"workload": "420-position prompt = 6 passes x 64 + 1 x 36, q8 frame, one captured graph "
                        "(prefill_frame_q8_meta, pass size on the device) replayed per pass",
            "ms": round(ms, 3), "positions_per_s": round(R / (ms * 1e-3), 1)}


def component_decode_single_launch(torch, pg, synth, reps=40):
    """The same decode frame as ONE persistent launch (decode_frame_q8), each
    weight copy's call captured into a graph and the graphs replayed alternately."""
    Ws, out = [], None
    for c in range(2):
        f = synth.frame_weights(seed=c)
        Ws.append(({k: q8_dev(torch, pg, f[k]) for k in ("qkv", "up", "down", "head")},
                   to_dev(torch, f["w1"]), to_dev(torch, f["w2"]), f["eps"]))
        del f
    for c in range(2, COPIES):
        W, w1, w2, eps = Ws[c % 2]
        Ws.append(({k: q8_clone(torch, pg, v) for k, v in W.items()}, w1, w2, eps))
    W0 = Ws[0][0]
    H, I = W0["qkv"].cols, W0["up"].rows
    out = {"qkv": torch.empty(W0["qkv"].rows, device="cuda"), "u": torch.empty(I, device="cuda"),
           "d": torch.empty(H, device="cuda"), "logits": torch.empty(W0["head"].rows, device="cuda")}
    rng = synth.streams(13, 2)
    x0 = to_dev(torch, synth.normal(rng[0], H))
    h = to_dev(torch, synth.normal(rng[1], H))
    ws = pg.decode_frame_q8_workspace(H, I)

    def call(c):
        W, w1, w2, eps = Ws[c]
        pg.decode_frame_q8(W["qkv"], W["up"], W["down"], W["head"], w1, w2, eps, x0, h, out, ws)

    graphs = []
    s = torch.cuda.Stream()
    for c in range(len(Ws)):
        call(c)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            call(c)
        graphs.append(g)
    for i in range(len(graphs)):
        graphs[i].replay()
    t = Timer(torch)
    torch.cuda.synchronize()
    s0 = t.start()
    for i in range(reps):
        graphs[i % len(graphs)].replay()
    t.stop(s0)
    torch.cuda.synchronize()
    us = t.total_ms() / reps * 1e3
    nbytes = sum(w.nbytes() for w in W0.values())
    pg.decode_frame_q8_status(ws)   # raises (PG_ETIMEOUT) if a barrier wait gave up: the time would mean nothing
    return {"workload": "q8 decode frame (hidden 4096) as one persistent launch, graph replays over 8 weight copies",
            "us_per_frame": round(us, 2), "GB_s": round(nbytes / (us * 1e-6) / 1e9, 1),
            "barrier_timeouts": pg.decode_frame_timeouts(ws)}


def component_read_ceiling(torch, pg, reps=5):
    """The achievable HBM read rate: pg_stream_read over 2 GiB (eight times the 256 MB
    Infinity Cache), each workgroup reading one contiguous share, at several grid sizes;
    the best grid's rate."""
    nbytes = 2 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(8192, dtype=torch.float32, device="cuda")
    rates = {}
    for wg in (256, 512, 1024, 2048, 4096, 8192):
        pg.stream_read(src, wg, sink)
        torch.cuda.synchronize()
        ms = time_graphs(torch, [one_graph(torch, [lambda wg=wg: pg.stream_read(src, wg, sink)] * reps)], 3) / reps
        rates[wg] = nbytes / (ms * 1e-3) / 1e9
    best = max(rates, key=rates.get)
    del src
    return {"workload": "pg_stream_read: 2 GiB read once with 16-byte non-temporal loads, one contiguous share "
                        "per workgroup, 512 threads", "GB_s": round(rates[best], 1), "workgroups": best,
            "frac_hbm_peak": round(rates[best] / HBM_PEAK_GBS, 4),
            "GB_s_by_workgroups": {str(k): round(v, 1) for k, v in rates.items()}}


def component_decode_eager(torch, frames, inp, reps=16):
    """The decode frame's four GEMV calls issued eagerly (no graph), one frame at a time
    between events, the weight copies in rotation: the time a caller sees without graphs."""
    t = Timer(torch)
    torch.cuda.synchronize()
    for r in range(reps):
        dec = frames[1][r % len(frames[1])]
        s = t.start()
        for st in dec.stages(inp["x1"], inp["h1"]):
            st()
        t.stop(s)
    torch.cuda.synchronize()
    return round(t.total_ms() / reps * 1e3, 2)


def component_moe(torch, pg, synth, reps=10):
    c = synth.moe(0)
    up, down = q8_dev(torch, pg, c["up"]), q8_dev(torch, pg, c["down"])
    X, Wr, w = to_dev(torch, c["X"]), to_dev(torch, c["Wr"]), to_dev(torch, c["w"])
    h0 = to_dev(torch, c["h"])
    h = h0.clone()
    n, H = c["X"].shape
    I = c["up"].q.shape[1]
    ws = torch.empty(pg.moe_grouped_workspace_bytes(n, H, I, Wr.shape[0], c["top_k"]), dtype=torch.uint8,
                     device="cuda")
    o = pg.moe_grouped(X, Wr, up, down, h, w, c["eps"], c["top_k"], workspace=ws)
    torch.cuda.synchronize()
    distinct = int((o["counts"] > 0).sum().item())
    t = Timer(torch)
    for _ in range(reps):
        h.copy_(h0)
        s = t.start()
        pg.moe_grouped(X, Wr, up, down, h, w, c["eps"], c["top_k"], workspace=ws, outputs=o)
        t.stop(s)
    torch.cuda.synchronize()
    ms = t.total_ms() / reps
    per_expert = (I * H + H * I) * 1.25
    nbytes = distinct * per_expert + Wr.numel() * 4
    return {"workload": "routed MoE pass: 64 positions, hidden 2688, 128 experts 2688->1856->2688, top-6",
            "distinct_experts": distinct, "ms": round(ms, 3), "bytes_per_pass": int(nbytes),
            "positions_per_s": round(n / (ms * 1e-3), 1),
            "GB_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


# ----------------------------------------------------------------- CPU baseline

def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(synth):
    """The oracle (plain f64 C, OpenMP over outputs) on the decode frame's four
    products at one position: repeated for about 10 s on every host thread it is
    given, then for about 8 s on one thread."""
    import numpy as np
    import oracle
    f = synth.frame_weights(seed=0)
    rng = np.random.default_rng(0)
    xs = {k: synth.normal(rng, f[k].cols) for k in ("qkv", "up", "down", "head")}
    nbytes = sum(f[k].nbytes() for k in xs)

    def run(seconds):
        frames = 0
        t0 = time.perf_counter()
        while True:
            for k, x in xs.items():
                oracle.gemm_q8(f[k].q, f[k].scale, f[k].bias, x)
            frames += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return frames, el
    cores = oracle.threads()
    frames, el = run(10.0)
    oracle.set_threads(1)
    frames1, el1 = run(8.0)
    oracle.set_threads(cores)
    return {"value": round(frames * nbytes / el / 1e9, 3), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{frames} decode frames (QKV, up, down, head q8 products at one position, "
                      f"{nbytes / 1e6:.1f} MB of weights each) in {el:.1f} s on {cores} threads; "
                      f"{frames1} frames in {el1:.1f} s on 1 thread",
            "single_thread_value": round(frames1 * nbytes / el1 / 1e9, 3),
            "cpu_model": cpu_model()}


# ----------------------------------------------------------------- main

def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU part (one process drives "
              "one device; --gpus must be 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        n = 1 << 28                      # 1 GiB f32 copy
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n * 4} bytes x3")
        return
    import prefill_gemm_amd as pg
    import synth
    if args.moe_only:
        print(json.dumps({"moe_pass": component_moe(torch, pg, synth)}), flush=True)
        return
    if args.formats_only:
        print(json.dumps({"q82_gemv_frame_shapes": component_q82(torch, pg, synth),
                          "q4tp_gemv_frame_shapes": component_q4tp_argmax(torch, pg, synth),
                          "prefill_attention": component_attn(torch, pg, synth),
                          "q82_expert_bank": component_q82_bank(torch, pg, synth),
                          "q4tp_expert_bank": component_q4tp_bank(torch, pg, synth)}), flush=True)
        return

    log("building inputs ...")
    frames, frame_bytes = make_frames(torch, pg, synth, (1, 64))
    rng = synth.streams(11, 4)
    inp = {"x1": to_dev(torch, synth.normal(rng[0], (1, 4096))),
           "h1_0": to_dev(torch, synth.normal(rng[1], (1, 4096))),
           "x64": to_dev(torch, synth.normal(rng[2], (64, 4096))),
           "h64_0": to_dev(torch, synth.normal(rng[3], (64, 4096)))}
    inp["h1"] = inp["h1_0"].clone()
    inp["h64"] = inp["h64_0"].clone()

    log("capturing graphs ...")
    graphs = capture_steps(torch, frames, inp)
    log(f"warmup {args.warmup} steps ...")
    for which in (0, 1):
        time_replays(torch, graphs, which, args.warmup)
    log(f"timing {args.steps} steps ...")
    inp["h1"].copy_(inp["h1_0"])
    inp["h64"].copy_(inp["h64_0"])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    dec_ms = time_replays(torch, graphs, 0, args.steps)
    pre_ms = time_replays(torch, graphs, 1, args.steps)
    wall = time.perf_counter() - t0
    K = args.steps
    flops_pass = 2 * 64 * sum(w.rows * w.cols for w in frames[64][0].W.values())
    # The prefill pass: the x0 staging launch (about 2 us) and four dense_kernel launches; the
    # average dense launch is taken as the pass time over four (staging included).
    dense_us = pre_ms * 1e3 / 4
    dense_traffic = recorded_traffic("dense_prefill64_counters.md", "HBM bytes per dense launch (scaled)",
                                     ["dense_q8.h", "mma_q8.hip"])
    gemv_traffic = recorded_traffic("gemv_q8_decode_frame_counters.md", "HBM bytes per launch (scaled)",
                                    ["gemv.hip"])
    dense = hbm_entry("dense_kernel (prefill pass at 64 positions: one x0 staging launch and 4 matrix-core "
                      "launches, QKV, up relu^2, down, head, the add + RMSNorm work in their epilogues)",
                      frame_bytes / 4, dense_us, dense_traffic,
                      mfma={"achieved": round(flops_pass / (pre_ms * 1e-3) / 1e12, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(flops_pass / (pre_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                            "flops_per_pass": flops_pass,
                            "note": "algorithmic flops (2 n rows cols); the bf16 hi + lo activation split runs "
                                    "twice as many on the matrix cores"},
                      arithmetic_intensity_flop_per_byte=round(flops_pass / frame_bytes, 1))
    gemv = hbm_entry("gemv_q8_kernel (decode GEMV at 1 position; a frame is 4 launches back to back, "
                     "QKV and down with the residual add, up and head with the 1/rms scaling)",
                     frame_bytes / 4, dec_ms * 1e3 / 4, gemv_traffic)

    result = {
        "metric": "weight-stream HBM GB/s (q8 GEMV decode) + prefill positions/s at B=64",
        "value": round(frame_bytes / (dec_ms * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 weights (q8 block: int8 + f32 scale + f32 bias per 32); f32 activations. Decode: f32 FMA, "
                 "f32 accumulate. Prefill: activations split into bf16 hi + lo on the bf16 matrix cores "
                 "(exact int8 weights), f32 accumulate",
        "data": "synthetic (seeded numpy: q8 U[-127,127], scale U(1e-3,1e-2), bias N(0,1e-3); x,h N(0,1))",
        "config": {"workload": "q8 layer frame, hidden 4096 (QKV 6144, up 14336 relu^2, down, head 32000, "
                               "2x add+RMSNorm): decode at 1 position + prefill pass at 64 positions",
                   "decode_batch": 1, "prefill_batch": 64, "weight_copies_rotated": COPIES,
                   "frame_weight_bytes": frame_bytes},
        "decode_frame_us": round(dec_ms * 1e3, 2),
        "decode_tokens_per_s": round(1.0 / (dec_ms * 1e-3), 1),
        "prefill_pass_us": round(pre_ms * 1e3, 2),
        "prefill_positions_per_s": round(64 / (pre_ms * 1e-3), 1),
        "prefill_frac_hbm_peak": round(frame_bytes / (pre_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "prefill_frac_mfma_bf16_peak": round(flops_pass / (pre_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline": dense,
        "rooflines": {"dense_kernel": dense, "gemv_q8_kernel": gemv},
    }
    result["decode_frame_eager_us"] = component_decode_eager(torch, frames, inp)
    if not args.no_components:
        log("components ...")
        comp = {"hbm_read_ceiling": component_read_ceiling(torch, pg),
                "gemv_add_norm_1024": component_gemv_norm(torch, pg, synth),
                "f16_gemv_4096": component_f16(torch, pg, synth),
                "prompt_420": component_prompt(torch, pg, frames, inp)}
        del frames, graphs
        torch.cuda.empty_cache()
        comp["decode_frame_single_launch"] = component_decode_single_launch(torch, pg, synth)
        torch.cuda.empty_cache()
        comp["moe_pass"] = component_moe(torch, pg, synth)
        torch.cuda.empty_cache()
        comp["q82_gemv_frame_shapes"] = component_q82(torch, pg, synth)
        comp["q4tp_gemv_frame_shapes"] = component_q4tp_argmax(torch, pg, synth)
        comp["prefill_attention"] = component_attn(torch, pg, synth)
        comp["q82_expert_bank"] = component_q82_bank(torch, pg, synth)
        comp["q4tp_expert_bank"] = component_q4tp_bank(torch, pg, synth)
        result["components"] = comp
        ceil = comp["hbm_read_ceiling"]["GB_s"]
        for e in (dense, gemv):
            e["frac_of_read_ceiling"] = round(e["achieved"] / ceil, 4)
        R = result["rooflines"]
        R["stream_read_kernel"] = hbm_entry("stream_read_kernel (the read ceiling itself)", 2 << 30,
                                            (2 << 30) / (ceil * 1e9) * 1e6, None, ceil)
        f16 = comp["f16_gemv_4096"]
        R["gemv_f16_kernel"] = hbm_entry("gemv_f16_kernel (4096 x 4096 f16)", 4096 * 4096 * 2, f16["us_per_gemv"],
                                         None, ceil)
        moe = comp["moe_pass"]
        R["expert_bank_kernel"] = hbm_entry(
            "routed-MoE pass (router, route, group, the up and down expert_bank_kernel launches, combine); "
            "bytes: each selected expert's up and down banks once plus the router", moe["bytes_per_pass"],
            moe["ms"] * 1e3, None, ceil)
        q82 = comp["q82_gemv_frame_shapes"]
        R["gemv_q82_kernel"] = hbm_entry("gemv_q82_kernel (q8_2f GEMVs on the frame's four shapes, per launch)",
                                         q82["weight_bytes"] / 4, q82["us_per_frame"] / 4, None, ceil)
        q4 = comp["q4tp_gemv_frame_shapes"]
        R["gemv_q4tp_kernel"] = hbm_entry("gemv_q4tp_kernel (q4tp GEMVs on the frame's four shapes, per launch)",
                                          q4["weight_bytes"] / 4, q4["us_per_frame"] / 4, None, ceil)
        bank = comp["q82_expert_bank"]
        R["expert_bank_kernel_q82"] = hbm_entry("expert_bank_kernel<AL, true> (q8_2f bank, MoE up shape)",
                                                bank["bytes"], bank["us"], None, ceil)
        qb = comp["q4tp_expert_bank"]
        R["expert_bank_kernel_q4tp"] = hbm_entry("expert_bank_kernel<1, kExpQ4> (q4tp bank, MoE up shape)",
                                                 qb["bytes"], qb["us"], None, ceil)
        att = comp["prefill_attention"]
        R["attn_prefill_kernel"] = {"kernel": "attn_prefill_kernel + merge (context 4096, f32 matrix cores)",
                                    "bound": "mfma", "achieved": att["ctx4096_TFLOP_s"], "peak": 157.3,
                                    "unit": "TFLOP/s", "frac": round(att["ctx4096_TFLOP_s"] / 157.3, 4),
                                    "traffic": None, "avg_launch_us": att["ctx4096_us"]}
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(synth)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
