"""Per-workgroup timeline of a verify round: a measurement tool.

The library built with -DSV_TIMELINE (same kernels and results) records the
GPU's 100 MHz real-time counter per workgroup: every GEMM and attention
workgroup at its start and its end; the small-row GEMMs also at the end of
their main loop (latest wave), when wave 0 has its staged rows and norm
factors, after the barrier that joins the K splits, when thread 0 has
issued the epilogue's stores and when those are acknowledged.  It runs
graph-replayed rounds of a workload; the last round's records are
summarized per kernel class: the span of each launch (first start to last
end), the gap before it (previous launch's last end to its first start),
and for the GEMMs the median and maximum main-loop time, the median
epilogue (workgroup end minus its latest wave's loop end) and the median
epilogue parts: staging (staged rows ready minus loop end; negative when
wave 0 was done before the last wave), barrier (barrier passed minus the
later of loop end and staging), arithmetic (barrier to stores issued),
stores (issued to acknowledged) and end (acknowledged to workgroup end).

Usage:
  python -m target_verification_amd.timeline build           (host: builds the measurement library)
  python -u -m target_verification_amd.timeline run --nt 3    (GPU: q14b_48l round, nt rows)
"""

import argparse
import ctypes
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libspecverify_timeline.so")
LAYERS, KINDS, WG, FIELDS = 64, 7, 1024, 7   # the table of csrc/sv_timeline.h
NAMES = ("qkv", "chunk", "merge", "o", "gu", "down", "lm")
ORDER = (0, 1, 2, 3, 4, 5)        # kernel classes in a layer's launch order
GEMM = (0, 3, 4, 5)


def build_lib():
    from target_verification_amd.build import build, BUILD
    return build(defines=("SV_TIMELINE",), out=LIB, build_dir=os.path.join(BUILD, "timeline"))


def read_tables(lib):
    t = np.zeros((LAYERS, KINDS, WG, FIELDS), dtype=np.int64)
    for fn in ("sv_timeline_read_gemm", "sv_timeline_read_attn"):
        part = np.zeros_like(t)
        f = getattr(lib, fn)
        f.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
        if f(part.ctypes.data, part.nbytes) != 0:
            raise RuntimeError(f"{fn} failed")
        t = np.where(part != 0, part, t)
    return t


EPI_PARTS = ("staging", "barrier", "arithmetic", "stores", "end")


def summarize(t, n_layer):
    """{class: dict(span, gap, loop_p50, loop_max, epi_p50 and the epilogue
    parts)} in microseconds, means over layers 1..n_layer-1 (layer 0
    follows the embedding)."""
    keys = ("span", "gap", "loop_p50", "loop_max", "epi_p50") + EPI_PARTS
    acc = {k: {f: [] for f in keys} for k in ORDER}
    for l in range(1, n_layer):
        x = t[l - 1, 5]
        prev_end = x[x[:, 0] != 0][:, 2].max()
        for k in ORDER:
            x = t[l, k]
            x = x[x[:, 0] != 0]
            s0, e1 = x[:, 0].min(), x[:, 2].max()
            acc[k]["span"].append((e1 - s0) / 100)
            acc[k]["gap"].append((s0 - prev_end) / 100)
            if k in GEMM:
                med = lambda v: float(np.median(v)) / 100
                acc[k]["loop_p50"].append(med(x[:, 1] - x[:, 0]))
                acc[k]["loop_max"].append((x[:, 1] - x[:, 0]).max() / 100)
                acc[k]["epi_p50"].append(med(x[:, 2] - x[:, 1]))
                acc[k]["staging"].append(med(x[:, 3] - x[:, 1]))
                acc[k]["barrier"].append(med(x[:, 5] - np.maximum(x[:, 1], x[:, 3])))
                acc[k]["arithmetic"].append(med(x[:, 4] - x[:, 5]))
                acc[k]["stores"].append(med(x[:, 6] - x[:, 4]))
                acc[k]["end"].append(med(x[:, 2] - x[:, 6]))
            prev_end = e1
    return {NAMES[k]: {f: float(np.mean(v)) if v else None for f, v in d.items()}
            for k, d in acc.items()}


def run(nt, steps, warmup):
    import torch
    import target_verification_amd as tva
    tva.LIB_PATH = LIB
    lib = tva.lib()
    from synth.configs import CONFIGS
    from synth.make import make_weights, make_kv, kv_capacity
    cfg = CONFIGS["q14b_48l"]
    spec = cfg.model
    cap = kv_capacity(cfg, nt)
    w = make_weights(spec, cfg.seed, "cuda")
    model = tva.Model(spec, w, max_pos=cap)
    del w
    K, V, lens = make_kv(cfg, cap, "cuda")
    kv = tva.KVCache.from_logical(K, V, lens)
    del K, V
    rng = np.random.default_rng(cfg.seed)
    ids = torch.from_numpy(rng.integers(0, spec.vocab, size=(cfg.n_seq, nt)).astype(np.int32)).cuda()
    S = cfg.n_seq
    ws = model.workspace(S, nt, tva.SV_GREEDY)
    outs = dict(accepted_len=torch.empty(S, dtype=torch.int32, device="cuda"),
                emitted=torch.empty(S, dtype=torch.int32, device="cuda"),
                argmax=torch.empty((S, nt), dtype=torch.int32, device="cuda"), logits=None)

    max_len = int(lens.max())   # dry runs: the lengths stay as they are

    def step():
        tva.verify_round(model, kv, ids, commit=0, workspace=ws, outs=outs, max_len=max_len)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=st):
        step()
    torch.cuda.current_stream().wait_stream(st)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    t = read_tables(lib)
    s = summarize(t, spec.n_layer)
    print(f"{cfg.name}, nt = {nt}: {ms:.4f} ms per round (timeline build, {steps} graph replays)")
    print("| kernel | span us | gap before us | loop p50 us | loop max us | epilogue p50 us | "
          + " | ".join(EPI_PARTS) + " |")
    print("|---|---|---|---|---|---|" + "---|" * len(EPI_PARTS))
    tot = 0.0
    for name, d in s.items():
        tot += d["span"] + d["gap"]
        f = lambda v: "-" if v is None else f"{v:.2f}"
        print(f"| {name} | {f(d['span'])} | {f(d['gap'])} | {f(d['loop_p50'])} | "
              f"{f(d['loop_max'])} | {f(d['epi_p50'])} | "
              + " | ".join(f(d[p]) for p in EPI_PARTS) + " |")
    print(f"per layer (spans + gaps, layers 1..{spec.n_layer - 1}): {tot:.2f} us")


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    sub.add_parser("build")
    r = sub.add_parser("run")
    r.add_argument("--nt", type=int, default=3)
    r.add_argument("--steps", type=int, default=20)
    r.add_argument("--warmup", type=int, default=5)
    a = p.parse_args(argv)
    if a.cmd == "build":
        print(build_lib())
    else:
        if ROOT not in sys.path:
            sys.path.insert(0, ROOT)
        run(a.nt, a.steps, a.warmup)


if __name__ == "__main__":
    main()
