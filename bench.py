#!/usr/bin/env python3
"""Batched target-verify rounds on one MI355X.

A step is one verify round (embed, every layer's projections, attention and
FFN, lm_head, decision) over the workload's synthetic batch, replayed from a
HIP graph with commit=0 so every step has the same shape.  The headline line
is the Qwen2.5-14B-shaped 48-layer stack at context 4096 with nt = 3 (one
anchor + 2 drafts); nt = 9 on the same stack and the batch-12 block verify
(8 layers, vocab 248320, context 512, nt = 16 against nt = 1) are reported in
extra fields.  Throughput is rounds/s and committed tokens/s; bandwidth is
(weights once + KV read) per round / round time against the 8 TB/s peak.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verify rounds/s & accepted tok/s at nt=3/9/16; achieved HBM GB/s vs peak"
PEAK_HBM = 8.0e12  # B/s, MI355X published HBM3E bandwidth


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-extra", action="store_true", help="only the nt=3 headline line")
    p.add_argument("--no-graph", action="store_true", help="eager launches instead of a graph")
    p.add_argument("--profile-rounds", type=int, default=3)
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="only run a device copy of BYTES (counter calibration) and exit")
    return p.parse_args()


class Workload:
    """One model + KV cache + draft ids on the GPU."""

    def __init__(self, cfg, nt_max, keep_host_layers=0):
        import target_verification_amd as tva
        from synth.make import make_weights, make_kv, kv_capacity
        self.cfg, self.spec = cfg, cfg.model
        t0 = time.time()
        w = make_weights(self.spec, cfg.seed, "cuda")
        torch.cuda.synchronize()
        log(f"{cfg.name}: weights generated in {time.time() - t0:.1f}s")
        self.host = None
        if keep_host_layers:
            self.host = {k: ([t.cpu().numpy() for t in v[:keep_host_layers]]
                             if isinstance(v, list) else v.cpu().numpy())
                         for k, v in w.items()}
        self.cap = kv_capacity(cfg, nt_max)
        t0 = time.time()
        self.model = tva.Model(self.spec, w, max_pos=self.cap)
        torch.cuda.synchronize()
        log(f"{cfg.name}: model created (repacked) in {time.time() - t0:.1f}s")
        del w
        torch.cuda.empty_cache()
        K, V, self.lens = make_kv(cfg, self.cap, "cuda")
        if keep_host_layers:
            self.host_kv = (K[:keep_host_layers].cpu().numpy(), V[:keep_host_layers].cpu().numpy())
        self.kv = tva.KVCache.from_logical(K, V, self.lens)
        del K, V
        torch.cuda.empty_cache()

    def drafts(self, nt):
        """Synthetic drafts that follow the model's own argmax chain with the
        workload's per-depth acceptance (GPU dry runs build the chain)."""
        import target_verification_amd as tva
        from synth.make import make_anchors, chain_drafts
        anchors = make_anchors(self.cfg)

        def argmax_fn(prefix, need=None):
            ids = torch.from_numpy(np.ascontiguousarray(prefix, dtype=np.int32)).cuda()
            out = tva.verify_round(self.model, self.kv, ids, commit=0, want_logits=False)
            return out["argmax"][:, -1].cpu().numpy()
        return chain_drafts(self.cfg, anchors, nt, argmax_fn)

    def weight_bytes(self):
        from synth.configs import weight_bytes
        return weight_bytes(self.spec)

    def kv_bytes(self, nt):
        from synth.configs import kv_read_bytes
        return kv_read_bytes(self.cfg, nt)


def time_round(wl, ids_np, steps, warmup, graph=True):
    import target_verification_amd as tva
    S, nt = ids_np.shape
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).cuda()
    ws = wl.model.workspace(S, nt, tva.SV_GREEDY)
    outs = dict(accepted_len=torch.empty(S, dtype=torch.int32, device="cuda"),
                emitted=torch.empty(S, dtype=torch.int32, device="cuda"),
                argmax=torch.empty((S, nt), dtype=torch.int32, device="cuda"), logits=None)

    def step():
        tva.verify_round(wl.model, wl.kv, ids, commit=0, workspace=ws, outs=outs)

    for _ in range(max(1, warmup)):
        step()
    torch.cuda.synchronize()
    if graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        with torch.cuda.graph(g):
            step()
        run = g.replay
        for _ in range(max(1, warmup)):
            run()
    else:
        run = step
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    acc = outs["accepted_len"].cpu().numpy()
    return ms, acc, ids, ws, outs


def profile_round(wl, ids, ws, outs, rounds):
    """Per-kernel-class event timing on the round's own stream (eager)."""
    import target_verification_amd as tva
    tva.sv_profile_begin(rounds * (12 * wl.spec.n_layer + 16))
    for _ in range(rounds):
        tva.verify_round(wl.model, wl.kv, ids, commit=0, workspace=ws, outs=outs)
    torch.cuda.synchronize()
    return tva.sv_profile_end()


def class_bytes(wl, nt):
    """Algorithmic bytes of one launch of each kernel class (weights once; KV
    of one layer for attention)."""
    from synth.configs import tensor_bytes
    m = wl.spec
    fp, q, kv = m.fmt_proj, m.n_head * m.head_dim, m.n_kv_head * m.head_dim
    return {
        "gemm_qkv": tensor_bytes(fp, q + 2 * kv, m.hidden),
        "gemm_o": tensor_bytes(fp, m.hidden, q),
        "gemm_gu": tensor_bytes(fp, 2 * m.ffn, m.hidden),
        "gemm_down": tensor_bytes(fp, m.hidden, m.ffn),
        "gemm_lm": tensor_bytes(m.fmt_lm, m.vocab, m.hidden),
        "attn": wl.kv_bytes(nt) // max(1, m.n_layer),
    }


def traffic_for(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current GEMM source (else None)."""
    from target_verification_amd.profiling import gemm_source_hash
    path = os.path.join(ROOT, "profiles", "gemm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != gemm_source_hash():
        return None
    k = d.get("kernels", {}).get(kernel_key)
    return None if k is None else k.get("hbm_bytes_per_launch")


def copy_calibration(nbytes):
    """A plain streaming kernel of known size (reads nbytes, writes nbytes:
    b = 2 * a elementwise), for scaling HBM byte counters.  A same-type
    copy_ would go to the DMA engines, which the counters do not see."""
    n = nbytes // 4
    a = torch.full((n,), 1.0, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(a, 2.0, out=b)
    torch.cuda.synchronize()
    log(f"copy calibration: 3 launches of b = 2a over {nbytes} bytes")


def cpu_baseline(wl, ids_np, n_layers_sample=2):
    """The fp64 oracle on a bounded sample of the same round: the first
    n_layers_sample layers and the lm_head for the same rows, extrapolated
    linearly to all layers."""
    from oracle.model import OracleModel, rmsnorm
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    spec = wl.spec
    from dataclasses import replace
    sub = replace(spec, n_layer=n_layers_sample)
    om = OracleModel(sub, wl.host)
    kc, vc = (a.copy() for a in wl.host_kv)
    S, nt = ids_np.shape
    t0 = time.time()
    fin = np.zeros((S * nt, spec.hidden))
    for s in range(S):
        for r in range(nt):
            x = om.hidden_row(int(ids_np[s, r]), int(wl.lens[s]) + r, s, kc, vc)
            fin[s * nt + r] = rmsnorm(x, wl.host["out_norm"], spec.rms_eps)
    t_layers = time.time() - t0
    t0 = time.time()
    om.logits_rows(fin)
    t_lm = time.time() - t0
    est = t_layers * spec.n_layer / n_layers_sample + t_lm
    return {"value": 1.0 / est, "unit": "rounds/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"{wl.cfg.name} nt={nt}: {n_layers_sample} of {spec.n_layer} layers "
                       f"({t_layers:.1f}s, decode included) + lm_head ({t_lm:.1f}s), "
                       f"extrapolated linearly in layers to {est:.1f}s per round")}


def loop_line(wl, nt, rounds, p_accept, graph=True):
    """Device-resident multi-round greedy generation (sv_advance after every
    committed round; the emitted token is the next anchor on the device).
    The stub drafter proposes the target's own one-token stream with
    probability p_accept per position, else a noise id.  The one-token
    stream itself comes from a device-resident nt = 1 loop.  Times `rounds`
    rounds replayed back to back from one captured graph and checks that
    the committed tokens equal the one-token stream."""
    import target_verification_amd as tva
    from synth.make import make_anchors
    S, V, cap = wl.cfg.n_seq, wl.spec.vocab, wl.cap
    len0 = wl.kv.len.clone()
    l0 = len0.cpu().numpy().astype(np.int64)
    n_ref = rounds * nt + 2
    assert int(l0.max()) + n_ref + nt < cap, "KV capacity too small for the loop"
    anchors = np.asarray(make_anchors(wl.cfg), dtype=np.int32)
    mk = lambda: dict(accepted_len=torch.empty(S, dtype=torch.int32, device="cuda"),
                      emitted=torch.empty(S, dtype=torch.int32, device="cuda"),
                      argmax=None, logits=None)
    # the one-token stream, on the device
    ids1 = torch.from_numpy(anchors[:, None].copy()).cuda()
    outs1, ws1 = mk(), wl.model.workspace(S, 1, tva.SV_GREEDY)
    ref = torch.full((S, cap), -1, dtype=torch.int32, device="cuda")
    for _ in range(n_ref):
        tva.verify_round(wl.model, wl.kv, ids1, commit=1, workspace=ws1, outs=outs1)
        tva.sv_advance(ids1, outs1["accepted_len"], outs1["emitted"], wl.kv.len, tokens=ref)
    torch.cuda.synchronize()
    # the speculative loop
    rng = np.random.default_rng(wl.cfg.seed)
    draw_np = rng.random((S, cap)).astype(np.float32)
    noise_np = rng.integers(0, V, (S, cap)).astype(np.int32)
    ref_np = ref.cpu().numpy()
    ids0 = np.zeros((S, nt), dtype=np.int32)
    ids0[:, 0] = anchors
    for s in range(S):
        for j in range(nt - 1):
            P = l0[s] + 1 + j
            ids0[s, 1 + j] = ref_np[s, P] if draw_np[s, P] < p_accept else noise_np[s, P]
    ids0_t = torch.from_numpy(ids0).cuda()
    draw, noise = torch.from_numpy(draw_np).cuda(), torch.from_numpy(noise_np).cuda()
    ids = ids0_t.clone()
    outs, ws = mk(), wl.model.workspace(S, nt, tva.SV_GREEDY)
    tokens = torch.full((S, cap), -1, dtype=torch.int32, device="cuda")
    committed = torch.zeros(S, dtype=torch.int32, device="cuda")

    def reset():
        wl.kv.len.copy_(len0)
        ids.copy_(ids0_t)
        committed.zero_()

    def step():
        tva.verify_round(wl.model, wl.kv, ids, commit=1, workspace=ws, outs=outs)
        tva.sv_advance(ids, outs["accepted_len"], outs["emitted"], wl.kv.len, tokens=tokens,
                       committed=committed, ref=ref, draw=draw, noise=noise,
                       p_accept=p_accept, p_decay=1.0)

    reset()
    if graph:
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g, stream=st):
            step()
        torch.cuda.current_stream().wait_stream(st)
        run = g.replay
    else:
        run = step
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ms = []
    for _ in range(2):                      # the first pass warms up
        reset()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(rounds):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    c = committed.cpu().numpy()
    tk = tokens.cpu().numpy()
    same = all(np.array_equal(tk[s, l0[s] + 1: l0[s] + 1 + c[s]], ref_np[s, l0[s] + 1: l0[s] + 1 + c[s]])
               for s in range(S))
    wl.kv.len.copy_(len0)
    torch.cuda.synchronize()
    t = ms[-1]
    return {"rounds": rounds, "nt": nt, "p_accept": p_accept, "graph": graph,
            "ms_per_round": round(t / rounds, 4),
            "committed_per_round": round(float(c.sum()) / rounds / S, 3),
            "committed_tok_s": round(float(c.sum()) / (t * 1e-3), 1),
            "identical_to_one_token_stream": bool(same)}


def stochastic_line(steps, warmup, graph=True):
    """The batch-12 stochastic workload: 6-bit 248320 x 5120 lm_head over
    N(0,1) hidden states, nt = 8, T = 0.8; draft logits = target logits +
    N(0, 0.5^2) (the target logits come from a GPU round: input construction
    only), drafts sampled from them.  Times strict rejection sampling and
    exact-match sampled verify, and reports each mode's accepted lengths."""
    import target_verification_amd as tva
    from synth.configs import CONFIGS
    from synth.configs import weight_bytes
    from synth.make import (draft_logits_from_target, make_anchors, make_hidden, make_weights,
                            sample_drafts_from_q)
    from synth.rng import round_uniforms, sample_uniforms
    cfg = CONFIGS["lm248k_reject"]
    S, nt, V, T = cfg.n_seq, cfg.nt[0], cfg.model.vocab, cfg.temperature
    w = make_weights(cfg.model, cfg.seed, "cuda")
    model = tva.Model(cfg.model, w, max_pos=128)
    del w
    torch.cuda.empty_cache()
    hidden = make_hidden(cfg, nt, "cuda")
    ids0 = np.zeros((S, nt), dtype=np.int32)
    ids0[:, 0] = make_anchors(cfg)
    tgt = tva.verify_round(model, None, torch.from_numpy(ids0).cuda(), hidden=hidden,
                           commit=0)["logits"].cpu().numpy()
    dl = draft_logits_from_target(cfg, tgt)
    ids = torch.from_numpy(sample_drafts_from_q(cfg, make_anchors(cfg), dl)).cuda()
    dl_t = torch.from_numpy(dl).cuda()
    lens0 = np.zeros(S, np.int64)
    res = {}
    for name, mode, u in (("reject", tva.SV_REJECT, round_uniforms(cfg.seed, lens0, nt)),
                          ("sample", tva.SV_SAMPLE, sample_uniforms(cfg.seed, lens0, nt))):
        u_t = torch.from_numpy(u).cuda()
        ws = model.workspace(S, nt, mode)
        outs = dict(accepted_len=torch.empty(S, dtype=torch.int32, device="cuda"),
                    emitted=torch.empty(S, dtype=torch.int32, device="cuda"),
                    argmax=torch.empty((S, nt), dtype=torch.int32, device="cuda"),
                    logits=torch.empty((S, nt, V), dtype=torch.float32, device="cuda"))
        kw = dict(mode=mode, temperature=T, hidden=hidden, uniforms=u_t, commit=0,
                  workspace=ws, outs=outs)
        if mode == tva.SV_REJECT:
            kw["draft_logits"] = dl_t

        def step():
            tva.verify_round(model, None, ids, **kw)

        for _ in range(max(1, warmup)):
            step()
        torch.cuda.synchronize()
        run = step
        if graph:
            g = torch.cuda.CUDAGraph()
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.graph(g, stream=st):
                step()
            torch.cuda.current_stream().wait_stream(st)
            run = g.replay
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        acc = outs["accepted_len"].cpu().numpy()
        # bytes: the lm_head once, the logits written, the draft logits read
        nbytes = weight_bytes(cfg.model) + S * nt * V * 4 + (
            S * (nt - 1) * V * 4 if mode == tva.SV_REJECT else 0)
        res[name] = {"ms_per_round": round(ms, 4), "rounds_per_s": round(1e3 / ms, 2),
                     "committed_tok_s": round(1e3 / ms * float(np.sum(acc + 1)), 1),
                     "hbm_frac": round(nbytes / ms / 1e6 / (PEAK_HBM / 1e9), 4),
                     "accepted_len_hist": np.bincount(acc, minlength=nt).tolist(),
                     "emitted": outs["emitted"].cpu().numpy().tolist()}
        log(f"lm248k {name}: {res[name]}")
    del model
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(every box here has one GPU; see the design notes on sharding)", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    import target_verification_amd as tva
    tva.lib()
    from synth.configs import CONFIGS
    graph = not args.no_graph
    result = {}

    # ---- headline: 14B-shaped stack, nt = 3 (and 9) ----
    q14b_48l = CONFIGS["q14b_48l"]
    wl = Workload(q14b_48l, nt_max=9, keep_host_layers=0 if args.no_cpu else 2)
    wb = wl.weight_bytes()
    lines = {}
    for nt in ((3,) if args.no_extra else (3, 9)):
        t0 = time.time()
        ids = wl.drafts(nt)
        log(f"q14b_48l nt={nt}: drafts built in {time.time() - t0:.1f}s; timing {args.steps} steps")
        ms, acc, ids_t, ws, outs = time_round(wl, ids, args.steps, args.warmup, graph)
        metric_bytes = wb + wl.kv_bytes(nt)
        lines[nt] = dict(ms=ms, acc=acc, ids=ids, bytes=metric_bytes,
                         prof=profile_round(wl, ids_t, ws, outs, args.profile_rounds))
        log(f"q14b_48l nt={nt}: {ms:.4f} ms/round, {metric_bytes / ms / 1e6:.0f} GB/s, "
            f"a+1 = {(acc + 1).tolist()}")
    head = lines[3]
    prof = head["prof"]
    cb = class_bytes(wl, 3)
    gemm_classes = [c for c in prof if c in cb]
    dom = max(gemm_classes, key=lambda c: prof[c][1])
    n_l, tot, mn, mx = prof[dom]
    avg_ms = tot / n_l
    achieved = cb[dom] / (avg_ms * 1e-3) / 1e9
    # kernel template arguments: <format (2 = 4-bit/256, 3 = 6-bit/256),
    # 16-column tiles per wave, 16-row M tiles per wave (0: one tile of at
    # most 8 rows, high and low activation parts in one operand), epilogue
    # (1 = RoPE and cache write, 2 = residual add, 3 = SwiGLU, 4 = lm_head)>;
    # the 3 rows of this line run the packed (0) kernels
    kern = {"gemm_gu": "k_qgemm<2, 4, 0, 3>", "gemm_qkv": "k_qgemm<2, 2, 0, 1>",
            "gemm_down": "k_qgemm<2, 2, 0, 2>", "gemm_o": "k_qgemm<2, 2, 0, 2>",
            "gemm_lm": "k_qgemm<3, 2, 0, 4>", "attn": "k_attn_chunk"}[dom]
    traffic = traffic_for(kern) if dom == "gemm_gu" else None
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "frac": round(achieved / (PEAK_HBM / 1e9), 4),
                "traffic": traffic, "kernel": kern, "class": dom,
                "bytes_per_launch": cb[dom], "avg_launch_us": round(avg_ms * 1e3, 2),
                "launches_per_round": n_l // args.profile_rounds}
    per_class = {c: {"launches_per_round": v[0] // args.profile_rounds,
                     "ms_per_round": round(v[1] / args.profile_rounds, 4),
                     "avg_us": round(v[1] / v[0] * 1e3, 2)} for c, v in prof.items()}
    loop = None
    if not args.no_extra:
        loop = loop_line(wl, 3, 36, 0.74, graph)
        log(f"q14b_48l device loop nt=3: {loop}")
    if not args.no_cpu:
        log("cpu baseline (oracle sample) ...")
        cpu = cpu_baseline(wl, head["ids"])
    else:
        cpu = None
    del wl
    torch.cuda.empty_cache()

    extra = {}
    if loop is not None:
        extra["q14b_48l_loop_nt3"] = loop
    if 9 in lines:
        l9 = lines[9]
        extra["q14b_48l_nt9"] = {"ms_per_round": round(l9["ms"], 4), "rounds_per_s": round(1e3 / l9["ms"], 2),
                           "committed_tok_s": round(1e3 / l9["ms"] * float(np.mean(l9["acc"] + 1)), 1),
                           "hbm_gbps": round(l9["bytes"] / l9["ms"] / 1e6, 1),
                           "hbm_frac": round(l9["bytes"] / l9["ms"] / 1e6 / (PEAK_HBM / 1e9), 4)}
    if not args.no_extra:
        q14b_8l_block16 = CONFIGS["q14b_8l_block16"]
        wl5 = Workload(q14b_8l_block16, nt_max=16)
        res5 = {}
        for nt in (16, 1):
            ids = wl5.drafts(nt) if nt > 1 else wl5.drafts(1)
            ms, acc, *_ = time_round(wl5, ids, args.steps, args.warmup, graph)
            mb = wl5.weight_bytes() + wl5.kv_bytes(nt)
            res5[nt] = dict(ms=ms, acc=acc, bytes=mb)
            log(f"q14b_8l_block16 nt={nt}: {ms:.4f} ms/round, mean a+1 = {float(np.mean(acc + 1)):.2f}")
        extra["q14b_8l_block16_nt16_vs_nt1"] = {
            "nt16_ms": round(res5[16]["ms"], 4), "nt1_ms": round(res5[1]["ms"], 4),
            "ratio_nt16_over_nt1": round(res5[16]["ms"] / res5[1]["ms"], 3),
            "nt16_committed_tok_s": round(1e3 / res5[16]["ms"] * float(np.sum(res5[16]["acc"] + 1)), 1),
            "nt1_hbm_frac": round(res5[1]["bytes"] / res5[1]["ms"] / 1e6 / (PEAK_HBM / 1e9), 4),
            "batch": q14b_8l_block16.n_seq}
        del wl5
        torch.cuda.empty_cache()
        extra["lm248k_stochastic_nt8"] = stochastic_line(args.steps, args.warmup, graph)

    ms = head["ms"]
    rps = 1e3 / ms
    out = {
        "metric": METRIC, "value": round(rps, 3), "unit": "rounds/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "q14b_48l: Qwen2.5-14B-shaped stack (48 layers, hidden 5120, 40q/8kv "
                               "x 128, FFN 13824, vocab 152064), 4-bit super-block projections, "
                               "6-bit lm_head, fp16 KV ctx 4096, 1 sequence, nt=3 greedy",
                   "nt": 3, "seq_len": q14b_48l.ctx, "n_seq": 1, "graph": graph},
        "committed_tok_s": round(rps * float(np.mean(head["acc"] + 1)), 2),
        "hbm_gbps": round(head["bytes"] / ms / 1e6, 1),
        "hbm_frac": round(head["bytes"] / ms / 1e6 / (PEAK_HBM / 1e9), 4),
        "round_bytes": head["bytes"],
        "roofline": roofline,
        "kernel_classes": per_class,
        "cpu_baseline": cpu,
    }
    out.update(extra)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
