#!/usr/bin/env python3
"""Batched target-verify rounds on one MI355X.

A step is one verify round (embed, every layer's projections, attention and
FFN, lm_head, decision) over the workload's synthetic batch, replayed from a
HIP graph with commit=0 so every step has the same shape.  The headline line
is the Qwen2.5-14B-shaped 48-layer stack at context 4096 with nt = 3 (one
anchor + 2 drafts); further fields report nt = 9 on the same stack, device-
resident multi-round loops at nt = 3 and 9, an adaptive-depth loop, the
batch-12 and single-sequence block verify (8 layers, vocab 248320, context
512, nt = 16 against nt = 1) and the stochastic lm_head workload.  Rates are
rounds/s and committed tokens/s (the closed-form expectation of committed
tokens per round printed beside each); bandwidth is (weights once + KV read)
per round / round time against the 8 TB/s peak.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]
                       [--only LINE]   (LINE: q14b_48l_nt3 | q14b_48l_nt9 |
                                        block16_nt16 | block16_nt1 | lm248k;
                                        that line alone, for profiling runs)
"""

import argparse
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
# headroom of the bench's cache past the workload's context: room for the
# device-resident loops' committed tokens (chunks past a sequence's length
# are skipped by the attention kernels)
LOOP_HEADROOM = 512
ONLY = ("q14b_48l_nt3", "q14b_48l_nt9", "block16_nt16", "block16_nt1", "lm248k")


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
    p.add_argument("--only", choices=ONLY, help="time one line only (for profiling runs)")
    p.add_argument("--profile-rounds", type=int, default=3)
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="only run a device copy of BYTES (counter calibration) and exit")
    return p.parse_args()


def closed_form_committed(p, d, decay=1.0):
    """E[a + 1] for a drafter whose depth-i draft is accepted with
    probability p * decay^i, independently, until the first miss (the
    DFlash/DSpark page, 'Is it worth it?': A = (1 - p^(K+1)) / (1 - p) for
    a constant p)."""
    e, run = 1.0, 1.0
    for i in range(d):
        run *= p * decay ** i
        e += run
    return e


class Workload:
    """One model + KV cache + draft ids on the GPU."""

    def __init__(self, cfg, nt_max, keep_host=False, headroom=0):
        import target_verification_amd as tva
        from synth.make import make_weights, make_kv, kv_capacity
        self.cfg, self.spec = cfg, cfg.model
        t0 = time.time()
        w = make_weights(self.spec, cfg.seed, "cuda")
        torch.cuda.synchronize()
        log(f"{cfg.name}: weights generated in {time.time() - t0:.1f}s")
        self.host = None
        if keep_host:
            self.host = {k: ([t.cpu().numpy() for t in v] if isinstance(v, list)
                             else v.cpu().numpy()) for k, v in w.items()}
        self.cap = kv_capacity(cfg, nt_max) + headroom
        t0 = time.time()
        self.model = tva.Model(self.spec, w, max_pos=self.cap)
        torch.cuda.synchronize()
        log(f"{cfg.name}: model created (repacked) in {time.time() - t0:.1f}s")
        del w
        torch.cuda.empty_cache()
        K, V, self.lens = make_kv(cfg, self.cap, "cuda")
        if keep_host:
            self.host_kv = (K.cpu().numpy(), V.cpu().numpy())
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

    def kv_bytes(self, nt, n_seq=None):
        from synth.configs import kv_read_bytes
        cfg = self.cfg if n_seq is None else self.cfg.with_(n_seq=n_seq)
        return kv_read_bytes(cfg, nt)


def _graph(step):
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=st):
        step()
    torch.cuda.current_stream().wait_stream(st)
    return g


def _timed(run, steps):
    """Time exactly `steps` calls of run() between two synchronizations; an
    event pair per call gives the per-step spread.  Returns (mean ms,
    per-step ms list)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        run()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return ev[0].elapsed_time(ev[-1]) / steps, per


def _spread(per):
    return {"median_ms": round(float(np.median(per)), 4), "min_ms": round(float(np.min(per)), 4),
            "max_ms": round(float(np.max(per)), 4)}


def time_round(wl, ids_np, steps, warmup, graph=True, kv=None, max_len=None):
    import target_verification_amd as tva
    kv = kv or wl.kv
    S, nt = ids_np.shape
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).cuda()
    ws = wl.model.workspace(S, nt, tva.SV_GREEDY)
    outs = dict(accepted_len=torch.empty(S, dtype=torch.int32, device="cuda"),
                emitted=torch.empty(S, dtype=torch.int32, device="cuda"),
                argmax=torch.empty((S, nt), dtype=torch.int32, device="cuda"), logits=None)
    if max_len is None:
        max_len = int(kv.len.max())   # dry runs: the lengths stay as they are

    def step():
        tva.verify_round(wl.model, kv, ids, commit=0, workspace=ws, outs=outs, max_len=max_len)

    for _ in range(max(1, warmup)):
        step()
    torch.cuda.synchronize()
    run = step
    if graph:
        run = _graph(step).replay
        for _ in range(max(1, warmup)):
            run()
    ms, per = _timed(run, steps)
    acc = outs["accepted_len"].cpu().numpy()
    return ms, per, acc, ids, ws, outs


def profile_round(wl, ids, ws, outs, rounds):
    """Per-kernel-class event timing on the round's own stream (eager)."""
    import target_verification_amd as tva
    tva.sv_profile_begin(rounds * (12 * wl.spec.n_layer + 16))
    max_len = int(wl.kv.len.max())
    for _ in range(rounds):
        tva.verify_round(wl.model, wl.kv, ids, commit=0, workspace=ws, outs=outs, max_len=max_len)
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


def committed_profile(kernel):
    """The committed rocprofv3 kernel-stats summary's average duration (us)
    of `kernel` for the 48-layer nt = 3 round, or None.  Table rows read
    'name ... calls total_ms avg_us min_us max_us share'."""
    path = os.path.join(ROOT, "profiles", "verify_q14b_48l_nt3_kernel_stats.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.lstrip().startswith(("void " + kernel + "(", kernel + "(")):
            tail = (line.rsplit("...", 1) if "..." in line else line.rsplit(")", 1))[-1].split()
            try:
                return float(tail[2])
            except (IndexError, ValueError):
                return None
    return None


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


def stream_ceiling(nbytes=1 << 31, reps=10):
    """Context for the HBM fractions: what a plain streaming kernel reaches
    on this GPU (torch's elementwise b = 2a over nbytes, counted as read +
    write bytes), against the 8 TB/s peak."""
    n = nbytes // 4
    a = torch.full((n,), 1.0, device="cuda")
    b = torch.empty_like(a)
    fn = lambda: torch.mul(a, 2.0, out=b)
    for _ in range(3):
        fn()
    ms, per = _timed(fn, reps)
    out = {"read_write_gbps": round(2 * nbytes / (float(np.min(per)) * 1e-3) / 1e9, 1),
           "bytes_each_way": nbytes,
           "note": "best of %d launches of torch's b = 2a; not this library's kernel" % reps}
    del a, b
    torch.cuda.empty_cache()
    return out


def capacity_line(steps, warmup, graph=True, capacity=32768):
    """The 14B nt = 3 round in a cache of `capacity` positions holding the
    workload's 4096 tokens, with attention over the whole capacity
    (max_len = 0) and bounded by the lengths (max_len = 4096)."""
    from synth.configs import CONFIGS
    from synth.make import kv_capacity
    cfg = CONFIGS["q14b_48l"]
    wl = Workload(cfg, nt_max=3, headroom=capacity - kv_capacity(cfg, 3))
    ids = wl.drafts(3)
    out = {"capacity": wl.cap, "len": int(wl.kv.len.max())}
    for name, ml in (("unbounded", 0), ("bounded", out["len"])):
        ms, per, acc, *_ = time_round(wl, ids, steps, warmup, graph, max_len=ml)
        out[name + "_ms"] = round(ms, 4)
        out[name + "_a_plus_1"] = int(acc[0] + 1)
        log(f"q14b_48l nt=3 at capacity {wl.cap}, max_len={ml}: {ms:.4f} ms/round")
    del wl
    torch.cuda.empty_cache()
    return out


def cpu_baseline(wl, ids_np):
    """One whole verify round of the fp64 oracle (every layer, the lm_head and
    the greedy decision) on the same rows, timed on the host cores."""
    from oracle.model import OracleModel
    from oracle.round import verify_round as oracle_round
    om = OracleModel(wl.spec, wl.host, cache_weights=False)
    kc, vc = (a.copy() for a in wl.host_kv)
    S, nt = ids_np.shape
    t0 = time.time()
    out = oracle_round(om, ids_np, wl.lens[:S], kc, vc, commit=False)
    t = time.time() - t0
    return {"value": round(1.0 / t, 5), "unit": "rounds/s", "cores": int(om.threads),
            "kind": "oracle",
            "sample": (f"one whole {wl.cfg.name} round at nt={nt} ({wl.spec.n_layer} layers, "
                       f"lm_head and decision) in {t:.1f}s; oracle a = "
                       f"{int(out['accepted_len'][0])}")}, out


def reference_stream(wl, n_ref):
    """The target's own greedy one-token stream (nt = 1 rounds on the device,
    committed), [S][cap] by absolute position; the cache length is restored."""
    import target_verification_amd as tva
    from synth.make import make_anchors
    S, cap = wl.cfg.n_seq, wl.cap
    len0 = wl.kv.len.clone()
    anchors = np.asarray(make_anchors(wl.cfg), dtype=np.int32)
    ids1 = torch.from_numpy(anchors[:, None].copy()).cuda()
    outs1 = dict(accepted_len=torch.empty(S, dtype=torch.int32, device="cuda"),
                 emitted=torch.empty(S, dtype=torch.int32, device="cuda"),
                 argmax=None, logits=None)
    ws1 = wl.model.workspace(S, 1, tva.SV_GREEDY)
    ref = torch.full((S, cap), -1, dtype=torch.int32, device="cuda")
    for _ in range(n_ref):
        tva.verify_round(wl.model, wl.kv, ids1, commit=1, workspace=ws1, outs=outs1)
        tva.sv_advance(ids1, outs1["accepted_len"], outs1["emitted"], wl.kv.len, tokens=ref)
    torch.cuda.synchronize()
    wl.kv.len.copy_(len0)
    torch.cuda.synchronize()
    return ref, anchors


def _stub_draws(wl):
    rng = np.random.default_rng(wl.cfg.seed)
    S, cap, V = wl.cfg.n_seq, wl.cap, wl.spec.vocab
    return rng.random((S, cap)).astype(np.float32), rng.integers(0, V, (S, cap)).astype(np.int32)


def loop_line(wl, ref, anchors, nt, rounds, p_accept, graph=True):
    """Device-resident multi-round greedy generation (sv_advance after every
    committed round; the emitted token is the next anchor on the device).
    The stub drafter proposes the target's own one-token stream with
    probability p_accept per position, else a noise id.  Times `rounds`
    rounds replayed back to back from one captured graph and checks that
    the committed tokens equal the one-token stream."""
    import target_verification_amd as tva
    S, cap = wl.cfg.n_seq, wl.cap
    len0 = wl.kv.len.clone()
    l0 = len0.cpu().numpy().astype(np.int64)
    assert int(l0.max()) + rounds * nt + nt < cap, "KV capacity too small for the loop"
    draw_np, noise_np = _stub_draws(wl)
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
    outs = dict(accepted_len=torch.empty(S, dtype=torch.int32, device="cuda"),
                emitted=torch.empty(S, dtype=torch.int32, device="cuda"),
                argmax=None, logits=None)
    ws = wl.model.workspace(S, nt, tva.SV_GREEDY)
    tokens = torch.full((S, cap), -1, dtype=torch.int32, device="cuda")
    committed = torch.zeros(S, dtype=torch.int32, device="cuda")

    def reset():
        wl.kv.len.copy_(len0)
        ids.copy_(ids0_t)
        committed.zero_()

    # the largest length the replayed rounds can reach (each commits <= nt)
    max_len = int(l0.max()) + rounds * nt

    def step():
        tva.verify_round(wl.model, wl.kv, ids, commit=1, workspace=ws, outs=outs, max_len=max_len)
        tva.sv_advance(ids, outs["accepted_len"], outs["emitted"], wl.kv.len, tokens=tokens,
                       committed=committed, ref=ref, draw=draw, noise=noise,
                       p_accept=p_accept, p_decay=1.0)

    reset()
    run = _graph(step).replay if graph else step
    ms = []
    for _ in range(2):                      # the first pass warms up
        reset()
        t, _ = _timed(run, rounds)
        ms.append(t * rounds)
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
            "closed_form_committed_per_round": round(closed_form_committed(p_accept, nt - 1), 4),
            "committed_tok_s": round(float(c.sum()) / (t * 1e-3), 1),
            "identical_to_one_token_stream": bool(same)}


def adaptive_line(wl, ref, anchors, rounds, p_accept, d_max=8, d_start=2, draft_ms=0.0):
    """Adaptive draft depth in closed loop: before every round the library's
    depth policy (sv_depth_*) picks d from the acceptance it has observed and
    the round times this library measured (HIP events around each replay of
    the round's graph for nt = d + 1); the stub drafter proposes the target's
    own stream with probability p_accept per position.  The host reads each
    round's accepted length (the policy is host-side), so the rounds run one
    at a time.  draft_ms: the modelled drafter cost per drafted token that
    the policy adds to each round's cost."""
    import target_verification_amd as tva
    S = wl.cfg.n_seq
    assert S == 1
    len0 = wl.kv.len.clone()
    l0 = int(len0.cpu().numpy()[0])
    draw_np, noise_np = _stub_draws(wl)
    ref_np = ref.cpu().numpy()
    graphs, bufs = {}, {}
    max_len = l0 + rounds * (d_max + 1)   # the largest length the rounds can reach
    for nt in range(1, d_max + 2):
        ids = torch.zeros((S, nt), dtype=torch.int32, device="cuda")
        outs = dict(accepted_len=torch.empty(S, dtype=torch.int32, device="cuda"),
                    emitted=torch.empty(S, dtype=torch.int32, device="cuda"),
                    argmax=None, logits=None)
        ws = wl.model.workspace(S, nt, tva.SV_GREEDY)

        def step(ids=ids, outs=outs, ws=ws):
            tva.verify_round(wl.model, wl.kv, ids, commit=0, workspace=ws, outs=outs)
        step()
        torch.cuda.synchronize()
        graphs[nt] = _graph(lambda ids=ids, outs=outs, ws=ws: tva.verify_round(
            wl.model, wl.kv, ids, commit=1, workspace=ws, outs=outs, max_len=max_len))
        bufs[nt] = (ids, outs)
    pol = tva.DepthPolicy(d_max=d_max, d_start=d_start, hysteresis=0.10, draft_ms=draft_ms)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pos, anchor = l0, int(anchors[0])
    traj, tot_ms, committed, exact = [], 0.0, 0, True
    for _ in range(rounds):
        d = pol.next()
        nt = d + 1
        ids_np = np.zeros((1, nt), dtype=np.int32)
        ids_np[0, 0] = anchor
        for j in range(d):
            P = pos + 1 + j
            ids_np[0, 1 + j] = ref_np[0, P] if draw_np[0, P] < p_accept else noise_np[0, P]
        ids, outs = bufs[nt]
        ids.copy_(torch.from_numpy(ids_np))
        e0.record()
        graphs[nt].replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        a = int(outs["accepted_len"].cpu().numpy()[0])
        e = int(outs["emitted"].cpu().numpy()[0])
        got = list(ids_np[0, 1:1 + a]) + [e]
        exact &= got == list(ref_np[0, pos + 1: pos + 2 + a])
        pol.observe(d, [a], ms)
        traj.append(d)
        tot_ms += ms
        committed += a + 1
        pos += a + 1
        anchor = e
    wl.kv.len.copy_(len0)
    torch.cuda.synchronize()
    acc, cost, rate = pol.estimates()
    pol.close()
    best = int(np.argmax(rate))
    return {"rounds": rounds, "p_accept": p_accept, "d_max": d_max, "draft_ms": draft_ms,
            "depth_trajectory": traj,
            "committed_per_round": round(committed / rounds, 3),
            "committed_tok_s": round(committed / (tot_ms * 1e-3), 1),
            "policy_best_depth": best,
            "policy_cost_ms_by_depth": [round(float(c), 4) for c in cost],
            "policy_accept_by_depth": [round(float(x), 3) for x in acc],
            "closed_form_committed_per_round_at_best": round(closed_form_committed(p_accept, best), 4),
            "identical_to_one_token_stream": bool(exact)}


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
        run = _graph(step).replay if graph else step
        run()
        ms, per = _timed(run, steps)
        acc = outs["accepted_len"].cpu().numpy()
        # bytes: the lm_head once, the logits written, the draft logits read
        nbytes = weight_bytes(cfg.model) + S * nt * V * 4 + (
            S * (nt - 1) * V * 4 if mode == tva.SV_REJECT else 0)
        res[name] = {"ms_per_round": round(ms, 4), **_spread(per),
                     "rounds_per_s": round(1e3 / ms, 2),
                     "committed_tok_s": round(1e3 / ms * float(np.sum(acc + 1)), 1),
                     "hbm_frac": round(nbytes / ms / 1e6 / (PEAK_HBM / 1e9), 4),
                     "accepted_len_hist": np.bincount(acc, minlength=nt).tolist(),
                     "emitted": outs["emitted"].cpu().numpy().tolist()}
        log(f"lm248k {name}: {res[name]}")
    del model
    torch.cuda.empty_cache()
    return res


def block16_lines(args, graph, only=None):
    """The block verify: 8 layers at 14B dims, vocab 248320, context 512, with
    drafts accepted per position with probability 0.9 * 0.98^depth; nt = 16
    against nt = 1 for the 12-sequence batch (M = 192 rows) and for one
    sequence of it."""
    from synth.configs import CONFIGS
    cfg = CONFIGS["q14b_8l_block16"]
    wl = Workload(cfg, nt_max=16)
    out = {}
    nts = (16, 1) if only is None else ((16,) if only == "block16_nt16" else (1,))
    ids = {16: wl.drafts(16)}
    ids[1] = ids[16][:, :1].copy()
    res = {}
    for nt in nts:
        ms, per, acc, *_ = time_round(wl, ids[nt], args.steps, args.warmup, graph)
        res[nt] = dict(ms=ms, per=per, acc=acc, bytes=wl.weight_bytes() + wl.kv_bytes(nt))
        log(f"block16 batch {cfg.n_seq} nt={nt}: {ms:.4f} ms/round, mean a+1 = "
            f"{float(np.mean(acc + 1)):.2f}")
    if only is not None:
        return out
    out["q14b_8l_block16_nt16_vs_nt1"] = {
        "batch": cfg.n_seq,
        "nt16_ms": round(res[16]["ms"], 4), "nt1_ms": round(res[1]["ms"], 4),
        "nt16": _spread(res[16]["per"]), "nt1": _spread(res[1]["per"]),
        "ratio_nt16_over_nt1": round(res[16]["ms"] / res[1]["ms"], 3),
        "nt16_committed_tok_s": round(1e3 / res[16]["ms"] * float(np.sum(res[16]["acc"] + 1)), 1),
        "nt16_committed_per_seq_round": round(float(np.mean(res[16]["acc"] + 1)), 3),
        "closed_form_committed_per_round": round(closed_form_committed(cfg.p_accept, 15,
                                                                       cfg.p_decay), 4),
        "nt1_hbm_frac": round(res[1]["bytes"] / res[1]["ms"] / 1e6 / (PEAK_HBM / 1e9), 4)}
    # one sequence of the batch, same model and cache contents
    import target_verification_amd as tva
    kv1 = tva.KVCache(wl.kv.k[:, :1].contiguous(), wl.kv.v[:, :1].contiguous(),
                      wl.kv.len[:1].clone())
    r1 = {}
    for nt in (16, 1):
        ms, per, acc, *_ = time_round(wl, ids[nt][:1], args.steps, args.warmup, graph, kv=kv1)
        r1[nt] = dict(ms=ms, per=per, bytes=wl.weight_bytes() + wl.kv_bytes(nt, n_seq=1))
        log(f"block16 one sequence nt={nt}: {ms:.4f} ms/round")
    out["q14b_8l_block16_single_sequence_nt16_vs_nt1"] = {
        "batch": 1, "nt16_ms": round(r1[16]["ms"], 4), "nt1_ms": round(r1[1]["ms"], 4),
        "nt16": _spread(r1[16]["per"]), "nt1": _spread(r1[1]["per"]),
        "ratio_nt16_over_nt1": round(r1[16]["ms"] / r1[1]["ms"], 3),
        "nt1_hbm_frac": round(r1[1]["bytes"] / r1[1]["ms"] / 1e6 / (PEAK_HBM / 1e9), 4)}
    del wl, kv1
    torch.cuda.empty_cache()
    return out


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

    if args.only in ("block16_nt16", "block16_nt1"):
        block16_lines(args, graph, only=args.only)
        return
    if args.only == "lm248k":
        stochastic_line(args.steps, args.warmup, graph)
        return

    # ---- headline: 14B-shaped stack, nt = 3 (and 9) ----
    q14b_48l = CONFIGS["q14b_48l"]
    want_cpu = not args.no_cpu and args.only is None
    wl = Workload(q14b_48l, nt_max=9, keep_host=want_cpu, headroom=LOOP_HEADROOM)
    wb = wl.weight_bytes()
    lines = {}
    nts = (3,) if args.no_extra else (3, 9)
    if args.only:
        nts = (3,) if args.only == "q14b_48l_nt3" else (9,)
    for nt in nts:
        t0 = time.time()
        ids = wl.drafts(nt)
        log(f"q14b_48l nt={nt}: drafts built in {time.time() - t0:.1f}s; timing {args.steps} steps")
        ms, per, acc, ids_t, ws, outs = time_round(wl, ids, args.steps, args.warmup, graph)
        metric_bytes = wb + wl.kv_bytes(nt)
        lines[nt] = dict(ms=ms, per=per, acc=acc, ids=ids, bytes=metric_bytes,
                         prof=profile_round(wl, ids_t, ws, outs, args.profile_rounds))
        log(f"q14b_48l nt={nt}: {ms:.4f} ms/round, {metric_bytes / ms / 1e6:.0f} GB/s, "
            f"a+1 = {(acc + 1).tolist()}")
    if args.only:
        return
    head = lines[3]
    prof = head["prof"]
    cb = class_bytes(wl, 3)
    gemm_classes = [c for c in prof if c in cb]
    dom = max(gemm_classes, key=lambda c: prof[c][1])
    n_l, tot, mn, mx = prof[dom]
    avg_ms = tot / n_l
    achieved = cb[dom] / (avg_ms * 1e-3) / 1e9
    # kernel template arguments: <format (2 = 4-bit/256, 3 = 6-bit/256),
    # 16-column tiles per wave, row arrangement (1 or 2: 16-row M tiles; 0:
    # one tile of at most 8 rows, high and low activation parts in one
    # operand; 3: the same for at most 4 rows, two k-steps per activation
    # load), epilogue (1 = RoPE and cache write, 2 = residual add, 3 =
    # SwiGLU, 4 = lm_head)>; the 3 rows of this line run the packed kernels
    # (the 6-bit lm_head the 8-row one)
    kern = {"gemm_gu": "k_qgemm<2, 4, 3, 3>", "gemm_qkv": "k_qgemm<2, 2, 3, 1>",
            "gemm_down": "k_qgemm<2, 2, 3, 2>", "gemm_o": "k_qgemm<2, 2, 3, 2>",
            "gemm_lm": "k_qgemm<3, 2, 0, 4>", "attn": "k_attn_chunk"}[dom]
    traffic = traffic_for(kern) if dom == "gemm_gu" else None
    prof_us = committed_profile(kern)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "frac": round(achieved / (PEAK_HBM / 1e9), 4),
                "traffic": traffic, "kernel": kern, "class": dom,
                "bytes_per_launch": cb[dom], "avg_launch_us": round(avg_ms * 1e3, 2),
                "launches_per_round": n_l // args.profile_rounds,
                "rocprof_avg_us": prof_us,
                "frac_at_rocprof_avg": (round(cb[dom] / (prof_us * 1e-6) / PEAK_HBM, 4)
                                        if prof_us else None)}
    per_class = {c: {"launches_per_round": v[0] // args.profile_rounds,
                     "ms_per_round": round(v[1] / args.profile_rounds, 4),
                     "avg_us": round(v[1] / v[0] * 1e3, 2)} for c, v in prof.items()}
    extra = {}
    if 9 in lines:
        l9 = lines[9]
        extra["q14b_48l_nt9"] = {
            "ms_per_round": round(l9["ms"], 4), **_spread(l9["per"]),
            "rounds_per_s": round(1e3 / l9["ms"], 2),
            "hbm_gbps": round(l9["bytes"] / l9["ms"] / 1e6, 1),
            "hbm_frac": round(l9["bytes"] / l9["ms"] / 1e6 / (PEAK_HBM / 1e9), 4),
            "ratio_to_nt3": round(l9["ms"] / head["ms"], 3),
            "replayed_round_committed": int(l9["acc"][0] + 1),
            "closed_form_committed_per_round": round(closed_form_committed(q14b_48l.p_accept, 8), 4)}
    if not args.no_extra:
        n_ref = 40 * 9 + 2
        t0 = time.time()
        ref, anchors = reference_stream(wl, n_ref)
        log(f"q14b_48l: one-token reference stream of {n_ref} tokens in {time.time() - t0:.1f}s")
        for nt in (3, 9):
            lp = loop_line(wl, ref, anchors, nt, 36, q14b_48l.p_accept, graph)
            extra[f"q14b_48l_loop_nt{nt}"] = lp
            log(f"q14b_48l device loop nt={nt}: {lp}")
        if 9 in extra.get("q14b_48l_nt9", {}) or "q14b_48l_nt9" in extra:
            extra["q14b_48l_nt9"]["loop_committed_tok_s"] = extra["q14b_48l_loop_nt9"]["committed_tok_s"]
        # the drafter cost the pages measured relative to a one-row verify
        # (the minfer plan: C_D 2.9 ms per token against C_T(1) 39.0 ms),
        # applied to this library's measured nt = 3 round
        draft_ms = round(2.9 / 39.0 * head["ms"], 4)
        for dms in (0.0, draft_ms):
            ad = adaptive_line(wl, ref, anchors, 40, q14b_48l.p_accept, draft_ms=dms)
            extra["q14b_48l_adaptive_depth" + ("" if dms == 0.0 else "_with_draft_cost")] = ad
            log(f"q14b_48l adaptive depth (draft {dms} ms/token): {ad}")
    cpu = None
    if want_cpu:
        log("cpu baseline: one whole oracle round ...")
        cpu, _ = cpu_baseline(wl, head["ids"])
        log(f"cpu baseline: {cpu}")
    del wl
    torch.cuda.empty_cache()

    if not args.no_extra:
        extra["stream_ceiling"] = stream_ceiling()
        log(f"stream ceiling: {extra['stream_ceiling']}")
        extra["q14b_48l_nt3_capacity32k"] = capacity_line(args.steps, args.warmup, graph)
        extra.update(block16_lines(args, graph))
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
        "replays": _spread(head["per"]),
        "committed_tok_s": round(rps * float(np.mean(head["acc"] + 1)), 2),
        "replayed_round_committed": int(head["acc"][0] + 1),
        "closed_form_committed_per_round": round(closed_form_committed(q14b_48l.p_accept, 2), 4),
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
