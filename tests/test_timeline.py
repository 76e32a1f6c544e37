"""Host logic of the timeline tool: the per-class summary of a synthetic
table whose spans, gaps, loop times and epilogue parts are known by
construction."""

import numpy as np

from target_verification_amd.timeline import summarize, LAYERS, KINDS, WG, FIELDS


def test_summary_of_a_constructed_timeline():
    t = np.zeros((LAYERS, KINDS, WG, FIELDS), dtype=np.int64)
    clock = 1000
    order = (0, 1, 2, 3, 4, 5)
    spans = {0: 900, 1: 700, 2: 400, 3: 800, 4: 2400, 5: 1600}   # ticks of 10 ns
    gap = 150
    for l in range(3):
        for k in order:
            start = clock + gap
            for wgi in range(4):                  # four workgroups, staggered starts
                s0 = start + 10 * wgi
                e = start + spans[k] - 10 * (3 - wgi)
                lp = s0 + (e - s0) // 2
                # staged 20 ticks after the loop, barrier 10 later, stores
                # issued 30 later and acknowledged 5 after that
                t[l, k, wgi] = (s0, lp, e, lp + 20, lp + 60, lp + 30, lp + 65)
            clock = start + spans[k]
    s = summarize(t, 3)
    for k, name in enumerate(("qkv", "chunk", "merge", "o", "gu", "down")):
        assert abs(s[name]["span"] - spans[k] / 100) < 1e-9, name
        assert abs(s[name]["gap"] - gap / 100) < 1e-9, name
    # GEMM loops end half way through each workgroup
    wg = [(spans[0] - 10 * (3 - i) - 10 * i) for i in range(4)]
    assert abs(s["qkv"]["loop_max"] - max(w // 2 for w in wg) / 100) < 1e-9
    for name in ("qkv", "o", "gu", "down"):
        assert abs(s[name]["staging"] - 0.20) < 1e-9, name
        assert abs(s[name]["barrier"] - 0.10) < 1e-9, name
        assert abs(s[name]["arithmetic"] - 0.30) < 1e-9, name
        assert abs(s[name]["stores"] - 0.05) < 1e-9, name
        assert abs(s[name]["end"] + 0.65 - s[name]["epi_p50"]) < 1e-9, name
    assert s["chunk"]["loop_p50"] is None and s["chunk"]["staging"] is None
