"""The library's host code under AddressSanitizer and UndefinedBehavior-
Sanitizer, on the CPU (no GPU needed or used).

The sources are compiled with both sanitizers for the host side only (the
device code is compiled as usual and never runs here) into a library of
its own under _build/sanitize/.  A child Python process loads it with the
ASan runtime preloaded (Python itself is not instrumented) and drives every
entry point that runs without a GPU: status strings and version, the
argument checks of every call (NULL, out-of-range and inconsistent
arguments), every branch of model-descriptor validation, and the adaptive
depth policy over a long simulated run with edge inputs.  Any sanitizer
report, or a result other than the documented status, fails the test.
Leak checking is off: the interpreter's own allocations are not ours."""

import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "target_verification_amd", "csrc")
OUT_DIR = os.path.join(ROOT, "_build", "sanitize")
LIB = os.path.join(OUT_DIR, "libspecverify_sanitize.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
# each host-side sanitizer flag follows its own -Xarch_host
HOST_SAN = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
            "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer").split()


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".h")))


def _build():
    os.makedirs(OUT_DIR, exist_ok=True)
    newest = max(os.path.getmtime(f) for f in _sources())
    if os.path.exists(LIB) and os.path.getmtime(LIB) > newest:
        return
    hips = [f for f in _sources() if f.endswith(".hip")]
    procs, objs = [], []
    for src in hips:
        obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
        objs.append(obj)
        procs.append(subprocess.Popen(
            [HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN,
             "-c", src, "-o", obj], stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
    for src, p in zip(hips, procs):
        out = p.communicate()[0].decode()
        assert p.returncode == 0, f"{src}:\n{out[-3000:]}"
    link = [HIPCC, "-shared", "--offload-arch=gfx950", *HOST_SAN[:4], "-Xarch_host",
            "-shared-libsan", "-o", LIB + ".tmp", *objs]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    os.replace(LIB + ".tmp", LIB)


CHILD = textwrap.dedent(r'''
    import ctypes, math, sys
    import numpy as np
    import target_verification_amd as tva
    lib = tva.lib()
    g = ctypes.CDLL(None)
    assert hasattr(g, "__asan_init") and hasattr(g, "__ubsan_handle_add_overflow")
    ok, st = tva.SV_OK, tva
    assert tva.sv_version() == 1
    for code in range(0, -9, -1):
        assert isinstance(tva.sv_status_string(code), str)
    assert isinstance(tva.sv_status_string(-99), str)
    out = ctypes.c_void_p()

    # ---- model descriptors: every validation branch before device work
    def desc(**kw):
        d = tva.SvModelDesc()
        f = dict(n_layer=2, hidden=512, n_head=8, n_kv_head=2, head_dim=128, ffn=1024,
                 vocab=2048, fmt_proj=tva.SV_B4_256, fmt_lm=tva.SV_B6_256, lm_only=0,
                 max_pos=256, rms_eps=1e-6, rope_base=1e6)
        f.update(kw)
        for k, v in f.items():
            setattr(d, k, v)
        for p in ("tok_embd", "attn_norm", "ffn_norm", "out_norm", "lm_head"):
            setattr(d, p, 4096)
        for p in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
            setattr(d, p, 4096)
        return d
    def create(d):
        return lib.sv_model_create(ctypes.byref(d), ctypes.byref(out))
    assert lib.sv_model_create(None, ctypes.byref(out)) == st.SV_E_INVALID
    assert lib.sv_model_create(ctypes.byref(desc()), None) == st.SV_E_INVALID
    cases = [
        (dict(n_layer=-1), st.SV_E_INVALID), (dict(hidden=0), st.SV_E_INVALID),
        (dict(vocab=0), st.SV_E_INVALID), (dict(fmt_lm=9), st.SV_E_UNSUPPORTED),
        (dict(hidden=300), st.SV_E_UNSUPPORTED), (dict(vocab=2047), st.SV_E_UNSUPPORTED),
        (dict(hidden=8448), st.SV_E_UNSUPPORTED), (dict(lm_only=1), st.SV_E_INVALID),
        (dict(n_layer=0), st.SV_E_INVALID), (dict(fmt_proj=tva.SV_B6_256), st.SV_E_UNSUPPORTED),
        (dict(n_head=0), st.SV_E_INVALID), (dict(n_head=6, n_kv_head=4), st.SV_E_INVALID),
        (dict(head_dim=96), st.SV_E_UNSUPPORTED), (dict(ffn=1000), st.SV_E_UNSUPPORTED),
        (dict(n_head=3, n_kv_head=1, head_dim=64), st.SV_E_UNSUPPORTED),
        (dict(max_pos=0), st.SV_E_INVALID), (dict(rms_eps=0.0), st.SV_E_INVALID),
        (dict(rms_eps=float("nan")), st.SV_E_INVALID), (dict(rope_base=-1.0), st.SV_E_INVALID),
    ]
    for kw, want in cases:
        got = create(desc(**kw))
        assert got == want, (kw, got, want)
        assert out.value is None, kw
    for p in ("tok_embd", "wq", "w_down", "lm_head"):
        d = desc(); setattr(d, p, None)
        assert create(d) == st.SV_E_INVALID, p

    # ---- calls that need a model or device buffers reject NULL and bad sizes
    assert lib.spec_verify_round(None, None, None, None, 0, None) == st.SV_E_INVALID
    assert lib.spec_verify_round_static(None, None, None, None) == st.SV_E_INVALID
    assert lib.sv_workspace_bytes(None, 1, 3, 0) == 0
    assert lib.sv_advance(None, None) == st.SV_E_INVALID
    a = tva.SvAdvanceArgs(); a.n_seq, a.nt = 1, 3
    assert lib.sv_advance(ctypes.byref(a), None) == st.SV_E_INVALID
    a.n_seq = -1
    assert lib.sv_advance(ctypes.byref(a), None) == st.SV_E_INVALID
    assert lib.sv_qweight_create(tva.SV_B4_256, 32, 256, None, ctypes.byref(out)) == st.SV_E_INVALID
    assert lib.sv_qweight_create(9, 32, 256, ctypes.c_void_p(16), ctypes.byref(out)) == st.SV_E_UNSUPPORTED
    for rows, cols in ((0, 256), (32, 0), (31, 256), (32, 100), (-32, 256)):
        rc = lib.sv_qweight_create(tva.SV_B4_256, rows, cols, ctypes.c_void_p(16), ctypes.byref(out))
        assert rc in (st.SV_E_INVALID, st.SV_E_UNSUPPORTED), (rows, cols, rc)
    assert lib.sv_qgemm_workspace_bytes(None, 3) == 0

    # ---- adaptive depth policy (pure host code)
    h = ctypes.c_void_p()
    bad = [(0, 0, 1, 1, .1, 0), (16, 0, 1, 1, .1, 0), (4, 5, 1, 1, .1, 0), (4, -1, 1, 1, .1, 0),
           (4, 2, 0, 1, .1, 0), (4, 2, 1, -1, .1, 0), (4, 2, 1, 1, -.1, 0), (4, 2, 1, 1, .1, -1),
           (4, 2, float("nan"), 1, .1, 0)]
    for args in bad:
        assert lib.sv_depth_create(*args, ctypes.byref(h)) == st.SV_E_INVALID, args
        assert h.value is None
    rng = np.random.default_rng(5)
    for d_max in (1, 7, 15):
        pol = tva.DepthPolicy(d_max=d_max, d_start=min(2, d_max), draft_ms=0.05)
        d = pol.next()
        for r in range(400):
            n = int(rng.integers(1, 13))
            acc = np.minimum(rng.geometric(0.3, size=n) - 1, d).astype(np.int32)
            acc[rng.random(n) < 0.1] = -3                 # failed sequences are skipped
            pol.observe(d, acc, float(1.0 + 0.05 * d + rng.random() * 0.1) if r % 7 else 0.0)
            d = pol.next()
            assert 0 <= d <= d_max
        accp, cost, rate = pol.estimates()
        assert len(accp) == d_max and len(cost) == d_max + 1
        assert all(math.isfinite(x) for x in rate)
        hp = pol.handle
        assert lib.sv_depth_observe(hp, d_max + 1, 1, np.zeros(1, np.int32).ctypes.data, 1.0) == st.SV_E_INVALID
        over = np.array([d_max + 1], np.int32)
        assert lib.sv_depth_observe(hp, d_max, 1, over.ctypes.data, 1.0) == st.SV_E_INVALID
        assert lib.sv_depth_observe(hp, 0, 0, None, 1.0) in (st.SV_OK, st.SV_E_INVALID)
        assert lib.sv_depth_estimates(hp, None, None, None) == st.SV_OK
        pol.close()
    assert lib.sv_depth_next(None) < 0
    assert lib.sv_depth_observe(None, 1, 1, None, 1.0) == st.SV_E_INVALID
    lib.sv_depth_destroy(None)
    print("host checks passed")
''')


def test_host_code_under_asan_and_ubsan():
    if not os.path.exists(HIPCC) or not os.path.exists(CLANG):
        pytest.skip("hipcc / clang not available")
    _build()
    rt = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True).stdout.strip()
    assert os.path.exists(rt), rt
    env = dict(os.environ, LD_PRELOAD=rt, SPECVERIFY_LIB=LIB,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               HIP_VISIBLE_DEVICES="")
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    r = subprocess.run([sys.executable, "-c", CHILD], env=env, capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    # the library under test is the instrumented one
    assert subprocess.run(["nm", "-D", LIB], capture_output=True, text=True).stdout.count(
        "__asan_report") > 0
    assert "AddressSanitizer" not in report and "runtime error:" not in report, report[-4000:]
    assert "host checks passed" in r.stdout
