"""Python binding of libspecverify.so, the MI355X verify-round library.

Argument marshalling only: every step of the round runs in the library's HIP
kernels.  The functions below carry the C ABI's names (include/specverify.h)
and take torch CUDA tensors, whose device pointers and the current stream are
passed through ctypes.  Loading fails loudly if the library has not been
built (python -m target_verification_amd.build); there is no other path.
"""

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; SPECVERIFY_LIB may name another build of the same
# library (for example to compare two builds in one process session).
LIB_PATH = os.environ.get("SPECVERIFY_LIB") or os.path.join(_HERE, "libspecverify.so")

SV_OK, SV_E_INVALID, SV_E_UNSUPPORTED, SV_E_CAPACITY, SV_E_HIP, SV_E_FAULT_INJECTED, \
    SV_E_NOMEM, SV_E_NUMERIC, SV_E_TIMEOUT = 0, -1, -2, -3, -4, -5, -6, -7, -8
SV_B4_32, SV_B4_256, SV_B6_256 = 1, 2, 3
SV_GREEDY, SV_REJECT, SV_SAMPLE = 0, 1, 2
SV_MAX_NT = 16
KV_CHUNK = 128
FMT_CODE = {"b4_32": SV_B4_32, "b4_256": SV_B4_256, "b6_256": SV_B6_256}

EXPORTS = ("sv_model_create", "sv_model_destroy", "sv_workspace_bytes", "spec_verify_round",
           "spec_verify_round_static",
           "sv_qweight_create", "sv_qweight_destroy", "sv_qgemm_workspace_bytes", "sv_qgemm",
           "sv_advance", "sv_depth_create", "sv_depth_destroy", "sv_depth_observe",
           "sv_depth_next", "sv_depth_estimates", "sv_profile_begin", "sv_profile_end",
           "sv_status_string", "sv_version")
PROF_CLASSES = ("embed", "gemm_qkv", "epi_qkv", "attn", "combine", "gemm_o", "epi_o", "gemm_gu",
                "epi_gu", "gemm_down", "epi_down", "gemm_lm", "epi_lm", "decide", "other",
                "layer")

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


class SvModelDesc(ctypes.Structure):
    _fields_ = [("n_layer", _i32), ("hidden", _i32), ("n_head", _i32), ("n_kv_head", _i32),
                ("head_dim", _i32), ("ffn", _i32), ("vocab", _i32), ("max_pos", _i32),
                ("rms_eps", ctypes.c_float), ("rope_base", ctypes.c_float),
                ("fmt_proj", _i32), ("fmt_lm", _i32), ("lm_only", _i32), ("reserved", _i32),
                ("tok_embd", _vp), ("attn_norm", _vp), ("ffn_norm", _vp), ("out_norm", _vp),
                ("wq", _vp), ("wk", _vp), ("wv", _vp), ("wo", _vp), ("w_gate", _vp),
                ("w_up", _vp), ("w_down", _vp), ("lm_head", _vp)]


class SvKV(ctypes.Structure):
    _fields_ = [("n_seq", _i32), ("capacity", _i32), ("k", _vp), ("v", _vp), ("len", _vp)]


class SvProfileStat(ctypes.Structure):
    _fields_ = [("launches", _i32), ("reserved", _i32), ("total_ms", ctypes.c_double),
                ("min_ms", ctypes.c_double), ("max_ms", ctypes.c_double)]


class SvRound(ctypes.Structure):
    _fields_ = [("n_seq", _i32), ("nt", _i32), ("mode", _i32), ("temperature", ctypes.c_float),
                ("ids", _vp), ("hidden", _vp), ("draft_logits", _vp), ("uniforms", _vp),
                ("accepted_len", _vp), ("emitted", _vp), ("logits", _vp), ("argmax", _vp),
                ("commit", _i32), ("max_len", _i32), ("nts", _vp)]


class SvAdvanceArgs(ctypes.Structure):
    _fields_ = [("n_seq", _i32), ("nt", _i32), ("ids", _vp), ("accepted_len", _vp),
                ("emitted", _vp), ("len", _vp), ("tokens", _vp), ("tok_cap", _i32),
                ("committed", _vp), ("ref", _vp), ("draw", _vp), ("noise", _vp),
                ("ref_cap", _i32), ("p_accept", ctypes.c_float), ("p_decay", ctypes.c_float),
                ("utab", _vp), ("uniforms", _vp)]


_lib = None


def lib():
    """The loaded library (raises if it is missing: no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m target_verification_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.sv_model_create.argtypes = [ctypes.POINTER(SvModelDesc), ctypes.POINTER(_vp)]
        L.sv_model_create.restype = ctypes.c_int
        L.sv_model_destroy.argtypes = [_vp]
        L.sv_model_destroy.restype = None
        L.sv_workspace_bytes.argtypes = [_vp, _i32, _i32, _i32]
        L.sv_workspace_bytes.restype = ctypes.c_size_t
        L.spec_verify_round.argtypes = [_vp, ctypes.POINTER(SvKV), ctypes.POINTER(SvRound), _vp,
                                        ctypes.c_size_t, _vp]
        L.spec_verify_round.restype = ctypes.c_int
        L.spec_verify_round_static.argtypes = [_vp, ctypes.POINTER(SvKV), ctypes.POINTER(SvRound),
                                               _vp]
        L.spec_verify_round_static.restype = ctypes.c_int
        L.sv_qweight_create.argtypes = [_i32, ctypes.c_int64, ctypes.c_int64, _vp,
                                        ctypes.POINTER(_vp)]
        L.sv_qweight_create.restype = ctypes.c_int
        L.sv_qweight_destroy.argtypes = [_vp]
        L.sv_qweight_destroy.restype = None
        L.sv_qgemm_workspace_bytes.argtypes = [_vp, _i32]
        L.sv_qgemm_workspace_bytes.restype = ctypes.c_size_t
        L.sv_qgemm.argtypes = [_vp, _vp, _vp, _i32, _vp, _vp, ctypes.c_size_t, _vp]
        L.sv_qgemm.restype = ctypes.c_int
        L.sv_advance.argtypes = [ctypes.POINTER(SvAdvanceArgs), _vp]
        L.sv_advance.restype = ctypes.c_int
        L.sv_depth_create.argtypes = [_i32, _i32, ctypes.c_float, ctypes.c_float,
                                      ctypes.c_float, ctypes.c_float, ctypes.POINTER(_vp)]
        L.sv_depth_create.restype = ctypes.c_int
        L.sv_depth_destroy.argtypes = [_vp]
        L.sv_depth_destroy.restype = None
        L.sv_depth_observe.argtypes = [_vp, _i32, _i32, _vp, ctypes.c_double]
        L.sv_depth_observe.restype = ctypes.c_int
        L.sv_depth_next.argtypes = [_vp]
        L.sv_depth_next.restype = _i32
        L.sv_depth_estimates.argtypes = [_vp, _vp, _vp, _vp]
        L.sv_depth_estimates.restype = ctypes.c_int
        L.sv_profile_begin.argtypes = [_i32]
        L.sv_profile_begin.restype = ctypes.c_int
        L.sv_profile_end.argtypes = [ctypes.POINTER(SvProfileStat)]
        L.sv_profile_end.restype = ctypes.c_int
        L.sv_status_string.argtypes = [_i32]
        L.sv_status_string.restype = ctypes.c_char_p
        L.sv_version.argtypes = []
        L.sv_version.restype = _i32
        _lib = L
    return _lib


class SvError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__(f"{what}: {sv_status_string(status)} ({status})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def sv_status_string(status: int) -> str:
    return lib().sv_status_string(int(status)).decode()


def sv_version() -> int:
    return int(lib().sv_version())


def sv_model_create(desc: SvModelDesc):
    out = _vp()
    rc = lib().sv_model_create(ctypes.byref(desc), ctypes.byref(out))
    if rc != SV_OK:
        raise SvError(rc, "sv_model_create")
    return out


def sv_model_destroy(handle):
    lib().sv_model_destroy(handle)


def sv_workspace_bytes(handle, n_seq, nt, mode) -> int:
    return int(lib().sv_workspace_bytes(handle, n_seq, nt, mode))


def spec_verify_round(handle, kv: SvKV, rnd: SvRound, workspace: torch.Tensor,
                      stream=None) -> int:
    """Enqueue one round; returns the sv_status (asynchronous on success)."""
    st = _stream() if stream is None else ctypes.c_void_p(stream)
    return int(lib().spec_verify_round(handle, ctypes.byref(kv) if kv is not None else None,
                                       ctypes.byref(rnd), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), st))


def spec_verify_round_static(handle, kv: SvKV, rnd: SvRound, stream=None) -> int:
    """Enqueue one round on the library's own scratch array (no workspace,
    nothing allocated); returns the sv_status."""
    st = _stream() if stream is None else ctypes.c_void_p(stream)
    return int(lib().spec_verify_round_static(handle, ctypes.byref(kv) if kv is not None
                                              else None, ctypes.byref(rnd), st))


def sv_advance(ids, accepted_len, emitted, lens, *, tokens=None, committed=None, ref=None,
               draw=None, noise=None, p_accept=0.0, p_decay=1.0, utab=None, uniforms=None,
               stream=None):
    """Enqueue the next round's ids from a committed round (device tensors:
    ids int32 [S][nt] updated in place, accepted_len / emitted / lens int32
    [S]; tokens int32 [S][tok_cap] log by position; committed int32 [S]
    running count; ref / noise int32 and draw fp32 [S][ref_cap] for the stub
    drafter; utab fp64 [S][ref_cap] draws by position, gathered into
    uniforms fp64 [S][nt] for the next SV_SAMPLE round).  Raises SvError on
    a returned error status."""
    S, nt = ids.shape
    a = SvAdvanceArgs()
    a.n_seq, a.nt = S, nt
    a.ids, a.accepted_len, a.emitted, a.len = (_ptr(ids), _ptr(accepted_len), _ptr(emitted),
                                               _ptr(lens))
    a.tokens = _ptr(tokens) if tokens is not None else None
    a.tok_cap = tokens.shape[1] if tokens is not None else 0
    a.committed = _ptr(committed) if committed is not None else None
    a.ref = _ptr(ref) if ref is not None else None
    a.draw = _ptr(draw) if draw is not None else None
    a.noise = _ptr(noise) if noise is not None else None
    cap_src = noise if noise is not None else utab
    a.ref_cap = cap_src.shape[1] if cap_src is not None else 0
    a.utab = _ptr(utab) if utab is not None else None
    a.uniforms = _ptr(uniforms) if uniforms is not None else None
    a.p_accept, a.p_decay = float(p_accept), float(p_decay)
    st = _stream() if stream is None else ctypes.c_void_p(stream)
    rc = int(lib().sv_advance(ctypes.byref(a), st))
    if rc != SV_OK:
        raise SvError(rc, "sv_advance")


class DepthPolicy:
    """Adaptive draft depth (host only): marshals sv_depth_* (host arrays)."""

    def __init__(self, d_max=7, d_start=2, prior_a=1.0, prior_b=1.0, hysteresis=0.10,
                 draft_ms=0.0):
        self.d_max = d_max
        h = _vp()
        rc = lib().sv_depth_create(d_max, d_start, prior_a, prior_b, hysteresis, draft_ms,
                                   ctypes.byref(h))
        if rc != SV_OK:
            raise SvError(rc, "sv_depth_create")
        self.handle = h

    def observe(self, d, accepted_len, round_ms=0.0):
        acc = np.ascontiguousarray(np.asarray(accepted_len, dtype=np.int32))
        rc = lib().sv_depth_observe(self.handle, int(d), acc.size,
                                    acc.ctypes.data_as(_vp), float(round_ms))
        if rc != SV_OK:
            raise SvError(rc, "sv_depth_observe")

    def next(self) -> int:
        d = int(lib().sv_depth_next(self.handle))
        if d < 0:
            raise SvError(d, "sv_depth_next")
        return d

    def estimates(self):
        acc = np.zeros(self.d_max)
        cost = np.zeros(self.d_max + 1)
        rate = np.zeros(self.d_max + 1)
        ptr = lambda x: x.ctypes.data_as(_vp)
        rc = lib().sv_depth_estimates(self.handle, ptr(acc), ptr(cost), ptr(rate))
        if rc != SV_OK:
            raise SvError(rc, "sv_depth_estimates")
        return acc, cost, rate

    def close(self):
        if getattr(self, "handle", None):
            lib().sv_depth_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def sv_qweight_create(fmt: int, rows: int, cols: int, canonical: torch.Tensor):
    out = _vp()
    rc = lib().sv_qweight_create(fmt, rows, cols, _ptr(canonical), ctypes.byref(out))
    if rc != SV_OK:
        raise SvError(rc, "sv_qweight_create")
    return out


def sv_qweight_destroy(handle):
    lib().sv_qweight_destroy(handle)


def sv_qgemm_workspace_bytes(handle, m_rows) -> int:
    return int(lib().sv_qgemm_workspace_bytes(handle, m_rows))


def sv_qgemm(handle, x: torch.Tensor, scale, m_rows: int, y: torch.Tensor,
             workspace: torch.Tensor) -> int:
    return int(lib().sv_qgemm(handle, _ptr(x), _ptr(scale), m_rows, _ptr(y), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream()))


def sv_profile_begin(max_launches: int) -> None:
    rc = lib().sv_profile_begin(int(max_launches))
    if rc != SV_OK:
        raise SvError(rc, "sv_profile_begin")


def sv_profile_end() -> dict:
    """Per-kernel-class timing of the launches since sv_profile_begin:
    {class: (launches, total_ms, min_ms, max_ms)}."""
    arr = (SvProfileStat * len(PROF_CLASSES))()
    rc = lib().sv_profile_end(arr)
    if rc < 0:
        raise SvError(rc, "sv_profile_end")
    return {name: (arr[i].launches, arr[i].total_ms, arr[i].min_ms, arr[i].max_ms)
            for i, name in enumerate(PROF_CLASSES) if arr[i].launches}


# ---- marshalling helpers ----------------------------------------------------

def kv_to_library_layout(K: torch.Tensor, V: torch.Tensor):
    """[layer][seq][pos][kv_head][hd] fp16 -> (k [layer][seq][kv_head][pos][hd],
    v [layer][seq][kv_head][hd][pos]), both contiguous."""
    return (K.permute(0, 1, 3, 2, 4).contiguous(), V.permute(0, 1, 3, 4, 2).contiguous())


def kv_from_library_layout(k: torch.Tensor, v: torch.Tensor):
    return (k.permute(0, 1, 3, 2, 4).contiguous(), v.permute(0, 1, 4, 2, 3).contiguous())


class QWeight:
    """A repacked single tensor for sv_qgemm (owns the library handle)."""

    def __init__(self, fmt: str, canonical: torch.Tensor, rows: int, cols: int):
        self.rows, self.cols = rows, cols
        self.handle = sv_qweight_create(FMT_CODE[fmt], rows, cols, canonical)

    def gemm(self, x: torch.Tensor, scale=None) -> torch.Tensor:
        m = x.shape[0]
        ws = torch.empty(sv_qgemm_workspace_bytes(self.handle, m), dtype=torch.uint8,
                         device=x.device)
        y = torch.empty((m, self.rows), dtype=torch.float32, device=x.device)
        rc = sv_qgemm(self.handle, x.contiguous(), scale, m, y, ws)
        if rc != SV_OK:
            raise SvError(rc, "sv_qgemm")
        return y

    def __del__(self):
        try:
            if getattr(self, "handle", None) is not None and _lib is not None:
                sv_qweight_destroy(self.handle)
                self.handle = None
        except Exception:
            pass


class Model:
    """Creates an sv_model from canonical tensors on the GPU.

    tensors: dict as made by synth.make.make_weights (device tensors).  The
    model keeps references to the tensors it borrows (token table, norms)."""

    def __init__(self, spec, tensors: dict, max_pos: int):
        self.spec = spec
        self._keep = []
        d = SvModelDesc()
        d.n_layer = 0 if spec.lm_only else spec.n_layer
        d.hidden, d.n_head, d.n_kv_head = spec.hidden, spec.n_head, spec.n_kv_head
        d.head_dim, d.ffn, d.vocab, d.max_pos = spec.head_dim, spec.ffn, spec.vocab, max_pos
        d.rms_eps, d.rope_base = spec.rms_eps, spec.rope_base
        d.fmt_proj, d.fmt_lm = FMT_CODE[spec.fmt_proj], FMT_CODE[spec.fmt_lm]
        d.lm_only = 1 if spec.lm_only else 0

        def keep(t):
            t = t.contiguous()
            self._keep.append(t)
            return t.data_ptr()

        if not spec.lm_only:
            d.tok_embd = keep(tensors["tok_embd"])
            d.attn_norm = keep(tensors["attn_norm"].float())
            d.ffn_norm = keep(tensors["ffn_norm"].float())
            d.out_norm = keep(tensors["out_norm"].float())
            arrays = []
            for name in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
                arr = (_vp * spec.n_layer)(*[keep(t) for t in tensors[name]])
                arrays.append(arr)
                setattr(d, name, ctypes.cast(arr, _vp).value)
            self._arrays = arrays
        d.lm_head = keep(tensors["lm_head"])
        self.desc = d
        self.handle = sv_model_create(d)
        # kept on the object: at interpreter exit the module's globals may be
        # cleared before this object is collected
        self._destroy = sv_model_destroy
        # the quantized tensors were repacked; drop our references to them
        self._keep = [t for t in self._keep if t.dtype != torch.uint8]

    def workspace(self, n_seq, nt, mode, device="cuda"):
        n = sv_workspace_bytes(self.handle, n_seq, nt, mode)
        return torch.empty(n, dtype=torch.uint8, device=device)

    def close(self):
        if getattr(self, "handle", None) is not None:
            self._destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class KVCache:
    """The library-layout cache plus the device length array."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, lens: torch.Tensor):
        self.k, self.v, self.len = k, v, lens
        self.n_seq, self.capacity = k.shape[1], k.shape[3]
        self.sv = SvKV(self.n_seq, self.capacity, k.data_ptr(), v.data_ptr(), lens.data_ptr())

    @classmethod
    def from_logical(cls, K, V, lens):
        k, v = kv_to_library_layout(K, V)
        return cls(k, v, torch.as_tensor(lens, dtype=torch.int32, device=k.device).clone())


def verify_round(model: Model, kv, ids, *, mode=SV_GREEDY, temperature=0.0, hidden=None,
                 draft_logits=None, uniforms=None, want_logits=True, commit=1,
                 workspace=None, outs=None, nts=None, static_scratch=False, max_len=0):
    """Marshal one spec_verify_round call (spec_verify_round_static with
    static_scratch: no workspace).  ids int32 [S][nt] (device).  max_len: 0,
    or an upper bound on every sequence's length this round (attention then
    visits only the key chunks below max_len + nt).  Returns dict
    of device tensors (accepted_len, emitted, logits, argmax); raises SvError
    on a returned error status."""
    S, nt = ids.shape
    dev = ids.device
    if outs is None:
        outs = dict(accepted_len=torch.empty(S, dtype=torch.int32, device=dev),
                    emitted=torch.empty(S, dtype=torch.int32, device=dev),
                    argmax=torch.empty((S, nt), dtype=torch.int32, device=dev),
                    logits=(torch.empty((S, nt, model.spec.vocab), dtype=torch.float32,
                                        device=dev) if want_logits else None))
    if workspace is None and not static_scratch:
        workspace = model.workspace(S, nt, mode, dev)
        if workspace.numel() == 0:   # sizes the library refuses: let it say why
            workspace = torch.empty(256, dtype=torch.uint8, device=dev)
    r = SvRound()
    r.n_seq, r.nt, r.mode, r.temperature = S, nt, mode, float(temperature)
    r.ids = ids.data_ptr()
    r.hidden = hidden.data_ptr() if hidden is not None else None
    r.draft_logits = draft_logits.data_ptr() if draft_logits is not None else None
    r.uniforms = uniforms.data_ptr() if uniforms is not None else None
    r.accepted_len = outs["accepted_len"].data_ptr()
    r.emitted = outs["emitted"].data_ptr()
    r.logits = outs["logits"].data_ptr() if outs.get("logits") is not None else None
    r.argmax = outs["argmax"].data_ptr() if outs.get("argmax") is not None else None
    r.commit = int(commit)
    r.max_len = int(max_len)
    r.nts = nts.data_ptr() if nts is not None else None
    if static_scratch:
        rc = spec_verify_round_static(model.handle, kv.sv if kv is not None else None, r)
    else:
        rc = spec_verify_round(model.handle, kv.sv if kv is not None else None, r, workspace)
    if rc != SV_OK:
        raise SvError(rc, "spec_verify_round_static" if static_scratch else "spec_verify_round")
    return outs
