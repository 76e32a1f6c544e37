"""fp64 forward of the target model's verify rows.

TEST INFRASTRUCTURE (part of the oracle): see oracle/__init__.py.

Model (the workloads name a pre-norm decoder with RMSNorm, RoPE, GQA
attention and a SwiGLU FFN; biases are absent):

  x   = E[id]                                           (fp16 table -> fp64)
  per layer l:
    h   = RMSNorm(x; g_attn[l])
    q   = Wq h,  k = Wk h,  v = Wv h
    q,k = RoPE(q, k; pos)                               (pairs i, i + hd/2)
    K[pos] = fp16(k), V[pos] = fp16(v)                  (write the cache row)
    o_j = sum_i softmax_i(q_j . K_i / sqrt(hd)) V_i     (keys 0..pos, read from
                                                         the fp16 cache, kv head
                                                         j // (n_head/n_kv_head))
    x  += Wo o
    h2  = RMSNorm(x; g_ffn[l])
    x  += Wd (silu(Wg h2) * (Wu h2)),   silu(z) = z / (1 + e^-z)
  logits = W_lm RMSNorm(x; g_out)

RMSNorm(x; g) = x * g / sqrt(mean(x^2) + eps).  RoPE angle of pair i at
position pos is pos * base^(-2i/hd).

Row r of a verify round sits at position len + r.  Every row goes through
exactly this sequence of fp64 operations, whether it is computed alone (one
row of plain autoregressive decoding with the drafted ids teacher-forced)
or together with other rows: this is the "one target pass over the anchor and
the proposal block" of the Power page's exactness transaction, evaluated the
slow way.  Rows are evaluated layer by layer (all rows of the call through
layer l, then layer l + 1), so only one layer's decoded weights are needed at
a time.  Inside a layer every row's new K/V row is written into the fp16
cache before any row attends; row r reads keys 0..pos_r only, so in-block
rows see the fp16-rounded keys and values of the rows before them, the same
values a one-row decode would read back, and never a later row.

A product W h is computed per fixed chunk of output features: the chunk's
weights are decoded, and each fixed sub-chunk of them is multiplied against
each row's h separately (one matrix-vector product per row and sub-chunk,
on a block of weights that stays in the processor's cache).  The chunk and
sub-chunk boundaries depend only on the tensor, so a row's bits never
depend on how many rows share a call.  Chunks run on a pool of host threads
(the BLAS library itself runs single-threaded meanwhile), which changes no
arithmetic.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .formats import decode

CHUNK_ROWS = 512   # output features per decoded chunk
SUB_ROWS = 32      # output features per matrix-vector product


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x * np.asarray(g, dtype=np.float64) / np.sqrt(np.mean(x * x) + eps)


def rope_angles(pos: int, head_dim: int, base: float) -> np.ndarray:
    i = np.arange(head_dim // 2, dtype=np.float64)
    return float(pos) * np.power(float(base), -2.0 * i / head_dim)


def rope(v: np.ndarray, pos: int, base: float) -> np.ndarray:
    """Rotate each head of v [n_heads][hd]: pair (i, i + hd/2) by pos*theta_i."""
    hd = v.shape[-1]
    half = hd // 2
    ang = rope_angles(pos, hd, base)
    c, s = np.cos(ang), np.sin(ang)
    a, b = v[..., :half], v[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """One query row q [hd] over keys K [n][hd] and values V [n][hd]."""
    s = (K @ q) / np.sqrt(q.shape[-1])
    w = np.exp(s - s.max())
    w = w / w.sum()
    return w @ V


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


class _OneBlasThread:
    """Run BLAS single-threaded while the chunk pool is active."""

    def __enter__(self):
        try:
            from threadpoolctl import threadpool_limits
            self._lim = threadpool_limits(limits=1, user_api="blas")
        except Exception:
            self._lim = None
        return self

    def __exit__(self, *exc):
        if self._lim is not None:
            self._lim.restore_original_limits()


class OracleModel:
    """Holds canonical tensors (numpy) and decodes them to fp64 on demand.

    tensors: tok_embd fp16 [V][H]; attn_norm, ffn_norm fp32 [L][H];
    out_norm fp32 [H]; wq..w_down lists of uint8 canonical bytes per layer;
    lm_head uint8 canonical bytes.  With cache_weights, a tensor decoded
    whole (weight()) is kept; products read their chunks from it.
    """

    def __init__(self, spec, tensors: dict, cache_weights: bool = True, threads: int = None):
        self.spec = spec
        self.t = tensors
        self.cache_weights = cache_weights
        self._w = {}
        self.threads = threads or _threads()

    def _shape(self, name):
        m = self.spec
        q, kv = m.n_head * m.head_dim, m.n_kv_head * m.head_dim
        return {"wq": (q, m.hidden), "wk": (kv, m.hidden), "wv": (kv, m.hidden),
                "wo": (m.hidden, q), "w_gate": (m.ffn, m.hidden),
                "w_up": (m.ffn, m.hidden), "w_down": (m.hidden, m.ffn),
                "lm_head": (m.vocab, m.hidden)}[name]

    def _fmt_raw(self, name, layer):
        fmt = self.spec.fmt_lm if name == "lm_head" else self.spec.fmt_proj
        raw = self.t[name] if name == "lm_head" else self.t[name][layer]
        return fmt, np.asarray(raw)

    def weight(self, name: str, layer: int = 0) -> np.ndarray:
        """The whole decoded tensor [rows][cols] (kept with cache_weights)."""
        key = (name, layer)
        if key in self._w:
            return self._w[key]
        rows, cols = self._shape(name)
        fmt, raw = self._fmt_raw(name, layer)
        w = decode(fmt, raw, rows, cols)
        if self.cache_weights:
            self._w[key] = w
        return w

    def matvec(self, name: str, layer: int, hs: np.ndarray) -> np.ndarray:
        """y[i] = W h_i for every row h_i of hs [n][cols] -> [n][rows]."""
        rows, cols = self._shape(name)
        hs = np.asarray(hs, dtype=np.float64).reshape(-1, cols)
        n = hs.shape[0]
        out = np.empty((n, rows), dtype=np.float64)
        cached = self._w.get((name, layer))
        fmt, raw = self._fmt_raw(name, layer)

        def work(r0):
            r1 = min(rows, r0 + CHUNK_ROWS)
            Wc = cached[r0:r1] if cached is not None else decode(fmt, raw[r0:r1], r1 - r0, cols)
            for b0 in range(0, r1 - r0, SUB_ROWS):
                Wb = Wc[b0:b0 + SUB_ROWS]
                for i in range(n):
                    out[i, r0 + b0:r0 + b0 + Wb.shape[0]] = Wb @ hs[i]

        starts = range(0, rows, CHUNK_ROWS)
        if self.threads <= 1 or rows <= CHUNK_ROWS:
            with _OneBlasThread():
                for r0 in starts:
                    work(r0)
        else:
            with _OneBlasThread(), ThreadPoolExecutor(self.threads) as ex:
                list(ex.map(work, starts))
        return out

    # ---- the forward -----------------------------------------------------
    def forward_rows(self, rows, kc: np.ndarray, vc: np.ndarray, progress=None) -> np.ndarray:
        """Final pre-norm hidden states [n][H] of the rows (s, pos, token);
        writes each row's cache rows at its position, in every layer.

        kc, vc: caches [layer][seq][capacity][n_kv_head][head_dim].  With the
        workloads' fp16 caches the rows' k and v are rounded to fp16 before
        any row reads them.  With fp64 caches they are kept unrounded: that
        variant measures how far the fp16 rounding of in-block rows moves a
        row.  Two rows of one call must not share a (sequence, position).
        progress, if given, is called with (layer, n_layer) after each layer."""
        m = self.spec
        G = m.n_head // m.n_kv_head
        rows = [(int(s), int(p), int(t)) for s, p, t in rows]
        x = np.stack([np.asarray(self.t["tok_embd"][t], dtype=np.float64) for _, _, t in rows])
        for l in range(m.n_layer):
            h = np.stack([rmsnorm(xi, self.t["attn_norm"][l], m.rms_eps) for xi in x])
            q = self.matvec("wq", l, h).reshape(-1, m.n_head, m.head_dim)
            k = self.matvec("wk", l, h).reshape(-1, m.n_kv_head, m.head_dim)
            v = self.matvec("wv", l, h).reshape(-1, m.n_kv_head, m.head_dim)
            for i, (s, pos, _) in enumerate(rows):
                q[i] = rope(q[i], pos, m.rope_base)
                kc[l, s, pos] = rope(k[i], pos, m.rope_base).astype(kc.dtype)
                vc[l, s, pos] = v[i].astype(vc.dtype)
            o = np.empty((len(rows), m.n_head * m.head_dim))
            for i, (s, pos, _) in enumerate(rows):
                Kl = kc[l, s, : pos + 1].astype(np.float64)
                Vl = vc[l, s, : pos + 1].astype(np.float64)
                o[i] = np.stack([attend(q[i, j], Kl[:, j // G], Vl[:, j // G])
                                 for j in range(m.n_head)]).reshape(-1)
            x = x + self.matvec("wo", l, o)
            h2 = np.stack([rmsnorm(xi, self.t["ffn_norm"][l], m.rms_eps) for xi in x])
            a = silu(self.matvec("w_gate", l, h2)) * self.matvec("w_up", l, h2)
            x = x + self.matvec("w_down", l, a)
            if progress is not None:
                progress(l, m.n_layer)
        return x

    def hidden_row(self, tok: int, pos: int, s: int, kc: np.ndarray,
                   vc: np.ndarray) -> np.ndarray:
        """One row alone (plain one-token decoding): forward_rows of one row."""
        return self.forward_rows([(s, pos, tok)], kc, vc)[0]

    def logits_rows(self, hrows: np.ndarray) -> np.ndarray:
        """lm_head over final-normed rows hrows [n][H] -> fp64 [n][V]."""
        return self.matvec("lm_head", 0, hrows)

    def verify_logits(self, ids: np.ndarray, lens: np.ndarray, kc: np.ndarray,
                      vc: np.ndarray) -> np.ndarray:
        """ids [S][nt] -> logits fp64 [S][nt][V]; caches updated in place."""
        m = self.spec
        S, nt = ids.shape
        rows = [(s, int(lens[s]) + r, int(ids[s, r])) for s in range(S) for r in range(nt)]
        x = self.forward_rows(rows, kc, vc)
        fin = np.stack([rmsnorm(xi, self.t["out_norm"], m.rms_eps) for xi in x])
        return self.logits_rows(fin).reshape(S, nt, m.vocab)

    def lm_only_logits(self, hidden: np.ndarray) -> np.ndarray:
        """lm_head-only workload: logits = W_lm h for given hidden rows
        [S][nt][H] (no norm: the hidden states are the lm_head's input)."""
        S, nt, H = hidden.shape
        return self.logits_rows(hidden.reshape(S * nt, H)).reshape(S, nt, -1)
