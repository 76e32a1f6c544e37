"""fp64 forward of the target model's verify rows, one row at a time.

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

Row r of a verify round sits at position len + r.  Rows are processed in
order, each through all layers, exactly as plain autoregressive decoding with
the drafted ids teacher-forced: this is the "one target pass over the anchor
and the proposal block" of the Power page's exactness transaction, evaluated
the slow way.  The new K/V rows are written into the fp16 cache before any
later row reads them, so in-block rows see fp16-rounded keys and values, the
same values a one-row decode would read back.
"""

import numpy as np

from .formats import decode


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


class OracleModel:
    """Holds canonical tensors (numpy) and decodes them to fp64 on demand.

    tensors: tok_embd fp16 [V][H]; attn_norm, ffn_norm fp32 [L][H];
    out_norm fp32 [H]; wq..w_down lists of uint8 canonical bytes per layer;
    lm_head uint8 canonical bytes.
    """

    def __init__(self, spec, tensors: dict, cache_weights: bool = True):
        self.spec = spec
        self.t = tensors
        self.cache_weights = cache_weights
        self._w = {}

    def _shape(self, name):
        m = self.spec
        q, kv = m.n_head * m.head_dim, m.n_kv_head * m.head_dim
        return {"wq": (q, m.hidden), "wk": (kv, m.hidden), "wv": (kv, m.hidden),
                "wo": (m.hidden, q), "w_gate": (m.ffn, m.hidden),
                "w_up": (m.ffn, m.hidden), "w_down": (m.hidden, m.ffn),
                "lm_head": (m.vocab, m.hidden)}[name]

    def weight(self, name: str, layer: int = 0) -> np.ndarray:
        key = (name, layer)
        if key in self._w:
            return self._w[key]
        rows, cols = self._shape(name)
        fmt = self.spec.fmt_lm if name == "lm_head" else self.spec.fmt_proj
        raw = self.t[name] if name == "lm_head" else self.t[name][layer]
        w = decode(fmt, np.asarray(raw), rows, cols)
        if self.cache_weights:
            self._w[key] = w
        return w

    # ---- the row forward -------------------------------------------------
    def hidden_row(self, tok: int, pos: int, s: int, kc: np.ndarray,
                   vc: np.ndarray) -> np.ndarray:
        """Final pre-norm hidden state of one row; writes cache rows at pos.

        kc, vc: caches [layer][seq][capacity][n_kv_head][head_dim].  With the
        workloads' fp16 caches the row's k and v are rounded to fp16 before
        any row reads them (in-block rows read the cache as nt = 1 decoding
        would).  With fp64 caches they are kept unrounded: that variant
        measures how far the fp16 rounding of in-block rows moves a row."""
        m = self.spec
        G = m.n_head // m.n_kv_head
        x = np.asarray(self.t["tok_embd"][tok], dtype=np.float64)
        for l in range(m.n_layer):
            h = rmsnorm(x, self.t["attn_norm"][l], m.rms_eps)
            q = (self.weight("wq", l) @ h).reshape(m.n_head, m.head_dim)
            k = (self.weight("wk", l) @ h).reshape(m.n_kv_head, m.head_dim)
            v = (self.weight("wv", l) @ h).reshape(m.n_kv_head, m.head_dim)
            q = rope(q, pos, m.rope_base)
            k = rope(k, pos, m.rope_base)
            kc[l, s, pos] = k.astype(kc.dtype)
            vc[l, s, pos] = v.astype(vc.dtype)
            Kl = kc[l, s, : pos + 1].astype(np.float64)
            Vl = vc[l, s, : pos + 1].astype(np.float64)
            o = np.stack([attend(q[j], Kl[:, j // G], Vl[:, j // G])
                          for j in range(m.n_head)])
            x = x + self.weight("wo", l) @ o.reshape(-1)
            h2 = rmsnorm(x, self.t["ffn_norm"][l], m.rms_eps)
            a = silu(self.weight("w_gate", l) @ h2) * (self.weight("w_up", l) @ h2)
            x = x + self.weight("w_down", l) @ a
        return x

    def logits_rows(self, hrows: np.ndarray, chunk: int = 16384) -> np.ndarray:
        """lm_head over final-normed rows hrows [n][H] -> fp64 [n][V].

        Up to 16 rows are multiplied one at a time (so a row's bits never
        depend on how many rows share the call); more rows use one matrix
        product per chunk of vocabulary rows."""
        m = self.spec
        hrows = np.asarray(hrows, dtype=np.float64)
        n = hrows.shape[0]
        out = np.empty((n, m.vocab), dtype=np.float64)
        raw = np.asarray(self.t["lm_head"])
        cached = self._w.get(("lm_head", 0))
        for r0 in range(0, m.vocab, chunk):
            r1 = min(m.vocab, r0 + chunk)
            Wc = cached[r0:r1] if cached is not None else decode(
                m.fmt_lm, raw[r0:r1], r1 - r0, m.hidden)
            if n <= 16:
                for i in range(n):
                    out[i, r0:r1] = Wc @ hrows[i]
            else:
                out[:, r0:r1] = (Wc @ hrows.T).T
        return out

    def verify_logits(self, ids: np.ndarray, lens: np.ndarray, kc: np.ndarray,
                      vc: np.ndarray) -> np.ndarray:
        """ids [S][nt] -> logits fp64 [S][nt][V]; caches updated in place."""
        m = self.spec
        S, nt = ids.shape
        fin = np.empty((S, nt, m.hidden), dtype=np.float64)
        for s in range(S):
            for r in range(nt):
                x = self.hidden_row(int(ids[s, r]), int(lens[s]) + r, s, kc, vc)
                fin[s, r] = rmsnorm(x, self.t["out_norm"], m.rms_eps)
        return self.logits_rows(fin.reshape(S * nt, m.hidden)).reshape(S, nt, m.vocab)

    def lm_only_logits(self, hidden: np.ndarray) -> np.ndarray:
        """lm_head-only workload: logits = W_lm h for given hidden rows
        [S][nt][H] (no norm: the hidden states are the lm_head's input)."""
        S, nt, H = hidden.shape
        return self.logits_rows(hidden.reshape(S * nt, H)).reshape(S, nt, -1)
