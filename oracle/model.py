"""fp64 numpy reference of the nanochat GPT forward: batched prefill and KV-cache decode.

TEST INFRASTRUCTURE ONLY (tests, the graft smoke check and the benchmark's CPU-baseline
leg may use it; the product path must not).  It imports nothing from the product.

What is computed, and where the pages say so:
  * dense decoder-only Transformer, Llama-like but simplified
    [yelogs.com launch write-up, section "technical details and official Q&A",
    answer on the model architecture; szyisi.cn launch article, introduction];
  * rotary position embedding, no absolute position embedding [same answer; apidog.com/th
    "How to train your own ChatGPT for $50", section "How nanochat works" part 1 (GPT model),
    architecture features; geoz.com.cn summary, section on development tricks: a concise
    self-written RoPE with precomputed rotary tables];
  * QK-norm on queries and keys [yelogs.com architecture answer; apidog.com part 1];
  * RMSNorm without learnable parameters, after the token embedding and before the MLP
    [yelogs.com architecture answer; szyisi.cn, pretraining section: besides the matrices
    and embeddings the model has no other trainable parameters];
  * untied token embedding and LM head [yelogs.com architecture answer; apidog.com part 1];
  * squared-ReLU MLP activation [yelogs.com architecture answer (formula lost in the
    extracted text); geoz.com.cn development tricks; apidog.com part 1];
  * no bias in any linear layer [yelogs.com architecture answer];
  * multi-query attention, one K/V head shared by every query head [yelogs.com answer];
    grouped-query attention, fewer K/V heads than query heads, in the later version
    [apidog.com part 1, architecture features];
  * sliding-window attention with a configurable per-layer pattern of short and long
    windows ("SSSL"), passed to the attention call as a window size [apidog.com part 1,
    architecture features; part 5, the flash-attention call with window_size];
  * a softcap on the logits [yelogs.com architecture answer];
  * inference with a KV cache: prefill of the prompt, then one token per decode step
    [szyisi.cn, section on the base model and the Engine class; apidog.com part 6,
    inference engine];
  * batch generation: the prompt's cache copied to several rows that are sampled in
    parallel [apidog.com part 6];
  * later-version blocks [apidog.com part 1, architecture features and the three learned
    mechanisms after them]: value embeddings on some layers, added to v through a gate of
    3 sigmoid(...) per K/V head that reads the first channels of the attention input;
    per-layer scaling of the residual stream against the first layer's input x0;
    "smear", a gated copy of the previous token's embedding added to the current one;
    "backout", a multiple of a middle layer's residual stream subtracted at the end.

Readings where the pages are silent (each is listed with its reason in the design notes):
  * norm placement: pre-norm before attention and before the MLP, one norm right after the
    embedding, and a final norm before the LM head;
  * RMSNorm: x / sqrt(mean(x^2) + eps), eps a config value (1e-6), also used for QK-norm;
  * RoPE: rotation of the pair (i, i + hd/2) by angle p * base^(-2i/hd), positions from 0,
    applied before QK-norm (the two commute, since the rotation keeps mean(x^2));
  * attention: scale 1/sqrt(hd), causal including the diagonal, full max-subtracted softmax;
  * MLP: d -> d_ff -> d, activation relu(x)^2, no gate;
  * residual: plain x <- x + f(norm(x));
  * softcap: cap * tanh(z / cap);
  * sliding window w >= 0: a query at position p sees keys p - w .. p (w + 1 keys, the
    left extent of the window_size argument of the pages' flash-attention call; its
    right extent is 0 under causality); w < 0 means the whole causal context;
  * window pattern: character l mod len(pattern) of the pattern gives layer l's window,
    'S' the short window and 'L' the whole context;
  * later-version blocks, where the pages give only their update rules:
      - smear: x_t = e_t + smear_lambda sigmoid(e_t[:C_s] . smear_gate) e_{t-1}, with e the
        normalised token embedding, t the position in the row (position 0: x_0 = e_0);
      - x0 = the stream after smear; layer l starts with
        x <- resid_lambda[l] x + x0_lambda[l] x0;
      - backout: xb = the stream at the start of layer backout_layer (after its scaling),
        and x <- x - backout_lambda xb after the last layer, before the final norm;
      - value embedding of layer l (where given): for K/V head j,
        v_j += 3 sigmoid(h[:C_v] . ve_gate[l][j]) ve[l][token][j hd:(j + 1) hd], with h the
        attention input norm(x);
  * sampling (the pages name parallel sampling but give no formula): keep the logits at
    or above the k-th largest (all with top_k <= 0), take probabilities proportional to
    exp(logit / temperature), and return the smallest token index whose cumulative
    probability exceeds a uniform number u in [0, 1) given by the caller; temperature <= 0
    is the greedy argmax.  NaN logits have probability 0.

Everything is evaluated in float64 with plain numpy operations: no tiling, no online
softmax, no fusion.  Weights may arrive in any float dtype; they are widened to float64
exactly once, when the model object is built.
"""

from __future__ import annotations

import numpy as np

F64 = np.float64


def rms_norm(x, eps):
    """Parameter-free RMSNorm over the last axis: x / sqrt(mean(x^2) + eps)."""
    x = np.asarray(x, dtype=F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps)


def rope_tables(n_pos, head_dim, base):
    """cos/sin of the rotation angles, shape [n_pos, head_dim/2].

    Angle for position p and pair i is p * base^(-2i/head_dim), computed in float64
    (the precomputed rotary table of the geoz.com.cn development-tricks section)."""
    half = head_dim // 2
    i = np.arange(half, dtype=F64)
    inv_freq = np.power(F64(base), -2.0 * i / head_dim)
    ang = np.arange(n_pos, dtype=F64)[:, None] * inv_freq[None, :]
    return np.cos(ang), np.sin(ang)


def rope(x, pos, cos, sin):
    """Rotate the last axis of x by the angles of integer positions `pos`.

    x has shape [..., hd]; pos is an integer array broadcastable against x.shape[:-1].
    The first half of the vector is paired with the second half: (x1, x2) ->
    (x1 cos - x2 sin, x1 sin + x2 cos)."""
    x = np.asarray(x, dtype=F64)
    half = x.shape[-1] // 2
    c = cos[pos]
    s = sin[pos]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def relu2(z):
    """Squared ReLU: max(z, 0)^2."""
    r = np.maximum(np.asarray(z, dtype=F64), 0.0)
    return r * r


def softcap(z, cap):
    """Logit softcap cap * tanh(z / cap)."""
    return cap * np.tanh(np.asarray(z, dtype=F64) / cap)


def linear(x, w):
    """Bias-free linear layer with a weight stored [out, in]: y = x W^T."""
    return np.asarray(x, dtype=F64) @ np.asarray(w, dtype=F64).T


def causal_attention(q, k, v, q_pos, window=-1):
    """Causal softmax attention with shared K/V heads.

    q: [Tq, H, hd]; k, v: [Tk, n_kv, hd] holding key positions 0..Tk-1;
    q_pos: [Tq] absolute position of each query.  Query t sees keys j <= q_pos[t], and
    with window >= 0 only those with j >= q_pos[t] - window.
    Query head h reads K/V head h // (H / n_kv); with n_kv = 1 every query head shares
    the single K/V head (multi-query attention)."""
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    tq, n_head, hd = q.shape
    tk, n_kv, _ = k.shape
    group = n_head // n_kv
    j = np.arange(tk)[None, :]
    qp = np.asarray(q_pos)[:, None]
    hidden = j > qp
    if window >= 0:
        hidden = hidden | (j < qp - window)
    y = np.empty((tq, n_head, hd), dtype=F64)
    for h in range(n_head):
        g = h // group
        s = (q[:, h, :] @ k[:, g, :].T) / np.sqrt(F64(hd))
        s = np.where(hidden, -np.inf, s)
        s = s - np.max(s, axis=1, keepdims=True)
        p = np.exp(s)
        p = p / np.sum(p, axis=1, keepdims=True)
        y[:, h, :] = p @ v[:, g, :]
    return y


def layer_windows(pattern, n_layer, short_window):
    """Per-layer windows from a pattern of 'S' (short window) and 'L' (whole context)
    characters, repeated over the layers: layer l takes character l mod len(pattern)."""
    out = []
    for layer in range(n_layer):
        ch = pattern[layer % len(pattern)]
        if ch == "S":
            out.append(int(short_window))
        elif ch == "L":
            out.append(-1)
        else:
            raise ValueError(f"window pattern character {ch!r} is not S or L")
    return out


def sample(logits, temperature, top_k, u):
    """One token per row of logits [B, V] (see the sampling reading above); u: [B]."""
    logits = np.asarray(logits, dtype=F64)
    out = np.empty(logits.shape[0], dtype=np.int64)
    for b, row in enumerate(logits):
        z = np.where(np.isnan(row), -np.inf, row)
        if temperature <= 0:
            out[b] = int(np.argmax(z))  # first maximum
            continue
        if 0 < top_k < z.shape[0]:
            kth = np.sort(z)[::-1][top_k - 1]
            z = np.where(z >= kth, z, -np.inf)
        m = np.max(z)
        if not np.isfinite(m):
            out[b] = 0
            continue
        p = np.exp((z - m) / temperature)
        cdf = np.cumsum(p) / np.sum(p)
        out[b] = min(int(np.searchsorted(cdf, u[b], side="right")), z.shape[0] - 1)
        while p[out[b]] == 0:  # cdf flat at the end: the last token with mass
            out[b] -= 1
    return out


def param_count(n_layer, d_model, n_head, n_kv_head, head_dim, d_ff, vocab):
    """Number of weights: untied embedding and head, four attention matrices and two MLP
    matrices per layer, no biases and no norm parameters."""
    per_layer = (d_model * n_head * head_dim          # Wq
                 + 2 * d_model * n_kv_head * head_dim  # Wk, Wv
                 + n_head * head_dim * d_model         # Wo
                 + 2 * d_model * d_ff)                 # Wfc, Wproj
    return 2 * vocab * d_model + n_layer * per_layer


_CFG_FIELDS = ("n_layer", "d_model", "n_head", "n_kv_head", "head_dim", "d_ff", "vocab",
               "rope_base", "softcap", "norm_eps")
_LAYER_KEYS = ("wq", "wk", "wv", "wo", "wfc", "wproj")


class OracleModel:
    """The forward pass of one model, holding float64 copies of its weights.

    cfg: any object with the attributes n_layer, d_model, n_head, n_kv_head, head_dim, d_ff,
    vocab, rope_base, softcap, norm_eps.
    weights: {"wte": [V, d], "layers": [{"wq": [H*hd, d], "wk": [n_kv*hd, d],
    "wv": [n_kv*hd, d], "wo": [d, H*hd], "wfc": [d_ff, d], "wproj": [d, d_ff]}, ...],
    "lm_head": [V, d]}.
    windows: per-layer attention windows (see causal_attention), or None for the whole
    causal context in every layer.
    extras: the later-version blocks (see the readings above), a dict with any of
    "resid_lambda", "x0_lambda" (n_layer floats each), "smear_gate" ([C_s]) with
    "smear_lambda", "backout_layer" (-1: none) with "backout_lambda", and "ve", "ve_gate"
    (dicts layer -> [V, n_kv*hd] and [n_kv, C_v]); None or missing keys: the plain model.
    """

    def __init__(self, cfg, weights, windows=None, extras=None):
        for f in _CFG_FIELDS:
            setattr(self, f, getattr(cfg, f))
        assert self.n_head % self.n_kv_head == 0
        self.wte = np.asarray(weights["wte"], dtype=F64)
        self.lm_head = np.asarray(weights["lm_head"], dtype=F64)
        self.layers = [{k: np.asarray(lw[k], dtype=F64) for k in _LAYER_KEYS}
                       for lw in weights["layers"]]
        assert len(self.layers) == self.n_layer
        self.windows = [-1] * self.n_layer if windows is None else [int(w) for w in windows]
        assert len(self.windows) == self.n_layer
        ex = extras or {}
        self.resid_lambda = [float(a) for a in ex.get("resid_lambda", [1.0] * self.n_layer)]
        self.x0_lambda = [float(a) for a in ex.get("x0_lambda", [0.0] * self.n_layer)]
        g = ex.get("smear_gate")
        self.smear_gate = None if g is None else np.asarray(g, dtype=F64)
        self.smear_lambda = float(ex.get("smear_lambda", 0.0))
        self.backout_layer = int(ex.get("backout_layer", -1))
        self.backout_lambda = float(ex.get("backout_lambda", 0.0))
        self.ve = {int(k): np.asarray(v, dtype=F64) for k, v in ex.get("ve", {}).items()}
        self.ve_gate = {int(k): np.asarray(v, dtype=F64) for k, v in ex.get("ve_gate", {}).items()}
        assert set(self.ve) == set(self.ve_gate)
        self._cos = np.zeros((0, self.head_dim // 2))
        self._sin = self._cos

    # -- helpers ---------------------------------------------------------------------
    def _tables(self, n_pos):
        if self._cos.shape[0] < n_pos:
            self._cos, self._sin = rope_tables(max(n_pos, 2 * self._cos.shape[0]),
                                               self.head_dim, self.rope_base)
        return self._cos, self._sin

    def _embed(self, toks, prev):
        """Stream entering layer 0 (before its scaling) for tokens toks [T] of one row;
        prev is the row's token before toks[0], or None at position 0."""
        e = rms_norm(self.wte[toks], self.norm_eps)
        if self.smear_gate is None:
            return e
        c = self.smear_gate.shape[0]
        gate = self.smear_lambda / (1.0 + np.exp(-(e[:, :c] @ self.smear_gate)))
        before = np.zeros_like(e)
        before[1:] = e[:-1]
        if prev is not None:
            before[0] = rms_norm(self.wte[prev], self.norm_eps)
        return e + gate[:, None] * before

    def _qkv(self, lw, x, pos, li=None, toks=None):
        """Pre-attention norm, projections, RoPE and QK-norm for rows x at positions pos
        (layer li's value embedding of tokens toks added to v where the layer has one)."""
        t = x.shape[0]
        h = rms_norm(x, self.norm_eps)
        q = linear(h, lw["wq"]).reshape(t, self.n_head, self.head_dim)
        k = linear(h, lw["wk"]).reshape(t, self.n_kv_head, self.head_dim)
        v = linear(h, lw["wv"]).reshape(t, self.n_kv_head, self.head_dim)
        if li in self.ve:
            c = self.ve_gate[li].shape[1]
            gate = 3.0 / (1.0 + np.exp(-(h[:, :c] @ self.ve_gate[li].T)))  # [t, n_kv]
            v = v + gate[:, :, None] * self.ve[li][toks].reshape(t, self.n_kv_head, self.head_dim)
        cos, sin = self._tables(int(np.max(pos)) + 1)
        q = rms_norm(rope(q, pos[:, None], cos, sin), self.norm_eps)
        k = rms_norm(rope(k, pos[:, None], cos, sin), self.norm_eps)
        return q, k, v

    def _mlp(self, lw, x):
        return linear(relu2(linear(rms_norm(x, self.norm_eps), lw["wfc"])), lw["wproj"])

    def _head(self, x):
        return softcap(linear(rms_norm(x, self.norm_eps), self.lm_head), self.softcap)

    # -- cache -----------------------------------------------------------------------
    def new_cache(self, batch, max_seq):
        shape = (self.n_layer, batch, max_seq, self.n_kv_head, self.head_dim)
        return {"k": np.zeros(shape, dtype=F64), "v": np.zeros(shape, dtype=F64),
                "tok": np.zeros((batch, max_seq), dtype=np.int64),
                "lens": np.zeros(batch, dtype=np.int64), "max_seq": max_seq}

    def _layers(self, x, on_layer):
        """The layers over stream x (from _embed); on_layer(li, lw, x) runs attention and MLP
        of layer li on its (scaled) input and returns the new stream."""
        x0 = x
        xb = None
        for li, lw in enumerate(self.layers):
            x = self.resid_lambda[li] * x + self.x0_lambda[li] * x0
            if li == self.backout_layer:
                xb = x
            x = on_layer(li, lw, x)
        if xb is not None:
            x = x - self.backout_lambda * xb
        return x

    # -- prefill ---------------------------------------------------------------------
    def prefill(self, tokens, max_seq=None, logits_at=None, cache=None):
        """Full-sequence forward of tokens [B, T] at positions 0..T-1.

        Returns (logits, cache).  logits is [B, T, V], or [B, len(logits_at), V] when
        logits_at lists the positions whose logits are wanted (the others are simply not
        evaluated).  The cache holds the post-RoPE, post-norm keys and the values of every
        layer, and lens = T."""
        tokens = np.asarray(tokens)
        b_sz, t_len = tokens.shape
        max_seq = t_len if max_seq is None else max_seq
        if cache is None:
            cache = self.new_cache(b_sz, max_seq)
        assert np.all(cache["lens"] == 0)
        at = np.arange(t_len) if logits_at is None else np.asarray(logits_at)
        logits = np.empty((b_sz, at.shape[0], self.vocab), dtype=F64)
        pos = np.arange(t_len)
        for b in range(b_sz):
            def layer(li, lw, x, b=b):
                q, k, v = self._qkv(lw, x, pos, li, tokens[b])
                cache["k"][li, b, :t_len] = k
                cache["v"][li, b, :t_len] = v
                y = causal_attention(q, k, v, pos, self.windows[li])
                x = x + linear(y.reshape(t_len, -1), lw["wo"])
                return x + self._mlp(lw, x)
            x = self._layers(self._embed(tokens[b], None), layer)
            logits[b] = self._head(x[at])
        cache["tok"][:, :t_len] = tokens
        cache["lens"][:] = t_len
        return logits, cache

    # -- decode ----------------------------------------------------------------------
    def decode_step(self, cache, tokens):
        """One new token per row: row b sits at position lens[b] and attends to cache
        positions 0..lens[b] (its own key included).  Returns logits [B, V]; lens += 1."""
        tokens = np.asarray(tokens).reshape(-1)
        b_sz = tokens.shape[0]
        assert b_sz == cache["lens"].shape[0]
        assert np.all(cache["lens"] < cache["max_seq"])
        logits = np.empty((b_sz, self.vocab), dtype=F64)
        for b in range(b_sz):
            p = int(cache["lens"][b])
            pos = np.array([p])

            def layer(li, lw, x, b=b, p=p, pos=pos):
                q, k, v = self._qkv(lw, x, pos, li, tokens[b:b + 1])
                cache["k"][li, b, p] = k[0]
                cache["v"][li, b, p] = v[0]
                y = causal_attention(q, cache["k"][li, b, :p + 1], cache["v"][li, b, :p + 1],
                                     pos, self.windows[li])
                x = x + linear(y.reshape(1, -1), lw["wo"])
                return x + self._mlp(lw, x)
            prev = int(cache["tok"][b, p - 1]) if p > 0 else None
            x = self._layers(self._embed(tokens[b:b + 1], prev), layer)
            cache["tok"][b, p] = tokens[b]
            logits[b] = self._head(x)[0]
        cache["lens"] += 1
        return logits

    def extend(self, cache, tokens):
        """Append tokens [B, T]: row b takes them at positions lens[b] .. lens[b] + T - 1.
        Returns logits [B, T, V].  By causality this is T decode steps, which is how it is
        computed."""
        tokens = np.asarray(tokens)
        return np.stack([self.decode_step(cache, tokens[:, t]) for t in range(tokens.shape[1])],
                        axis=1)

    @staticmethod
    def copy_rows(dst_cache, dst_rows, src_cache, src_rows):
        """Row dst_rows[i] of dst_cache takes the keys, values and length of row
        src_rows[i] of src_cache (batch generation: one prefilled prompt copied to the rows
        that sample from it)."""
        n = min(dst_cache["max_seq"], src_cache["max_seq"])
        k = src_cache["k"][:, list(src_rows), :n].copy()
        v = src_cache["v"][:, list(src_rows), :n].copy()
        tk = src_cache["tok"][list(src_rows), :n].copy()
        lens = src_cache["lens"][list(src_rows)].copy()
        assert np.all(lens <= dst_cache["max_seq"])
        for i, d in enumerate(dst_rows):
            dst_cache["k"][:, d] = 0.0
            dst_cache["v"][:, d] = 0.0
            dst_cache["k"][:, d, :n] = k[:, i]
            dst_cache["v"][:, d, :n] = v[:, i]
            dst_cache["tok"][d] = 0
            dst_cache["tok"][d, :n] = tk[i]
            dst_cache["lens"][d] = lens[i]

    def truncate(self, cache, lens):
        """Shrink the cached length of each row (keys beyond the new length are dropped)."""
        lens = np.asarray(lens, dtype=np.int64)
        assert np.all(lens <= cache["lens"])
        for b, n in enumerate(lens):
            cache["k"][:, b, n:] = 0.0
            cache["v"][:, b, n:] = 0.0
        cache["lens"][:] = lens

    def greedy(self, prompt, steps, max_seq=None):
        """Greedy continuation of prompt [B, T] for `steps` tokens (ties: lowest index).

        Returns (tokens [B, steps], logits [B, steps, V]) where logits[:, s] are the
        logits that produced tokens[:, s + 1] (so tokens[:, 0] is the argmax of the
        prompt's last position and step s feeds tokens[:, s])."""
        prompt = np.asarray(prompt)
        b_sz, t_len = prompt.shape
        max_seq = t_len + steps if max_seq is None else max_seq
        logits0, cache = self.prefill(prompt, max_seq=max_seq, logits_at=[t_len - 1])
        tok = np.argmax(logits0[:, 0], axis=-1)
        toks = np.empty((b_sz, steps), dtype=np.int64)
        step_logits = np.empty((b_sz, steps, self.vocab), dtype=F64)
        for s in range(steps):
            toks[:, s] = tok
            step_logits[:, s] = self.decode_step(cache, tok)
            tok = np.argmax(step_logits[:, s], axis=-1)
        return toks, step_logits
