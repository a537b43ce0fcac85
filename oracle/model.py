"""Plain NumPy training step of a Llama-style decoder (oracle; test use only).

Every function takes the float dtype of its inputs (float32 for parity,
float64 for the finite-difference pins).  Matrices are stored [out x in],
so a projection is ``y = x @ W.T``.

Citations are to the MegaTrain pages: the chatpaper.ai abstract (parameters
stream in per layer, gradients stream out; the GPU is a transient engine),
radar.chestersoft.de "Methodik" (double-buffered streaming, stateless layer
templates, layer-contiguous store of bf16 weights and gradients with fp32
Adam moments, Adam on the host CPU).  The model itself (RMSNorm, RoPE,
causal attention, SwiGLU, untied head, mean next-token cross-entropy) is
not described on the pages; it is the plain reading of a Llama-style
decoder.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def _per_sequence(fn, n):
    """fn(b) for every sequence b < n.  Sequences are independent (attention
    never looks across them), so they run on threads; each result lands in
    its own slot, so the outcome does not depend on the order."""
    if n == 1:
        fn(0)
        return
    workers = min(n, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1))
    with ThreadPoolExecutor(max(1, workers)) as ex:
        list(ex.map(fn, range(n)))


# ---------------------------------------------------------------- RMSNorm --
def rmsnorm_fwd(x, g, eps):
    """y = x / sqrt(mean(x^2) + eps) * g over the last axis; returns (y, r)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    r = (1.0 / np.sqrt(ms + x.dtype.type(eps))).astype(x.dtype)
    return x * r * g, r


def rmsnorm_bwd(dy, x, g, r):
    """Gradient of rmsnorm_fwd: returns (dx, dg).

    With xh = x * r:  dg = sum_rows dy*xh,
    dx = r * (dy*g - xh * mean(dy*g*xh)).
    """
    xh = x * r
    dyg = dy * g
    dg = np.sum((dy * xh).reshape(-1, x.shape[-1]), axis=0)
    dx = r * (dyg - xh * np.mean(dyg * xh, axis=-1, keepdims=True))
    return dx, dg


# ------------------------------------------------------------------- RoPE --
def rope_tables(T, hd, theta, dtype=np.float32):
    """cos/sin of t * theta^(-2i/hd) for t < T, i < hd/2 (float64, then cast)."""
    i = np.arange(hd // 2, dtype=np.float64)
    w = theta ** (-2.0 * i / hd)
    ang = np.arange(T, dtype=np.float64)[:, None] * w[None, :]
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rope_apply(x, cos, sin, inverse=False):
    """Rotate pairs (x_i, x_{i+hd/2}) by +t*w_i (or -t*w_i when inverse).

    x: [..., T, hd] with the position on axis -2.
    """
    h = x.shape[-1] // 2
    a, b = x[..., :h], x[..., h:]
    s = -sin if inverse else sin
    return np.concatenate([a * cos - b * s, a * s + b * cos], axis=-1)


# -------------------------------------------------------------- attention --
def attention_fwd(q, k, v):
    """Causal softmax attention per head.  q, k, v: [H, T, hd] -> (o, p)."""
    T, hd = q.shape[-2], q.shape[-1]
    scale = q.dtype.type(1.0 / np.sqrt(hd))
    s = (q @ np.swapaxes(k, -1, -2)) * scale
    future = np.triu(np.ones((T, T), dtype=bool), k=1)
    s = np.where(future, -np.inf, s)
    s = s - np.max(s, axis=-1, keepdims=True)
    e = np.exp(s)
    p = e / np.sum(e, axis=-1, keepdims=True)
    return p @ v, p


def attention_bwd(do, q, k, v, p):
    """Gradient of attention_fwd given its probabilities p: (dq, dk, dv)."""
    hd = q.shape[-1]
    scale = q.dtype.type(1.0 / np.sqrt(hd))
    dv = np.swapaxes(p, -1, -2) @ do
    dp = do @ np.swapaxes(v, -1, -2)
    ds = p * (dp - np.sum(dp * p, axis=-1, keepdims=True))
    dq = (ds @ k) * scale
    dk = (np.swapaxes(ds, -1, -2) @ q) * scale
    return dq, dk, dv


def attention_rows(q, k, v, do, rows):
    """Rows of attention_fwd / attention_bwd for one head, one query at a time.

    q, k, v, do: [T, hd]; returns (o, dq) for the query rows ``rows``.  Query
    i sees keys 0..i only, so its output and its query gradient need nothing
    but its own score row; this evaluates single rows of sequences too long
    for the T x T matrices.
    """
    hd = q.shape[-1]
    scale = q.dtype.type(1.0 / np.sqrt(hd))
    o = np.empty((len(rows), hd), q.dtype)
    dq = np.empty((len(rows), hd), q.dtype)
    for n, i in enumerate(rows):
        s = (k[:i + 1] @ q[i]) * scale
        e = np.exp(s - np.max(s))
        p = e / np.sum(e)
        o[n] = p @ v[:i + 1]
        dp = v[:i + 1] @ do[i]
        ds = p * (dp - np.sum(dp * p))
        dq[n] = (ds @ k[:i + 1]) * scale
    return o, dq


def attention_key_tail(q, k, v, do, n):
    """dk, dv of the last n keys of one head ([T, hd] operands).

    Key j is seen only by queries i >= j, so the last n keys take gradient
    from the last n queries alone: their full score rows (n x T) suffice.
    """
    T, hd = q.shape
    scale = q.dtype.type(1.0 / np.sqrt(hd))
    qi = np.arange(T - n, T)
    s = (q[T - n:] @ k.T) * scale
    s = np.where(np.arange(T)[None, :] > qi[:, None], -np.inf, s)
    s = s - np.max(s, axis=-1, keepdims=True)
    e = np.exp(s)
    p = e / np.sum(e, axis=-1, keepdims=True)
    dp = do[T - n:] @ v.T
    ds = p * (dp - np.sum(dp * p, axis=-1, keepdims=True))
    dv = p[:, T - n:].T @ do[T - n:]
    dk = (ds[:, T - n:].T @ q[T - n:]) * scale
    return dk, dv


# ----------------------------------------------------------------- SwiGLU --
def silu(z):
    return z / (1 + np.exp(-z))


def silu_grad(z):
    s = 1 / (1 + np.exp(-z))
    return s * (1 + z * (1 - s))


# ---------------------------------------------------------- cross-entropy --
def cross_entropy(logits, tokens):
    """Mean next-token loss over the B*(T-1) labelled positions.

    logits: [B, T, V]; the label of (b, t) is tokens[b, t+1]; position T-1
    has no label.  Returns (loss, dlogits) with dlogits = (softmax - onehot)/N
    on labelled rows and 0 on the last position of each sequence.
    """
    B, T, V = logits.shape
    n = B * (T - 1)
    z = logits[:, :-1, :]
    m = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - m)
    se = np.sum(e, axis=-1, keepdims=True)
    lse = (m + np.log(se))[..., 0]
    lab = tokens[:, 1:]
    picked = np.take_along_axis(z, lab[..., None], axis=-1)[..., 0]
    loss = np.sum(lse - picked) / n
    d = e / se
    bi, ti = np.meshgrid(np.arange(B), np.arange(T - 1), indexing="ij")
    d[bi, ti, lab] -= 1
    dl = np.zeros_like(logits)
    dl[:, :-1, :] = d / logits.dtype.type(n)
    return logits.dtype.type(loss), dl


# ------------------------------------------------------------------- Adam --
def adam_update(w, g, m, v, t, lr, b1, b2, eps):
    """One bias-corrected Adam step (no weight decay, no clipping).

    Returns (w', m', v').  The pages put fp32 Adam moments in the host store
    (radar.chestersoft.de, "Methodik", layer-contiguous tiling).
    """
    dt = w.dtype.type
    m2 = dt(b1) * m + dt(1 - b1) * g
    v2 = dt(b2) * v + dt(1 - b2) * g * g
    mh = m2 / dt(1 - b1 ** t)
    vh = v2 / dt(1 - b2 ** t)
    return w - dt(lr) * mh / (np.sqrt(vh) + dt(eps)), m2, v2


# ------------------------------------------------------------------ model --
class Oracle:
    """One training step of the decoder described by a datagen.ModelShape."""

    def __init__(self, cfg, dtype=np.float32):
        self.cfg = cfg
        self.dt = np.dtype(dtype)
        self.cos, self.sin = rope_tables(cfg.seq_len, cfg.head_dim, cfg.rope_theta, self.dt)

    # ----------------------------------------------------------- pieces --
    def _heads(self, x):
        c = self.cfg
        return x.reshape(c.batch, c.seq_len, c.n_heads, c.head_dim).transpose(0, 2, 1, 3)

    def _merge(self, x):
        c = self.cfg
        return x.transpose(0, 2, 1, 3).reshape(c.batch * c.seq_len, c.d_model)

    def layer_fwd(self, x, P, l):
        """One decoder layer on x [M, d]; returns (x_next, cache)."""
        c = self.cfg
        a, f = P[f"{l}.attn_norm"], P[f"{l}.ffn_norm"]
        h, r1 = rmsnorm_fwd(x, a, c.rms_eps)
        q = self._heads(h @ P[f"{l}.wq"].T)
        k = self._heads(h @ P[f"{l}.wk"].T)
        v = self._heads(h @ P[f"{l}.wv"].T)
        qr = rope_apply(q, self.cos, self.sin)
        kr = rope_apply(k, self.cos, self.sin)
        o = np.empty_like(qr)
        probs = [None] * c.batch

        def attend(b):
            o[b], probs[b] = attention_fwd(qr[b], kr[b], v[b])

        _per_sequence(attend, c.batch)
        om = self._merge(o)
        x1 = x + om @ P[f"{l}.wo"].T
        h2, r2 = rmsnorm_fwd(x1, f, c.rms_eps)
        gt = h2 @ P[f"{l}.wg"].T
        u = h2 @ P[f"{l}.wu"].T
        y = silu(gt) * u
        x2 = x1 + y @ P[f"{l}.wd"].T
        cache = dict(x=x, h=h, r1=r1, qr=qr, kr=kr, v=v, probs=probs, om=om,
                     x1=x1, h2=h2, r2=r2, gt=gt, u=u, y=y)
        return x2, cache

    def layer_bwd(self, dx2, cache, P, l, grads):
        """Backward of layer_fwd; accumulates parameter grads; returns dx."""
        c = self.cfg
        C = cache
        a, f = P[f"{l}.attn_norm"], P[f"{l}.ffn_norm"]
        # down projection and SwiGLU
        grads[f"{l}.wd"] = dx2.T @ C["y"]
        dy = dx2 @ P[f"{l}.wd"]
        dgt = dy * C["u"] * silu_grad(C["gt"])
        du = dy * silu(C["gt"])
        grads[f"{l}.wg"] = dgt.T @ C["h2"]
        grads[f"{l}.wu"] = du.T @ C["h2"]
        dh2 = dgt @ P[f"{l}.wg"] + du @ P[f"{l}.wu"]
        dxa, grads[f"{l}.ffn_norm"] = rmsnorm_bwd(dh2, C["x1"], f, C["r2"])
        dx1 = dx2 + dxa
        # attention output projection
        grads[f"{l}.wo"] = dx1.T @ C["om"]
        dom = self._heads(dx1 @ P[f"{l}.wo"])
        dq = np.empty_like(dom)
        dk = np.empty_like(dom)
        dv = np.empty_like(dom)
        def attend_bwd(b):
            dq[b], dk[b], dv[b] = attention_bwd(dom[b], C["qr"][b], C["kr"][b], C["v"][b], C["probs"][b])

        _per_sequence(attend_bwd, c.batch)
        dq = self._merge(rope_apply(dq, self.cos, self.sin, inverse=True))
        dk = self._merge(rope_apply(dk, self.cos, self.sin, inverse=True))
        dv = self._merge(dv)
        grads[f"{l}.wq"] = dq.T @ C["h"]
        grads[f"{l}.wk"] = dk.T @ C["h"]
        grads[f"{l}.wv"] = dv.T @ C["h"]
        dh = dq @ P[f"{l}.wq"] + dk @ P[f"{l}.wk"] + dv @ P[f"{l}.wv"]
        dxb, grads[f"{l}.attn_norm"] = rmsnorm_bwd(dh, C["x"], a, C["r1"])
        return dx1 + dxb

    def head(self, xL, P, tokens):
        """Final norm, untied output head and loss; returns (loss, dxL, grads)."""
        c = self.cfg
        z, r = rmsnorm_fwd(xL, P["final_norm"], c.rms_eps)
        logits = (z @ P["wh"].T).reshape(c.batch, c.seq_len, c.vocab)
        loss, dl = cross_entropy(logits, tokens)
        dl = dl.reshape(-1, c.vocab)
        g = {"wh": dl.T @ z}
        dz = dl @ P["wh"]
        dxL, g["final_norm"] = rmsnorm_bwd(dz, xL, P["final_norm"], r)
        return loss, dxL, g, logits

    # ------------------------------------------------------------- step --
    def forward_backward(self, P, tokens, mode="streamed", keep=None, bwd_layers=None):
        """Loss and gradients of every logical parameter.

        mode 'resident' keeps every layer's intermediates from the forward;
        mode 'streamed' keeps only the layer-boundary checkpoints x^l and
        recomputes each layer's forward inside the backward sweep.
        ``keep`` (optional dict) receives the checkpoints and logits.
        ``bwd_layers`` (optional) stops the backward sweep after that many
        layers from the top: the head's gradients and those layers' are
        returned, the lower layers' and the embedding's are not computed.
        """
        c = self.cfg
        P = {k: np.asarray(v, dtype=self.dt) for k, v in P.items()}
        tok = np.asarray(tokens).reshape(c.batch, c.seq_len)
        x = P["E"][tok.reshape(-1)]
        ckpt = [x]
        caches = []
        for l in range(c.n_layers):
            x, cache = self.layer_fwd(x, P, l)
            ckpt.append(x)
            caches.append(cache if mode == "resident" else None)
        loss, dx, grads, logits = self.head(x, P, tok)
        stop = -1 if bwd_layers is None else max(-1, c.n_layers - 1 - bwd_layers)
        for l in range(c.n_layers - 1, stop, -1):
            cache = caches[l]
            if cache is None:
                _, cache = self.layer_fwd(ckpt[l], P, l)
            dx = self.layer_bwd(dx, cache, P, l, grads)
            caches[l] = None
        if stop == -1:
            dE = np.zeros_like(P["E"])
            np.add.at(dE, tok.reshape(-1), dx)
            grads["E"] = dE
        if keep is not None:
            keep["ckpt"] = ckpt
            keep["logits"] = logits
        return loss, grads

    def loss_only(self, P, tokens):
        c = self.cfg
        P = {k: np.asarray(v, dtype=self.dt) for k, v in P.items()}
        tok = np.asarray(tokens).reshape(c.batch, c.seq_len)
        x = P["E"][tok.reshape(-1)]
        for l in range(c.n_layers):
            x, _ = self.layer_fwd(x, P, l)
        z, _ = rmsnorm_fwd(x, P["final_norm"], c.rms_eps)
        logits = (z @ P["wh"].T).reshape(c.batch, c.seq_len, c.vocab)
        return cross_entropy(logits, tok)[0]

    def step(self, P, tokens, mode="streamed", t=1, moments=None):
        """Forward, backward and one Adam step over every parameter.

        Returns (loss, grads, new_params, new_moments); moments default to 0.
        """
        c = self.cfg
        loss, grads = self.forward_backward(P, tokens, mode)
        newP, newM = {}, {}
        for k, w in P.items():
            w = np.asarray(w, dtype=self.dt)
            if moments is None:
                m0 = np.zeros_like(w)
                v0 = np.zeros_like(w)
            else:
                m0, v0 = moments[k]
            newP[k], m1, v1 = adam_update(w, grads[k], m0, v0, t, c.lr, c.beta1, c.beta2, c.adam_eps)
            newM[k] = (m1, v1)
        return loss, grads, newP, newM
