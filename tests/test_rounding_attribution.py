"""Where a layer's error against the oracle comes from (CPU).

The device path rounds to bf16 at about sixteen points per layer: the
operands of every GEMM (normalised activations h and h2, the attention
output o, the SwiGLU output y, the incoming gradient dx and the
intermediate gradients dy, dgu, do), the stored q, k, v (once after the
projection, once after the rotation), the attention probabilities P and
score gradients dS fed to the matrix cores, and the attention backward's
dq, dk, dv.  This test evaluates one decoder layer in float64 with the
oracle's functions, rounding at one of those points at a time, and
measures the error each leaves in the layer's forward increment and in its
gradients.

Finding (also at the 1.3B width): no point dominates.  Each contributes a
comparable share and the shares add up, so a layer's error is the sum of
many independent bf16 roundings; over many layers it grows like a random
walk.  That is why the whole 1.3B step, compared end to end, grazes the
max-norm bar on some tensors while every block on its own meets the bars
with a wide margin.
"""
import numpy as np
import pytest

import datagen
from oracle import rmsnorm_bwd, rmsnorm_fwd, rope_apply, rope_tables, silu, silu_grad

SHAPE = datagen.ModelShape("attrib", 1, 512, 4, 128, 1408, 1000, 1, 256)
FWD_POINTS = ("h", "qkv", "rope", "p", "o", "h2", "gu", "y")
BWD_POINTS = ("dxb", "dy", "dgu", "do", "p_bwd", "ds", "dqkv", "rope_bwd")


def _rb(x):
    """Round to bf16 (nearest even) and back, as the device stores a value."""
    return datagen.bf16_bits_to_f32(datagen.f32_to_bf16_bits(np.asarray(x, np.float32))).astype(np.float64)


class Layer:
    def __init__(self, s):
        self.s = s
        self.P = {nm: datagen.init_tensor(s, nm, 0).astype(np.float64) for nm in datagen.LAYER_TENSORS}
        self.cos, self.sin = rope_tables(s.seq_len, s.head_dim, s.rope_theta, np.float64)
        self.g = np.ones(s.d_model)
        T = s.seq_len
        self.future = np.triu(np.ones((T, T), bool), 1)

    def heads(self, x):
        s = self.s
        return x.reshape(s.seq_len, s.n_heads, s.head_dim).transpose(1, 0, 2)

    def merge(self, x):
        return x.transpose(1, 0, 2).reshape(self.s.seq_len, self.s.d_model)

    def _attn_probs(self, qr, kr):
        sc = qr @ kr.transpose(0, 2, 1) / np.sqrt(self.s.head_dim)
        sc = np.where(self.future, -np.inf, sc)
        e = np.exp(sc - sc.max(-1, keepdims=True))
        return e, e.sum(-1, keepdims=True)

    def forward(self, x, R=()):
        r = (lambda k, v: _rb(v) if k in R else v)
        P, eps = self.P, self.s.rms_eps
        h = r("h", rmsnorm_fwd(x, self.g, eps)[0])
        q, k, v = (r("qkv", h @ P[n].T) for n in ("wq", "wk", "wv"))
        qr = r("rope", rope_apply(self.heads(q), self.cos, self.sin))
        kr = r("rope", rope_apply(self.heads(k), self.cos, self.sin))
        e, l = self._attn_probs(qr, kr)
        # the device multiplies unnormalised probabilities and divides by l
        o = r("o", self.merge((r("p", e) @ self.heads(v)) / l))
        x1 = x + o @ P["wo"].T
        h2 = r("h2", rmsnorm_fwd(x1, self.g, eps)[0])
        gt, u = r("gu", h2 @ P["wg"].T), r("gu", h2 @ P["wu"].T)
        y = r("y", silu(gt) * u)
        return x1 + y @ P["wd"].T

    def backward(self, x, dx2, R=()):
        """Gradients of every weight and gain and dl/dx, forward exact."""
        r = (lambda k, v: _rb(v) if k in R else v)
        P, eps, hd = self.P, self.s.rms_eps, self.s.head_dim
        h, r1 = rmsnorm_fwd(x, self.g, eps)
        q, k, v = (h @ P[n].T for n in ("wq", "wk", "wv"))
        qr, kr, vh = rope_apply(self.heads(q), self.cos, self.sin), rope_apply(self.heads(k), self.cos, self.sin), \
            self.heads(v)
        e, l = self._attn_probs(qr, kr)
        p = e / l
        o = self.merge(p @ vh)
        x1 = x + o @ P["wo"].T
        h2, r2 = rmsnorm_fwd(x1, self.g, eps)
        gt, u = h2 @ P["wg"].T, h2 @ P["wu"].T
        y = silu(gt) * u
        G = {}
        d2 = r("dxb", dx2)
        G["wd"] = d2.T @ y
        dy = r("dy", d2 @ P["wd"])
        dg, du = r("dgu", dy * u * silu_grad(gt)), r("dgu", dy * silu(gt))
        G["wg"], G["wu"] = dg.T @ h2, du.T @ h2
        dxa, G["ffn_norm"] = rmsnorm_bwd(dg @ P["wg"] + du @ P["wu"], x1, self.g, r2)
        dx1 = dx2 + dxa
        d1 = r("dxb", dx1)
        G["wo"] = d1.T @ o
        do = self.heads(r("do", d1 @ P["wo"]))
        dv = r("p_bwd", p).transpose(0, 2, 1) @ do
        dp = do @ vh.transpose(0, 2, 1)
        ds = r("ds", p * (dp - (dp * p).sum(-1, keepdims=True)))
        dq = r("dqkv", ds @ kr / np.sqrt(hd))
        dk = r("dqkv", ds.transpose(0, 2, 1) @ qr / np.sqrt(hd))
        dv = self.merge(r("dqkv", dv))
        dq = self.merge(r("rope_bwd", rope_apply(dq, self.cos, self.sin, inverse=True)))
        dk = self.merge(r("rope_bwd", rope_apply(dk, self.cos, self.sin, inverse=True)))
        G["wq"], G["wk"], G["wv"] = dq.T @ h, dk.T @ h, dv.T @ h
        dxb, G["attn_norm"] = rmsnorm_bwd(dq @ P["wq"] + dk @ P["wk"] + dv @ P["wv"], x, self.g, r1)
        G["dx"] = dx1 + dxb
        return G


def _one_minus_cos(a, b):
    a, b = a.ravel(), b.ravel()
    return 1.0 - float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


@pytest.fixture(scope="module")
def layer_and_inputs():
    s = SHAPE
    lay = Layer(s)
    tok = datagen.tokens(s)[0]
    x = datagen.init_tensor(s, "E").astype(np.float64)[tok]       # layer 0's input: embedding rows
    dx2 = np.random.default_rng(1).standard_normal((s.seq_len, s.d_model)) * 1e-4
    return lay, x, dx2


def test_forward_rounding_points_share_the_error(layer_and_inputs):
    lay, x, _ = layer_and_inputs
    ref = lay.forward(x) - x
    each = {p: _one_minus_cos(lay.forward(x, {p}) - x, ref) for p in FWD_POINTS}
    total = _one_minus_cos(lay.forward(x, set(FWD_POINTS)) - x, ref)
    for p, v in each.items():
        print(f"  forward increment, bf16 at {p:5s}: 1-cos {v:.2e} ({v / total:5.1%} of all points together)")
    print(f"  all {len(FWD_POINTS)} points: 1-cos {total:.2e}; sum of single points {sum(each.values()):.2e}")
    assert all(v <= 0.35 * total for v in each.values()), each
    assert 0.6 * total <= sum(each.values()) <= 1.6 * total


def test_backward_rounding_points_share_the_error(layer_and_inputs):
    lay, x, dx2 = layer_and_inputs
    G0 = lay.backward(x, dx2)

    def err(R):
        G = lay.backward(x, dx2, R)
        return float(np.mean([_one_minus_cos(G[k], G0[k]) for k in G0]))

    each = {p: err({p}) for p in BWD_POINTS}
    total = err(set(BWD_POINTS))
    for p, v in each.items():
        print(f"  gradients (mean over tensors), bf16 at {p:8s}: 1-cos {v:.2e} ({v / total:5.1%})")
    print(f"  all {len(BWD_POINTS)} points: 1-cos {total:.2e}; sum of single points {sum(each.values()):.2e}")
    assert all(v <= 0.35 * total for v in each.values()), each
    assert 0.6 * total <= sum(each.values()) <= 1.6 * total
