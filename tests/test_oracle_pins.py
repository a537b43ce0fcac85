"""Pins of the oracle against mathematics it does not itself use.

Each test fixes one part of the oracle to something outside it: finite
differences, closed forms, brute-force loops on tiny inputs, invariants.
"""
import math

import numpy as np
import pytest

import datagen
from oracle import (Oracle, adam_update, attention_bwd, attention_fwd, attention_key_tail, attention_rows,
                    cross_entropy,
                    rmsnorm_bwd, rmsnorm_fwd, rope_apply, rope_tables, silu, silu_grad)

TINY = datagen.PRESETS["tiny"]


@pytest.fixture(scope="module")
def tiny64():
    P = datagen.init_params(TINY)
    tok = datagen.tokens(TINY)
    o = Oracle(TINY, np.float64)
    loss, g = o.forward_backward(P, tok, mode="streamed")
    return P, tok, o, loss, g


# ------------------------------------------------- finite differences --
def test_fd_every_tensor(tiny64):
    """Central differences (h = 1e-5, float64) on 32 coordinates per tensor."""
    P, tok, o, loss, g = tiny64
    rng = np.random.default_rng(123)
    h = 1e-5
    present = np.unique(tok)
    for name, w in P.items():
        w = w.astype(np.float64)
        gi = g[name]
        worst = 0.0
        for _ in range(32):
            if name == "E":
                idx = (int(rng.choice(present)), int(rng.integers(w.shape[1])))
            else:
                idx = tuple(int(rng.integers(s)) for s in w.shape)
            Q = dict(P)
            wp = w.copy()
            wp[idx] += h
            Q[name] = wp
            lp = o.loss_only(Q, tok)
            wp[idx] -= 2 * h
            lm = o.loss_only(Q, tok)
            fd = (lp - lm) / (2 * h)
            worst = max(worst, abs(fd - gi[idx]))
        assert worst <= 1e-6 * np.abs(gi).max(), (name, worst, np.abs(gi).max())


def test_fd_directional(tiny64):
    """One random direction over the full parameter vector."""
    P, tok, o, loss, g = tiny64
    rng = np.random.default_rng(7)
    dirs = {k: rng.standard_normal(v.shape) for k, v in P.items()}
    nrm = math.sqrt(sum(float(np.sum(d * d)) for d in dirs.values()))
    dirs = {k: d / nrm for k, d in dirs.items()}
    h = 1e-5
    lp = o.loss_only({k: P[k] + h * dirs[k] for k in P}, tok)
    lm = o.loss_only({k: P[k] - h * dirs[k] for k in P}, tok)
    fd = (lp - lm) / (2 * h)
    an = sum(float(np.sum(g[k] * dirs[k])) for k in P)
    assert abs(fd - an) <= 1e-6 * abs(an)


def test_embedding_grad_zero_for_absent_tokens(tiny64):
    P, tok, o, loss, g = tiny64
    absent = np.setdiff1d(np.arange(TINY.vocab), np.unique(tok))
    assert absent.size > 0
    assert np.all(g["E"][absent] == 0)


# ---------------------------------------------------------------- modes --
def test_streamed_equals_resident_bitwise():
    P = datagen.init_params(TINY)
    tok = datagen.tokens(TINY)
    o = Oracle(TINY, np.float32)
    l1, g1 = o.forward_backward(P, tok, mode="streamed")
    l2, g2 = o.forward_backward(P, tok, mode="resident")
    assert l1 == l2
    for k in g1:
        assert np.array_equal(g1[k], g2[k]), k


# ----------------------------------------------------------------- Adam --
def test_adam_closed_form_first_step():
    """At t = 1 with zero moments, m_hat = g and v_hat = g^2, so the step is
    -lr * g / (|g| + eps) exactly (up to rounding)."""
    rng = np.random.default_rng(0)
    g = rng.standard_normal(10000) * 10.0 ** rng.uniform(-10, 0, 10000)
    w = rng.standard_normal(10000)
    z = np.zeros_like(w)
    w1, m1, v1 = adam_update(w, g, z, z, 1, 1e-3, 0.9, 0.95, 1e-8)
    expect = w - 1e-3 * g / (np.abs(g) + 1e-8)
    np.testing.assert_allclose(w1, expect, rtol=0, atol=1e-15)
    np.testing.assert_allclose(m1, 0.1 * g, rtol=1e-15)
    np.testing.assert_allclose(v1, 0.05 * g * g, rtol=1e-12)
    # worked value: g = 3e-9 -> step = -1e-3 * 3/13 = -2.3077e-4
    w1, _, _ = adam_update(np.zeros(1), np.array([3e-9]), np.zeros(1), np.zeros(1), 1, 1e-3, 0.9, 0.95, 1e-8)
    assert abs(w1[0] + 1e-3 * 3 / 13) < 1e-15


def test_adam_constant_gradient_steady_step():
    """With a constant g the bias-corrected moments are exactly g and g^2 at
    every t, so each step moves w by the same -lr*g/(|g|+eps)."""
    g = np.array([0.5, -2.0, 1e-4, 0.0])
    w = np.zeros(4)
    m = np.zeros(4)
    v = np.zeros(4)
    steps = []
    for t in range(1, 6):
        w2, m, v = adam_update(w, g, m, v, t, 1e-3, 0.9, 0.95, 1e-8)
        steps.append(w2 - w)
        w = w2
    expect = -1e-3 * g / (np.abs(g) + 1e-8)
    for s in steps:
        np.testing.assert_allclose(s, expect, rtol=1e-12, atol=1e-18)
    assert steps[0][3] == 0.0


def test_adam_golden_values():
    """Values in tests/golden/adam_t1.txt are derived by hand from the
    closed form -lr*g/(|g|+eps) (see the file header)."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "adam_t1.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    for g_s, dw_s in rows:
        w1, _, _ = adam_update(np.zeros(1), np.array([float(g_s)]), np.zeros(1), np.zeros(1),
                               1, 1e-3, 0.9, 0.95, 1e-8)
        assert abs(w1[0] - float(dw_s)) <= 1e-9 * 1e-3, (g_s, w1[0], dw_s)


# ------------------------------------------------------------ attention --
def _attention_loops(q, k, v):
    H, T, hd = q.shape
    o = np.zeros_like(q)
    for h in range(H):
        for t in range(T):
            s = [sum(q[h, t, i] * k[h, u, i] for i in range(hd)) / math.sqrt(hd) for u in range(t + 1)]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            tot = sum(e)
            for i in range(hd):
                o[h, t, i] = sum(e[u] / tot * v[h, u, i] for u in range(t + 1))
    return o


def test_attention_brute_force():
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((2, 6, 4)) for _ in range(3))
    o, _ = attention_fwd(q, k, v)
    np.testing.assert_allclose(o, _attention_loops(q, k, v), rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(4)
    # T = 1: the only key is the query's own position, so o = v
    q, k, v = (rng.standard_normal((3, 1, 8)) for _ in range(3))
    o, _ = attention_fwd(q, k, v)
    np.testing.assert_allclose(o, v, rtol=1e-14)
    # all keys equal: uniform weights over the causal prefix -> running mean of v
    q = rng.standard_normal((1, 7, 8))
    k = np.repeat(rng.standard_normal((1, 1, 8)), 7, axis=1)
    v = rng.standard_normal((1, 7, 8))
    o, _ = attention_fwd(q, k, v)
    run = np.cumsum(v, axis=1) / np.arange(1, 8)[None, :, None]
    np.testing.assert_allclose(o, run, rtol=1e-12, atol=1e-13)


def test_attention_bwd_finite_differences():
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((2, 5, 4)) for _ in range(3))
    do = rng.standard_normal((2, 5, 4))
    o, p = attention_fwd(q, k, v)
    dq, dk, dv = attention_bwd(do, q, k, v, p)
    h = 1e-6
    for X, dX in ((q, dq), (k, dk), (v, dv)):
        for idx in [(0, 0, 0), (1, 4, 3), (0, 2, 1), (1, 3, 2)]:
            X[idx] += h
            lp = np.sum(attention_fwd(q, k, v)[0] * do)
            X[idx] -= 2 * h
            lm = np.sum(attention_fwd(q, k, v)[0] * do)
            X[idx] += h
            assert abs((lp - lm) / (2 * h) - dX[idx]) < 1e-8


def test_attention_rows_and_key_tail_are_rows_of_the_full_result():
    """The long-sequence evaluators return exactly the corresponding rows of
    the full T x T computation (brute-force and finite-difference pinned
    above), including the first query, tile-crossing rows and the last key."""
    rng = np.random.default_rng(6)
    T, hd = 70, 8
    q, k, v, do = (rng.standard_normal((T, hd)) for _ in range(4))
    o, p = attention_fwd(q, k, v)
    dq, dk, dv = attention_bwd(do, q, k, v, p)
    rows = [0, 1, 31, 32, 63, 69]
    ro, rdq = attention_rows(q, k, v, do, rows)
    np.testing.assert_allclose(ro, o[rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(rdq, dq[rows], rtol=1e-11, atol=1e-12)
    for n in (1, 5, T):
        tk, tv = attention_key_tail(q, k, v, do, n)
        np.testing.assert_allclose(tk, dk[T - n:], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(tv, dv[T - n:], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- RoPE --
def test_rope_closed_form():
    # hd = 2: one pair at frequency theta^0 = 1 -> rotation by t radians
    cos, sin = rope_tables(4, 2, 10000.0, np.float64)
    x = np.tile(np.array([1.0, 0.0]), (4, 1))
    y = rope_apply(x, cos, sin)
    t = np.arange(4)
    np.testing.assert_allclose(y, np.stack([np.cos(t), np.sin(t)], 1), atol=1e-15)
    # hd = 4: second pair (x1, x3) has frequency 10000^(-1/2) = 0.01
    cos, sin = rope_tables(301, 4, 10000.0, np.float64)
    x = np.zeros((301, 4))
    x[:, 1] = 1.0
    y = rope_apply(x, cos, sin)
    assert abs(y[300, 1] - math.cos(3.0)) < 1e-14 and abs(y[300, 3] - math.sin(3.0)) < 1e-14
    assert np.all(y[:, [0, 2]] == 0)


def test_rope_invariants():
    rng = np.random.default_rng(6)
    T, hd = 40, 16
    cos, sin = rope_tables(T, hd, 10000.0, np.float64)
    q = rng.standard_normal(hd)
    k = rng.standard_normal(hd)
    Q = rope_apply(np.tile(q, (T, 1)), cos, sin)
    K = rope_apply(np.tile(k, (T, 1)), cos, sin)
    np.testing.assert_allclose(np.linalg.norm(Q, axis=1), np.linalg.norm(q), rtol=1e-13)
    # <R_t q, R_u k> depends only on t - u
    for d in (0, 3, 11):
        vals = [Q[t] @ K[t - d] for t in range(d, T)]
        np.testing.assert_allclose(vals, vals[0], rtol=1e-11, atol=1e-12)
    X = rng.standard_normal((T, hd))
    np.testing.assert_allclose(rope_apply(rope_apply(X, cos, sin), cos, sin, inverse=True), X, atol=1e-13)


# -------------------------------------------------------------- RMSNorm --
def test_rmsnorm_closed_form_and_scale():
    d = 64
    g = np.linspace(0.5, 1.5, d)
    x = np.full((1, d), -3.0)
    y, r = rmsnorm_fwd(x, g, 1e-5)
    np.testing.assert_allclose(y[0], -3.0 / math.sqrt(9.0 + 1e-5) * g, rtol=1e-14)
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, d))
    y1, _ = rmsnorm_fwd(x, g, 0.0)
    y2, _ = rmsnorm_fwd(37.0 * x, g, 0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-13)
    # backward against finite differences
    dy = rng.standard_normal((5, d))
    dx, dg = rmsnorm_bwd(dy, x, g, rmsnorm_fwd(x, g, 1e-5)[1])
    h = 1e-6
    for idx in [(0, 0), (3, 17), (4, 63)]:
        x[idx] += h
        lp = np.sum(rmsnorm_fwd(x, g, 1e-5)[0] * dy)
        x[idx] -= 2 * h
        lm = np.sum(rmsnorm_fwd(x, g, 1e-5)[0] * dy)
        x[idx] += h
        assert abs((lp - lm) / (2 * h) - dx[idx]) < 1e-8


# ----------------------------------------------------------------- SiLU --
def test_silu_values():
    assert silu(np.float64(0.0)) == 0.0
    assert abs(silu(np.float64(1.0)) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(silu(np.float64(-40.0))) < 1e-15
    assert abs(silu(np.float64(40.0)) - 40.0) < 1e-12
    assert silu_grad(np.float64(0.0)) == 0.5
    z = np.linspace(-6, 6, 25)
    h = 1e-6
    np.testing.assert_allclose(silu_grad(z), (silu(z + h) - silu(z - h)) / (2 * h), atol=1e-9)


# -------------------------------------------------------- cross-entropy --
def test_cross_entropy_uniform_and_rowsum():
    B, T, V = 2, 5, 37
    tok = np.random.default_rng(9).integers(0, V, (B, T))
    loss, dl = cross_entropy(np.full((B, T, V), 3.25), tok)
    assert abs(loss - math.log(V)) < 1e-14
    rng = np.random.default_rng(10)
    logits = rng.standard_normal((B, T, V)) * 4
    loss, dl = cross_entropy(logits, tok)
    np.testing.assert_allclose(dl.sum(-1), 0.0, atol=1e-16)
    assert np.all(dl[:, -1, :] == 0)
    # brute force
    tot = 0.0
    for b in range(B):
        for t in range(T - 1):
            row = logits[b, t]
            tot += math.log(sum(math.exp(z) for z in row)) - row[tok[b, t + 1]]
    assert abs(loss - tot / (B * (T - 1))) < 1e-13


# ---------------------------------------------------------- whole model --
def test_initial_loss_near_closed_form():
    """z rows have mean square ~1 and Wh ~ N(0, 0.02^2), so logits are
    ~N(0, 4e-4*d) and the initial loss is about ln V + sigma^2/2."""
    o = Oracle(TINY, np.float64)
    loss = o.loss_only(datagen.init_params(TINY), datagen.tokens(TINY))
    expect = math.log(TINY.vocab) + 0.5 * 4e-4 * TINY.d_model
    assert abs(loss - expect) < 0.02


def test_forward_is_causal():
    P = datagen.init_params(TINY)
    tok = datagen.tokens(TINY).copy()
    o = Oracle(TINY, np.float64)
    k1, k2 = {}, {}
    o.forward_backward(P, tok, keep=k1)
    tok[:, -1] = (tok[:, -1] + 1) % TINY.vocab
    tok[0, 40] = (tok[0, 40] + 7) % TINY.vocab
    o.forward_backward(P, tok, keep=k2)
    np.testing.assert_array_equal(k1["logits"][1, :-1], k2["logits"][1, :-1])
    np.testing.assert_array_equal(k1["logits"][0, :40], k2["logits"][0, :40])
    assert not np.array_equal(k1["logits"][0, 40], k2["logits"][0, 40])


def _micro_forward_loops(P, tok, cfg):
    """Pure-Python loop forward of the decoder (a different code path)."""
    B, T, d, H, hd, L = cfg.batch, cfg.seq_len, cfg.d_model, cfg.n_heads, cfg.head_dim, cfg.n_layers

    def rms(vec, g):
        s = math.sqrt(sum(a * a for a in vec) / len(vec) + cfg.rms_eps)
        return [a / s * gg for a, gg in zip(vec, g)]

    def mv(W, vec):
        return [sum(W[i][j] * vec[j] for j in range(len(vec))) for i in range(len(W))]

    def rot(vec, t):
        out = list(vec)
        for hh in range(H):
            for i in range(hd // 2):
                ang = t * cfg.rope_theta ** (-2.0 * i / hd)
                a, b = vec[hh * hd + i], vec[hh * hd + i + hd // 2]
                out[hh * hd + i] = a * math.cos(ang) - b * math.sin(ang)
                out[hh * hd + i + hd // 2] = a * math.sin(ang) + b * math.cos(ang)
        return out

    P = {k: np.asarray(v, dtype=np.float64).tolist() for k, v in P.items()}
    total = 0.0
    for b in range(B):
        xs = [list(P["E"][tok[b, t]]) for t in range(T)]
        for l in range(L):
            W = {k: P[f"{l}.{k}"] for k in datagen.LAYER_TENSORS}
            hs = [rms(x, P[f"{l}.attn_norm"]) for x in xs]
            qs = [rot(mv(W["wq"], h), t) for t, h in enumerate(hs)]
            ks = [rot(mv(W["wk"], h), t) for t, h in enumerate(hs)]
            vs = [mv(W["wv"], h) for h in hs]
            new = []
            for t in range(T):
                o = [0.0] * d
                for hh in range(H):
                    sl = range(hh * hd, (hh + 1) * hd)
                    sc = [sum(qs[t][i] * ks[u][i] for i in sl) / math.sqrt(hd) for u in range(t + 1)]
                    mx = max(sc)
                    e = [math.exp(s - mx) for s in sc]
                    z = sum(e)
                    for i in sl:
                        o[i] = sum(e[u] / z * vs[u][i] for u in range(t + 1))
                x1 = [a + c for a, c in zip(xs[t], mv(W["wo"], o))]
                h2 = rms(x1, P[f"{l}.ffn_norm"])
                gg = mv(W["wg"], h2)
                uu = mv(W["wu"], h2)
                y = [gv / (1 + math.exp(-gv)) * uv for gv, uv in zip(gg, uu)]
                new.append([a + c for a, c in zip(x1, mv(W["wd"], y))])
            xs = new
        for t in range(T - 1):
            z = rms(xs[t], P["final_norm"])
            logits = mv(P["wh"], z)
            mx = max(logits)
            total += mx + math.log(sum(math.exp(a - mx) for a in logits)) - logits[tok[b, t + 1]]
    return total / (B * (T - 1))


def test_micro_model_against_loops():
    cfg = datagen.ModelShape("micro", 2, 8, 2, 4, 12, 11, 2, 5, store_dtype=datagen.F32)
    P = datagen.init_params(cfg)
    rng = np.random.default_rng(11)
    # non-unit gains so that a gain applied to the wrong tensor is caught
    for k in P:
        if k.endswith("norm"):
            P[k] = (1.0 + 0.3 * rng.standard_normal(cfg.d_model)).astype(np.float32)
        else:
            P[k] = (P[k] * 20).astype(np.float32)
    tok = datagen.tokens(cfg)
    loss = Oracle(cfg, np.float64).loss_only(P, tok)
    assert abs(loss - _micro_forward_loops(P, tok, cfg)) < 1e-12


def test_truncated_backward_equals_the_top_of_the_full_backward():
    """bwd_layers=k returns exactly the head's and the top k layers' gradients
    of the full sweep, and nothing below them."""
    shape = datagen.PRESETS["tiny"].replace(n_layers=3)
    P = datagen.init_params(shape)
    tok = datagen.tokens(shape)
    o = Oracle(shape, np.float32)
    loss, full = o.forward_backward(P, tok)
    loss1, top = o.forward_backward(P, tok, bwd_layers=1)
    assert loss1 == loss
    want = {"wh", "final_norm"} | {f"2.{n}" for n in datagen.LAYER_TENSORS + ("attn_norm", "ffn_norm")}
    assert set(top) == want
    for k in want:
        assert np.array_equal(top[k], full[k]), k


def test_threaded_init_draws_the_same_values():
    shape = datagen.PRESETS["tiny"]
    a = datagen.init_params(shape)
    b = datagen.init_params(shape, threads=4)
    assert a.keys() == b.keys()
    for k in a:
        assert np.array_equal(a[k], b[k]), k
