"""The training step at the full configuration sizes, through the C ABI,
against the oracle on outputs it can compute one by one and on properties
that hold at any size.

* 1.3B shape (24 layers, d 2048, 16 heads, batch 4 x 2048): the loss of the
  oracle's whole forward (float32); the head's and the top two layers'
  gradients and post-Adam weights from the oracle's backward driven by the
  GPU's checkpoints; to the bars of tests/harness.py.
* 7B and 14B shapes with every layer, and the 120B shape with 2 layers (its
  96 layers need 1.47 TB of host memory):
  - one layer's forward, recomputed by the oracle from the GPU's own fp32
    checkpoint x^l on a prefix of one sequence (attention is causal, so the
    prefix is exact), at the first and the last layer; compared on the
    layer's increment x^{l+1} - x^l with the gradient bars;
  - per-position losses from the GPU's x^L, at sampled positions;
  - the loss is the mean of the per-position losses;
  - the host Adam relation, bit for bit, on a slice of every tensor;
  - embedding-gradient rows of tokens that do not occur are exactly zero.
* The streamed, serialized, resident and single-slot schedules agree bit for
  bit at the 14B and 120B per-layer shapes with 2 layers.
* Long context: the 7B width with 2 layers over one 131072-token sequence,
  whose output head runs in passes of 22272 tokens: the same checks, with
  head positions on both sides of every pass boundary.
"""
import gc
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import datagen
import host_memory_layer_amd as mt
from oracle import Oracle, adam_update
from tests.harness import (GRAD_COS, GRAD_MAXREL, LOSS_RTOL, as_f32, assert_parity, cosine, frob_rel, make_store,
                           maxnorm_rel, parity_report)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

P13 = datagen.PRESETS["1.3b"]
P7 = datagen.PRESETS["7b"]
P14 = datagen.PRESETS["14b"]
P120_L2 = datagen.PRESETS["120b"].replace(n_layers=2)


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
        self.store.free()
        gc.collect()


def pool():
    return ThreadPoolExecutor(datagen.default_threads())


def layer_params(shape, l, ex):
    P = {f"{l}.{nm}": datagen.init_tensor(shape, nm, l, pool=ex) for nm in datagen.LAYER_TENSORS}
    P[f"{l}.attn_norm"] = datagen.init_tensor(shape, "attn_norm")
    P[f"{l}.ffn_norm"] = datagen.init_tensor(shape, "ffn_norm")
    return P


# ------------------------------------------------------------ 1.3B parity --
def test_1p3b_loss_head_and_top_layers_match_oracle():
    """Loss: the oracle's whole forward from the seeded inputs.  Gradients
    and post-Adam weights of the head and the top two layers: the oracle's
    head and backward sweep driven by the GPU's own fp32 checkpoints x^l
    (each layer recomputed from x^l, as the streamed schedule does), so that
    every compared tensor measures the arithmetic of one block, not the drift
    that 24 layers of bf16 operands leave in the checkpoints."""
    need_gpu()
    shape = P13
    L = shape.n_layers
    top = (L - 1, L - 2)
    print(f"1.3B parity: {L} layers, {shape.batch}x{shape.seq_len} tokens", flush=True)
    r = Run(shape)
    try:
        keys = [("wh", None), ("final_norm", None)] + [
            (n, l) for l in top for n in datagen.LAYER_TENSORS + ("attn_norm", "ffn_norm")]
        name = lambda n, l: n if l is None else f"{l}.{n}"
        g = {name(n, l): as_f32(r.store.logical(n, l, "g")).copy() for n, l in keys}
        w = {name(n, l): as_f32(r.store.logical(n, l, "w")).copy() for n, l in keys}
        xs = {l: r.model.checkpoint(l).cpu().numpy() for l in top + (L,)}
        loss = r.loss
    finally:
        r.close()
    P = datagen.init_params(shape, threads=datagen.default_threads())
    o = Oracle(shape, np.float32)
    o_loss = float(o.loss_only(P, r.tok))
    _, dx, o_g, _ = o.head(xs[L], P, r.tok.reshape(shape.batch, shape.seq_len))
    for l in top:
        _, cache = o.layer_fwd(xs[l], P, l)
        dx = o.layer_bwd(dx, cache, P, l, o_g)
        del cache
    o_w = {}
    for k in g:
        z = np.zeros_like(P[k])
        o_w[k] = adam_update(P[k], o_g[k], z, z, 1, shape.lr, shape.beta1, shape.beta2, shape.adam_eps)[0]
    o_g = {k: o_g[k] for k in g}
    for k, c, e, we in parity_report(loss, g, w, o_loss, o_g, o_w)[1]:
        print(f"  {k:16s} cos {c:.6f} maxrel {e:.2e} frob {frob_rel(g[k], o_g[k]):.2e} w_rel {we:.2e}", flush=True)
    lrel, rows = assert_parity(loss, g, w, o_loss, o_g, o_w)
    print(f"loss {loss:.6f} vs {o_loss:.6f} rel {lrel:.2e}; min cos {min(x[1] for x in rows):.6f}; "
          f"max grad rel {max(x[2] for x in rows):.2e}; max w rel {max(x[3] for x in rows):.2e}")


# ------------------------------------------------------- sampled outputs --
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


@pytest.mark.parametrize("shape", [P7, P14, P120_L2], ids=["7b", "14b", "120b-2layers"])
def test_fullsize_sampled_outputs_and_properties(shape):
    need_gpu()
    L, T = shape.n_layers, shape.seq_len
    print(f"{shape.name}: {L} layers, d {shape.d_model}, {shape.batch}x{T} tokens", flush=True)
    r = Run(shape)
    try:
        with pool() as ex:
            check_layer_prefix(r, 0, 1, T, ex)
            check_layer_prefix(r, L - 1, shape.batch - 1, 512, ex)
            positions = [0, 1, T - 2, T - 1, T, 2 * T - 1, 3 * T // 2 + 5, shape.batch * T - 2, shape.batch * T - 1]
            check_head_rows(r, positions, ex)
            check_adam_relation(r, ex)
        check_embedding_rows(r)
    finally:
        r.close()


def test_long_context_7b_width_two_layers():
    shape = P7.replace(n_layers=2, batch=1, seq_len=131072)
    T = shape.seq_len
    print(f"{shape.name} long context: 2 layers, d {shape.d_model}, 1x{T} tokens", flush=True)
    r = Run(shape)
    try:
        with pool() as ex:
            check_layer_prefix(r, 0, 0, 4096, ex)
            check_layer_prefix(r, 1, 0, 512, ex)
            hc = 22272  # head pass: the largest multiple of 256 tokens within 4 GiB of logits and gradients
            assert hc * shape.vocab * 6 <= 4 << 30 < (hc + 256) * shape.vocab * 6
            edges = [p * hc + e for p in range(1, T // hc + 1) for e in (-1, 0) if p * hc + e < T]
            check_head_rows(r, [0, 1] + edges + [T - 2, T - 1], ex)
            check_adam_relation(r, ex)
        check_embedding_rows(r)
    finally:
        r.close()


@pytest.mark.parametrize("shape", [P14.replace(n_layers=2), P120_L2], ids=["14b-2layers", "120b-2layers"])
def test_fullsize_schedules_bitwise_equal(shape):
    need_gpu()
    print(f"{shape.name} with {shape.n_layers} layers: streamed vs serialized vs resident vs single slot "
          "vs streamed with layer 0's intermediates retained", flush=True)
    ref = Run(shape, "streamed")
    try:
        ref.drop_model()
        for mode, retain in (("serialized", 0), ("resident", 0), ("single_slot", 0), ("streamed", 1)):
            r = Run(shape, mode, retain_layers=retain)
            try:
                assert r.loss == ref.loss, mode
                for b in range(len(ref.store.blocks)):
                    for which in "wgmv":
                        assert np.array_equal(r.store.region(b, which), ref.store.region(b, which)), (mode, b, which)
            finally:
                r.close()
    finally:
        ref.close()
