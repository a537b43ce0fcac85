"""Whole training step on the GPU through the C ABI, against the oracle.

Tolerances (tests/harness.py): loss relative error <= 1e-2; per logical
tensor, gradient cosine >= 0.999 and max-norm relative error <= 3e-2;
post-Adam weights Frobenius relative error <= 1e-2.  The streamed,
serialized and resident schedules must agree bit for bit.
"""
import numpy as np
import pytest

import datagen
import host_memory_layer_amd as mt
from oracle import Oracle, adam_update
from tests.harness import (GRAD_COS, GRAD_MAXREL, W_RTOL, assert_parity, cosine, frob_rel, make_store,
                           maxnorm_rel, read_all)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

# A small bf16 decoder: two layers, head_dim 128, ragged vocabulary.
SMALL_BF16 = datagen.ModelShape("small-bf16", 2, 256, 2, 128, 512, 1000, 2, 128)
# The same decoder with an fp32 master copy of the weights on the host.
SMALL_MASTER = SMALL_BF16.replace(name="small-bf16m", store_dtype=datagen.BF16_MASTER)
# Sequences of 256 tokens: a micro-batch of one sequence still has 256
# tokens, enough for the layer backward's K-major weight-gradient GEMMs
# (contraction over tokens: a multiple of 64 and at least 192).
SMALL_T256 = SMALL_BF16.replace(name="small-bf16-T256", seq_len=256)


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_step(shape, mode="streamed", flags=0, steps=1, micro_batches=1, tok=None, head_chunk_tokens=0,
             retain_layers=0, token_chunk=0):
    cfg, store = make_store(shape, mode, flags=flags, micro_batches=micro_batches, head_chunk_tokens=head_chunk_tokens,
                            retain_layers=retain_layers, token_chunk=token_chunk)
    model = mt.Model(cfg, store, "cuda:0")
    tok = datagen.tokens(shape) if tok is None else tok
    losses = [model.step(tok) for _ in range(steps)]
    out = dict(loss=losses[-1], losses=losses, g=read_all(store, "g"), w=read_all(store, "w"),
               m=read_all(store, "m"), v=read_all(store, "v"), stats=model.stats(), t=store.step_count())
    if shape.store_dtype == datagen.BF16_MASTER:
        out["p"] = read_all(store, "p")
    if micro_batches > 1:
        out["a"] = read_all(store, "a")
    model.close()
    store.free()
    return out


def oracle_step(shape):
    P = datagen.init_params(shape)
    tok = datagen.tokens(shape)
    loss, g, w, _ = Oracle(shape, np.float32).step(P, tok, mode="streamed")
    return float(loss), g, w


@pytest.mark.parametrize("shape", [datagen.PRESETS["tiny"], SMALL_BF16], ids=["tiny-f32", "small-bf16"])
def test_step_matches_oracle(shape):
    need_gpu()
    print(f"step parity {shape.name}", flush=True)
    r = run_step(shape)
    o_loss, o_g, o_w = oracle_step(shape)
    lrel, rows = assert_parity(r["loss"], r["g"], r["w"], o_loss, o_g, o_w)
    assert r["t"] == 1
    print(f"loss {r['loss']:.6f} vs {o_loss:.6f} rel {lrel:.2e}; min cos {min(x[1] for x in rows):.6f}; "
          f"max grad rel {max(x[2] for x in rows):.2e}; max w rel {max(x[3] for x in rows):.2e}")


@pytest.mark.parametrize("shape", [datagen.PRESETS["tiny"], SMALL_BF16, SMALL_MASTER],
                         ids=["tiny-f32", "small-bf16", "small-bf16m"])
def test_schedules_bitwise_equal(shape):
    need_gpu()
    ref = run_step(shape, "streamed")
    # retain: layers whose forward intermediates stay on the device, so that
    # their backward skips the recompute
    sdma = mt.MT_FLAG_SDMA_QUEUES
    for mode, flags, retain in (("serialized", 0, 0), ("resident", 0, 0), ("single_slot", 0, 0),
                                ("streamed", mt.MT_FLAG_POISON, 0), ("single_slot", mt.MT_FLAG_POISON, 0),
                                ("streamed", 0, 1), ("streamed", mt.MT_FLAG_POISON, shape.n_layers),
                                ("single_slot", 0, 1), ("streamed", sdma, 0), ("serialized", sdma, 0),
                                ("single_slot", sdma | mt.MT_FLAG_POISON, 0), ("streamed", mt.MT_FLAG_DUPLEX_LINK, 0),
                                ("streamed", mt.MT_FLAG_KEEP_DX, 0), ("resident", mt.MT_FLAG_KEEP_DX, 0)):
        r = run_step(shape, mode, flags, retain_layers=retain)
        assert r["loss"] == ref["loss"], (mode, flags, retain)
        for key in ("g", "w", "m", "v", "p"):
            for k in ref.get(key, {}):
                assert np.array_equal(r[key][k], ref[key][k]), (mode, flags, retain, key, k)


@pytest.mark.parametrize("shape", [datagen.PRESETS["tiny"], SMALL_BF16], ids=["tiny-f32", "small-bf16"])
def test_kept_layer_gradients_follow_the_oracle_chain(shape):
    """MT_FLAG_KEEP_DX: the gradient arriving at every layer boundary,
    dl/dx^l, against the oracle's: its head on the GPU's x^L gives dl/dx^L,
    and each layer's backward, recomputed from the GPU's x^l, carries the
    GPU's dl/dx^{l+1} down to dl/dx^l."""
    need_gpu()
    cfg, store = make_store(shape, flags=mt.MT_FLAG_KEEP_DX)
    model = mt.Model(cfg, store, "cuda:0")
    tok = datagen.tokens(shape)
    model.step(tok)
    L = shape.n_layers
    x = [model.checkpoint(l).cpu().numpy() for l in range(L + 1)]
    dx = [model.grad(l).cpu().numpy() for l in range(L + 1)]
    gE = store.logical("E", None, "g").copy()
    model.close()
    store.free()
    P = datagen.init_params(shape)
    o = Oracle(shape, np.float32)
    _, ref, _, _ = o.head(x[L], P, tok)
    pairs = [(L, ref)]
    for l in range(L - 1, -1, -1):
        _, cache = o.layer_fwd(x[l], P, l)
        pairs.append((l, o.layer_bwd(dx[l + 1], cache, P, l, {})))
    for l, r in pairs:
        c, m = cosine(dx[l], r), maxnorm_rel(dx[l], r)
        print(f"  dx^{l}: cos {c:.6f} maxrel {m:.2e}", flush=True)
        assert c >= GRAD_COS and m <= GRAD_MAXREL, (l, c, m)
    # the embedding gradient is the fp32 sum of dl/dx^0 over each token's
    # positions in increasing order, then rounded to the store: bit for bit
    dE = np.zeros((shape.vocab, shape.d_model), np.float32)
    np.add.at(dE, tok.reshape(-1), dx[0])
    if shape.store_dtype == datagen.F32:
        assert np.array_equal(gE, dE)
    else:
        assert np.array_equal(gE, datagen.f32_to_bf16_bits(dE))


def _bitwise_same(a, b, what):
    assert a["loss"] == b["loss"], what
    for key in ("g", "w", "m", "v"):
        for k in a[key]:
            assert np.array_equal(a[key][k], b[key][k]), (what, key, k)


@pytest.mark.parametrize("shape,chunk", [(SMALL_T256, 256), (SMALL_T256.replace(name="small-bf16-3x256", batch=3), 256),
                                         (SMALL_T256.replace(name="small-bf16-5x256", batch=5), 448)],
                         ids=["2-passes", "3-passes", "3-ragged-passes"])
def test_token_passes(shape, chunk):
    """A layer's per-token work in passes of `chunk` tokens.  Everything
    computed per token does not depend on the passes: the loss, the gain
    gradients (their partial sums reduce in the single pass's order), the
    head and embedding gradients are bit for bit those of a single pass; the
    weight gradients are summed over the passes in fp32 and differ by
    rounding.  Parity with the oracle; the streamed, serialized and
    single-slot schedules (with poison, with SDMA queues) agree bit for bit."""
    need_gpu()
    print(f"token passes {shape.name} chunk {chunk}", flush=True)
    one = run_step(shape)
    r = run_step(shape, token_chunk=chunk)
    assert r["loss"] == one["loss"]
    for k in r["g"]:
        if k.endswith("norm") or k in ("E", "wh"):
            assert np.array_equal(r["g"][k], one["g"][k]), k
        else:
            assert cosine(r["g"][k], one["g"][k]) > 0.99999, k
    o_loss, o_g, o_w = oracle_step(shape)
    assert_parity(r["loss"], r["g"], r["w"], o_loss, o_g, o_w)
    for mode, flags in (("serialized", 0), ("single_slot", mt.MT_FLAG_POISON), ("streamed", mt.MT_FLAG_SDMA_QUEUES)):
        _bitwise_same(run_step(shape, mode, flags, token_chunk=chunk), r, (mode, flags))


@pytest.mark.parametrize("shape,chunk", [(SMALL_BF16, 0), (SMALL_T256, 256)], ids=["one-pass", "2-passes"])
def test_bf16_checkpoints(shape, chunk):
    """MT_FLAG_CKPT_BF16: the forward still carries the fp32 residual stream
    (the loss is bit for bit the fp32 checkpoints' one); the backward
    recomputes each layer from its rounded checkpoint.  Parity with the
    oracle; schedules bit for bit."""
    need_gpu()
    print(f"bf16 checkpoints {shape.name} chunk {chunk}", flush=True)
    ref = run_step(shape, token_chunk=chunk)
    r = run_step(shape, flags=mt.MT_FLAG_CKPT_BF16, token_chunk=chunk)
    assert r["loss"] == ref["loss"]
    o_loss, o_g, o_w = oracle_step(shape)
    lrel, rows = assert_parity(r["loss"], r["g"], r["w"], o_loss, o_g, o_w)
    print(f"  min cos {min(x[1] for x in rows):.6f} max grad rel {max(x[2] for x in rows):.2e}", flush=True)
    ck = mt.MT_FLAG_CKPT_BF16
    for mode, flags in (("serialized", ck), ("single_slot", ck | mt.MT_FLAG_POISON), ("streamed", ck | mt.MT_FLAG_SDMA_QUEUES)):
        _bitwise_same(run_step(shape, mode, flags, token_chunk=chunk), r, (mode, flags))


SMALL_L4 = SMALL_BF16.replace(name="small-bf16-L4", n_layers=4)
# a layer's backward outlasts moving its weights and gradients: offloads are
# held behind the next prefetch
YIELDING = SMALL_BF16.replace(name="small-bf16-16k", n_layers=3, batch=1, seq_len=16384)


@pytest.mark.parametrize("shape,mode,flags", [
    (datagen.PRESETS["tiny"], "streamed", 0), (SMALL_L4, "streamed", 0), (SMALL_L4, "serialized", 0),
    (SMALL_L4, "single_slot", mt.MT_FLAG_POISON), (SMALL_L4, "streamed", mt.MT_FLAG_POISON | mt.MT_FLAG_SDMA_QUEUES),
    (YIELDING, "streamed", 0), (YIELDING, "streamed", mt.MT_FLAG_SDMA_QUEUES)],
    ids=["tiny", "streamed", "serialized", "single-slot-poison", "sdma-poison", "yield", "yield-sdma"])
def test_injected_delays_change_nothing(shape, mode, flags):
    """MT_FLAG_DELAYS holds back prefetches, compute uses, offloads and Adam
    updates by seeded host-side delays of up to 2 ms: over two steps (the
    second fetches what the first step's Adam wrote) every result is bit for
    bit that of the undelayed run."""
    need_gpu()
    print(f"delays {shape.name} {mode} flags {flags}", flush=True)
    ref = run_step(shape, mode, flags, steps=2)
    r = run_step(shape, mode, flags | mt.MT_FLAG_DELAYS, steps=2)
    assert r["losses"] == ref["losses"]
    _bitwise_same(r, ref, (mode, flags))
    assert r["stats"]["step_ms"] > ref["stats"]["step_ms"]


def test_kernel_times_add_up_to_the_step_totals():
    """mt_get_kernel_times: one record per timed launch of the last step,
    GEMM flops 2mnk, and the records sum to the step's totals."""
    need_gpu()
    shape = SMALL_L4
    cfg, store = make_store(shape, flags=mt.MT_FLAG_TIME_KERNELS)
    model = mt.Model(cfg, store, "cuda:0")
    model.step(datagen.tokens(shape))
    st, kt = model.stats(), model.kernel_times()
    model.close()
    store.free()
    g = [t for t in kt if t["kind"] in (0, 2)]
    a = [t for t in kt if t["kind"] == 1]
    assert len(g) == st["gemm_launches"] and len(a) == st["attn_launches"] > 0
    assert all(t["flops"] == 2.0 * t["m"] * t["n"] * t["k"] and t["ms"] > 0 for t in g if t["kind"] == 0)
    d, F, M = shape.d_model, shape.d_ff, shape.batch * shape.seq_len
    assert all(t["flops"] == 2.0 * M * (2 * F * d + d * F + d * d) for t in g if t["kind"] == 2)
    assert abs(sum(t["ms"] for t in g) - st["gemm_ms"]) <= 1e-6 * st["gemm_ms"]
    assert sum(t["flops"] for t in g) == st["gemm_flops"]
    # per layer: forward 4, recompute 3 (no down projection), backward 5 data and q/k/v weight
    # gradients plus one grouped launch for the other weight gradients; 3 in the head
    assert len([t for t in g if t["kind"] == 2]) == shape.n_layers
    assert len(g) == 13 * shape.n_layers + 3


def test_repeated_step_is_deterministic_and_t_advances():
    need_gpu()
    shape = datagen.PRESETS["tiny"]
    a = run_step(shape, steps=2)
    b = run_step(shape, steps=2)
    assert a["t"] == 2 and a["losses"] == b["losses"]
    for k in a["w"]:
        assert np.array_equal(a["w"][k], b["w"][k])
    # two steps of the oracle with its own Adam state
    P = datagen.init_params(shape)
    tok = datagen.tokens(shape)
    o = Oracle(shape, np.float32)
    l1, _, P1, M1 = o.step(P, tok, t=1)
    l2, g2, P2, _ = o.step(P1, tok, t=2, moments=M1)
    assert abs(a["losses"][1] - l2) / abs(l2) < 1e-2
    assert a["losses"][1] < a["losses"][0]
    # weights after the second Adam step (t = 2 bias corrections)
    for k in a["w"]:
        assert frob_rel(a["w"][k], P2[k]) <= W_RTOL, k


def test_fp32_master_store_matches_oracle():
    """fp32 master store: the device step is the bf16 store's (same loss, G,
    m, v and, after one step, the same streamed W bit for bit); the master P
    follows the oracle's float32 weights over two steps, and W is P rounded
    to nearest even."""
    need_gpu()
    print("fp32 master store", flush=True)
    a = run_step(SMALL_BF16)
    b = run_step(SMALL_MASTER)
    assert b["loss"] == a["loss"]
    for key in "gwmv":
        for k in a[key]:
            assert np.array_equal(b[key][k], a[key][k]), (key, k)
    o_loss, o_g, o_w = oracle_step(SMALL_MASTER)
    assert_parity(b["loss"], b["g"], b["p"], o_loss, o_g, o_w)
    two = run_step(SMALL_MASTER, steps=2)
    assert two["t"] == 2 and two["losses"][0] == b["loss"]
    P = datagen.init_params(SMALL_MASTER)
    tok = datagen.tokens(SMALL_MASTER)
    o = Oracle(SMALL_MASTER, np.float32)
    _, _, P1, M1 = o.step(P, tok, t=1)
    l2, _, P2, _ = o.step(P1, tok, t=2, moments=M1)
    assert abs(two["losses"][1] - l2) / abs(l2) < 1e-2
    for k in two["p"]:
        assert frob_rel(two["p"][k], P2[k]) <= W_RTOL, k
        assert np.array_equal(datagen.f32_to_bf16_bits(two["p"][k]), datagen.f32_to_bf16_bits(two["w"][k])), k
    # the master keeps what bf16 rounding drops: it is not its own rounding
    assert any(not np.array_equal(two["p"][k], two["w"][k]) for k in two["p"])


@pytest.mark.parametrize("shape", [datagen.PRESETS["tiny"], SMALL_BF16, SMALL_MASTER, SMALL_T256],
                         ids=["tiny-f32", "small-bf16", "small-bf16m", "small-bf16-T256-kmajor"])
def test_micro_batches_accumulate_the_batch_gradient(shape):
    """Two micro-batches of one sequence each against the whole batch of two.

    Exact: the loss scale of a micro-batch is 1/(2*(T-1)), half that of a
    lone sequence, and halving commutes with every rounding, so the
    accumulator equals (g0 + g1)/2 of two single-sequence runs bit for bit,
    the loss is (l0 + l1)/2, and the update is the oracle's float32 Adam on
    that accumulator.  Against the oracle's step on the whole batch: the
    parity bars.  Streamed and resident schedules agree bit for bit."""
    need_gpu()
    print(f"micro-batches {shape.name}", flush=True)
    tok = datagen.tokens(shape)
    one = shape.replace(batch=1)
    r = run_step(one, micro_batches=2, tok=tok)
    s0 = run_step(one, tok=tok[0:1])
    s1 = run_step(one, tok=tok[1:2])
    assert r["loss"] == np.float32(0.5 * np.float64(s0["loss"]) + 0.5 * np.float64(s1["loss"]))
    P0 = datagen.init_params(one)
    for k in r["a"]:
        a = (s0["g"][k] + s1["g"][k]) * np.float32(0.5)
        assert np.array_equal(r["a"][k], a), k
        w2, m2, v2 = adam_update(P0[k], a, np.zeros_like(a), np.zeros_like(a), 1, shape.lr, shape.beta1,
                                 shape.beta2, shape.adam_eps)
        if shape.store_dtype == datagen.BF16_MASTER:
            assert np.array_equal(r["p"][k], w2), k
        if shape.store_dtype != datagen.F32:
            w2 = datagen.bf16_bits_to_f32(datagen.f32_to_bf16_bits(w2))
        assert np.array_equal(r["w"][k], w2) and np.array_equal(r["m"][k], m2) and np.array_equal(r["v"][k], v2), k
    o_loss, o_g, o_w = oracle_step(shape)
    assert_parity(r["loss"], r["a"], r["w"], o_loss, o_g, o_w)
    # resident, and streamed with layer 0's intermediates kept between the
    # sweeps' forward and backward (each micro-batch overwrites them)
    for mode, retain in (("resident", 0), ("streamed", 1)):
        res = run_step(one, mode, micro_batches=2, tok=tok, retain_layers=retain)
        assert res["loss"] == r["loss"], (mode, retain)
        for key in "awmv":
            for k in r[key]:
                assert np.array_equal(res[key][k], r[key][k]), (mode, retain, key, k)


@pytest.mark.parametrize("shape,chunk", [(datagen.PRESETS["tiny"], 48), (SMALL_BF16, 96)],
                         ids=["tiny-f32", "small-bf16"])
def test_head_in_passes(shape, chunk):
    """The output head in passes of `chunk` tokens (the last one ragged).
    Each token's logits, loss and logit gradients, and so dz and every
    gradient below the head, do not depend on the pass: bit for bit equal to
    the single pass.  The head weight gradient is summed over the passes in
    fp32, so it differs by rounding only.  Parity with the oracle and across
    schedules holds as for the single pass."""
    need_gpu()
    print(f"head passes {shape.name} chunk {chunk}", flush=True)
    one = run_step(shape)
    r = run_step(shape, head_chunk_tokens=chunk)
    assert r["loss"] == one["loss"]
    for k in r["g"]:
        if k == "wh":
            from tests.harness import cosine, maxnorm_rel
            assert cosine(r["g"][k], one["g"][k]) > 0.99999 and maxnorm_rel(r["g"][k], one["g"][k]) < 1e-2
        else:
            assert np.array_equal(r["g"][k], one["g"][k]), k
    o_loss, o_g, o_w = oracle_step(shape)
    assert_parity(r["loss"], r["g"], r["w"], o_loss, o_g, o_w)
    res = run_step(shape, "resident", head_chunk_tokens=chunk)
    assert res["loss"] == r["loss"]
    for key in "gwmv":
        for k in r[key]:
            assert np.array_equal(res[key][k], r[key][k]), (key, k)


@pytest.mark.parametrize("shape,resume_mode", [(datagen.PRESETS["tiny"], "streamed"), (SMALL_BF16, "single_slot"),
                                               (SMALL_MASTER, "streamed")],
                         ids=["tiny-f32", "small-bf16-single-slot", "small-bf16m"])
def test_checkpoint_resume_continues_bit_for_bit(shape, resume_mode, tmp_path):
    """Steps 1-2, checkpoint, steps 3-4 on one store; a fresh store resumed
    from the checkpoint (in the streamed or the single-slot schedule) gives
    the same losses and the same W, m, v bit for bit."""
    need_gpu()
    tok = datagen.tokens(shape)
    cfg, store = make_store(shape)
    model = mt.Model(cfg, store, "cuda:0")
    first = [model.step(tok) for _ in range(2)]
    path = tmp_path / "ckpt.bin"
    store.save(path)
    cont = [model.step(tok) for _ in range(2)]
    keys = "wmvp" if shape.store_dtype == datagen.BF16_MASTER else "wmv"
    ref = {k: read_all(store, k) for k in keys}
    assert store.step_count() == 4
    model.close()
    store.free()
    cfg2, store2 = make_store(shape, resume_mode)
    store2.load(path)
    assert store2.step_count() == 2
    model2 = mt.Model(cfg2, store2, "cuda:0")
    again = [model2.step(tok) for _ in range(2)]
    got = {k: read_all(store2, k) for k in keys}
    assert store2.step_count() == 4
    model2.close()
    store2.free()
    print(f"losses {first} | {cont} | resumed {again}", flush=True)
    assert again == cont
    for k in keys:
        for name in ref[k]:
            assert np.array_equal(got[k][name], ref[k][name]), (k, name)


def test_nonfinite_loss_leaves_store_untouched():
    need_gpu()
    shape = datagen.PRESETS["tiny"]
    cfg, store = make_store(shape)
    store.logical("wh", None, "w")[3, 5] = np.float32(np.nan)
    w0 = read_all(store, "w")
    model = mt.Model(cfg, store, "cuda:0")
    with pytest.raises(mt.MtError) as e:
        model.step(datagen.tokens(shape))
    assert e.value.code == mt.MT_E_NONFINITE
    w1 = read_all(store, "w")
    for k in w0:
        assert np.array_equal(w0[k], w1[k], equal_nan=True)
    assert store.step_count() == 0
    assert not np.any(read_all(store, "m")["wh"])
    model.close()
    store.free()


def test_bad_tokens_rejected():
    need_gpu()
    shape = datagen.PRESETS["tiny"]
    cfg, store = make_store(shape)
    model = mt.Model(cfg, store, "cuda:0")
    tok = datagen.tokens(shape).copy()
    tok[0, 3] = shape.vocab
    with pytest.raises(mt.MtError) as e:
        model.step(tok)
    assert e.value.code == mt.MT_E_INVALID
    model.close()
    store.free()
