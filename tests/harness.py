"""Shared helpers of the tests: build a host store from the seeded inputs,
run the HIP step, read tensors back, and the parity metrics."""
from __future__ import annotations

import numpy as np

import datagen
import host_memory_layer_amd as mt


def make_store(shape, mode="streamed", flags=0, host_threads=0, micro_batches=1, head_chunk_tokens=0,
               retain_layers=0, token_chunk=0):
    cfg = mt.make_config(shape, mode=mode, flags=flags, host_threads=host_threads, micro_batches=micro_batches,
                         head_chunk_tokens=head_chunk_tokens, retain_layers=retain_layers, token_chunk=token_chunk)
    store = mt.HostStore(cfg)
    mt.init_store_weights(store, datagen.store_filler(shape))
    return cfg, store


def as_f32(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return datagen.bf16_bits_to_f32(a)
    return a.astype(np.float32)


def oracle_key(name, layer):
    return name if layer is None else f"{layer}.{name}"


def read_all(store, which):
    return {oracle_key(n, l): as_f32(store.logical(n, l, which)).copy() for n, l in store.logical_names()}


def cosine(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))


def maxnorm_rel(a, ref):
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    diff = np.abs(np.asarray(a, np.float64) - ref).max()
    return float(diff / den) if den > 0 else float(diff)


def frob_rel(a, ref):
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(np.asarray(a, np.float64) - ref) / den) if den > 0 else 0.0


# Tolerances for the HIP step against the float32 oracle: loss relative
# error, per-tensor gradient cosine and max-norm relative error, post-Adam
# weight Frobenius relative error.
LOSS_RTOL = 1e-2
GRAD_COS = 0.999
GRAD_MAXREL = 3e-2
W_RTOL = 1e-2


def parity_report(loss, grads, weights, o_loss, o_grads, o_weights):
    rows = []
    for k in o_grads:
        rows.append((k, cosine(grads[k], o_grads[k]), maxnorm_rel(grads[k], o_grads[k]),
                     frob_rel(weights[k], o_weights[k])))
    return abs(loss - o_loss) / abs(o_loss), rows


def assert_parity(loss, grads, weights, o_loss, o_grads, o_weights):
    lrel, rows = parity_report(loss, grads, weights, o_loss, o_grads, o_weights)
    bad = [r for r in rows if not (r[1] >= GRAD_COS and r[2] <= GRAD_MAXREL and r[3] <= W_RTOL)]
    assert lrel <= LOSS_RTOL, f"loss {loss} vs oracle {o_loss}"
    assert not bad, "tensors out of tolerance (name, cos, maxrel, w_rel): " + repr(bad[:8])
    return lrel, rows
