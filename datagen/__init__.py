"""Seeded synthetic inputs for the layer-streamed training step.

This module is shared by the tests, the benchmark and the oracle.  It holds
no arithmetic of the method itself (no transformer, no loss, no optimizer):
only the model shapes, the parameter initialisation recipe, the token
generator, and the bfloat16 storage conversion of the initial values.

Recipe (applies to every preset):
  * every logical weight tensor (embedding, q/k/v/o projections, gate/up/down
    projections, output head) is drawn N(0, 0.02^2);
  * the tensor is split row-major into chunks of ``CHUNK`` elements; chunk c of
    tensor ``tid`` comes from ``Generator(PCG64(SeedSequence([seed, tid, c])))``
    via ``standard_normal(float32) * float32(0.02)``, so any slice of any tensor
    can be regenerated on its own;
  * RMSNorm gains start at exactly 1;
  * for a bfloat16 store, the float32 draw is rounded to bfloat16 (round to
    nearest, ties to even) and those rounded values are the initial weights;
  * tokens are ``integers(0, V, (B, T))`` from ``SeedSequence([seed, 0x70C])``.

Tensor ids: E = 0; in layer l: 1 + 16*l + {q:0, k:1, v:2, o:3, g:4, u:5, d:6};
final-norm gain 1 + 16*L + 0 (constant 1, no draw); head Wh = 1 + 16*L + 1.

The architecture (Llama-style decoder, RMSNorm, RoPE, SwiGLU) and the five
shapes follow the configuration list of the task; the pages (MegaTrain,
arXiv 2026, as summarised on radar.chestersoft.de "Methodik") fix only the
storage precisions: bfloat16 weights and gradients, float32 Adam moments.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22
INIT_STD = 0.02
TOKEN_STREAM = 0x70C

F32 = "f32"
BF16 = "bf16"
BF16_MASTER = "bf16m"  # bf16 W streamed, fp32 master copy on the host: same initial values as bf16


@dataclasses.dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    head_dim: int
    d_ff: int
    vocab: int
    batch: int
    seq_len: int
    store_dtype: str = BF16
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.95
    adam_eps: float = 1e-8
    seed: int = 0

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len

    def replace(self, **kw) -> "ModelShape":
        return dataclasses.replace(self, **kw)

    def n_params(self) -> int:
        d, F, V, L = self.d_model, self.d_ff, self.vocab, self.n_layers
        per_layer = 4 * d * d + 3 * d * F + 2 * d
        return V * d + L * per_layer + d + V * d


PRESETS = {
    "tiny": ModelShape("tiny", 2, 128, 4, 32, 512, 512, 2, 64, store_dtype=F32),
    "1.3b": ModelShape("1.3b", 24, 2048, 16, 128, 5504, 32000, 4, 2048),
    "7b": ModelShape("7b", 32, 4096, 32, 128, 11008, 32000, 8, 4096),
    "14b": ModelShape("14b", 48, 5120, 40, 128, 13824, 32000, 8, 4096),
    "120b": ModelShape("120b", 96, 10240, 80, 128, 27648, 32000, 4, 4096),
}

# logical tensor -> (tensor-id offset inside a layer)
LAYER_TENSORS = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")


def layer_tensor_shape(cfg: ModelShape, name: str) -> tuple:
    d, F = cfg.d_model, cfg.d_ff
    return {"wq": (d, d), "wk": (d, d), "wv": (d, d), "wo": (d, d),
            "wg": (F, d), "wu": (F, d), "wd": (d, F)}[name]


def tensor_id(cfg: ModelShape, name: str, layer: int | None = None) -> int:
    if name == "E":
        return 0
    if name == "wh":
        return 1 + 16 * cfg.n_layers + 1
    return 1 + 16 * layer + LAYER_TENSORS.index(name)


# ---------------------------------------------------------------- bfloat16 --
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even); bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ------------------------------------------------------------------- draws --
def _chunk_draw(seed: int, tid: int, c: int, n: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, c])))
    return g.standard_normal(n, dtype=np.float32) * np.float32(INIT_STD)


def draw_flat(seed: int, tid: int, start: int, stop: int, store_dtype: str,
              out: np.ndarray | None = None, pool: ThreadPoolExecutor | None = None) -> np.ndarray:
    """Elements [start, stop) of the row-major flattened tensor ``tid``.

    Returns float32 values already rounded to the store precision, or, when
    ``out`` is a uint16 array, writes the bfloat16 bit patterns into it.
    """
    n = stop - start
    if out is None:
        res = np.empty(n, dtype=np.float32)
    else:
        res = out
        assert res.shape == (n,)

    def work(c):
        lo = max(start, c * CHUNK)
        hi = min(stop, (c + 1) * CHUNK)
        # a chunk's draws form one sequential stream, so drawing its first
        # (hi - c*CHUNK) values gives the same prefix as drawing all CHUNK
        full = _chunk_draw(seed, tid, c, hi - c * CHUNK)
        vals = full[lo - c * CHUNK:]
        if res.dtype == np.uint16:
            res[lo - start: hi - start] = f32_to_bf16_bits(vals)
        elif store_dtype in (BF16, BF16_MASTER):
            res[lo - start: hi - start] = bf16_bits_to_f32(f32_to_bf16_bits(vals))
        else:
            res[lo - start: hi - start] = vals

    chunks = range(start // CHUNK, (stop - 1) // CHUNK + 1) if n > 0 else range(0)
    if pool is None:
        for c in chunks:
            work(c)
    else:
        list(pool.map(work, chunks))
    return res


def init_tensor(cfg: ModelShape, name: str, layer: int | None = None,
                rows: slice | None = None, pool: ThreadPoolExecutor | None = None) -> np.ndarray:
    """Initial value (float32, store-rounded) of a logical tensor, or of a row slice."""
    if name in ("attn_norm", "ffn_norm", "final_norm"):
        return np.ones(cfg.d_model, dtype=np.float32)
    if name == "E" or name == "wh":
        shape = (cfg.vocab, cfg.d_model)
    else:
        shape = layer_tensor_shape(cfg, name)
    tid = tensor_id(cfg, name, layer)
    r0, r1 = (0, shape[0]) if rows is None else (rows.start or 0, rows.stop if rows.stop is not None else shape[0])
    flat = draw_flat(cfg.seed, tid, r0 * shape[1], r1 * shape[1], cfg.store_dtype, pool=pool)
    return flat.reshape(r1 - r0, shape[1])


def init_params(cfg: ModelShape, threads: int = 1) -> dict:
    """All logical parameters as float32 arrays (store-rounded initial values).

    Keys: 'E', 'final_norm', 'wh', and per layer l: f'{l}.attn_norm',
    f'{l}.wq', ..., f'{l}.wd', f'{l}.ffn_norm'.  Only for shapes that fit in
    RAM.  ``threads`` > 1 draws the chunks of a tensor on that many threads
    (same values: every chunk has its own stream).
    """
    pool = ThreadPoolExecutor(threads) if threads > 1 else None
    try:
        p = {"E": init_tensor(cfg, "E", pool=pool)}
        for l in range(cfg.n_layers):
            p[f"{l}.attn_norm"] = init_tensor(cfg, "attn_norm")
            for nm in LAYER_TENSORS:
                p[f"{l}.{nm}"] = init_tensor(cfg, nm, l, pool=pool)
            p[f"{l}.ffn_norm"] = init_tensor(cfg, "ffn_norm")
        p["final_norm"] = init_tensor(cfg, "final_norm")
        p["wh"] = init_tensor(cfg, "wh", pool=pool)
    finally:
        if pool is not None:
            pool.shutdown()
    return p


def store_filler(cfg: ModelShape):
    """draw(name, layer, out, pool): write the initial value of a logical
    weight tensor into the flat buffer ``out`` (uint16 bf16 bits or float32)."""
    def draw(name, layer, out, pool=None):
        draw_flat(cfg.seed, tensor_id(cfg, name, layer), 0, out.size, cfg.store_dtype, out=out, pool=pool)
    return draw


def tokens(cfg: ModelShape) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, TOKEN_STREAM])))
    return g.integers(0, cfg.vocab, size=(cfg.batch, cfg.seq_len), dtype=np.int32)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1
