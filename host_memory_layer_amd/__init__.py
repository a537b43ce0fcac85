"""Python binding of libmt.so, the MI355X layer-streamed training library.

Argument marshalling only: every step of the training step runs in the HIP
library (include/mt.h, include/mt_kernels.h).  PyTorch provides the device
arena and the three streams (prefetch, compute, offload); the pinned host
store comes from the library.
The binding raises if the library has not been built — there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# MT_LIBRARY selects another build of the library (the AddressSanitizer
# variant libmt_asan.so for the host-code tests)
LIB_PATH = os.environ.get("MT_LIBRARY") or os.path.join(PKG_DIR, "libmt.so")

MT_OK = 0
MT_E_INVALID, MT_E_SIZE, MT_E_ALIGN, MT_E_NOT_BOUND, MT_E_HIP, MT_E_NONFINITE, MT_E_OOM, MT_E_STATE = range(-1, -9, -1)
MT_F32, MT_BF16, MT_BF16_MASTER = 0, 1, 2
STORE_DTYPES = {"f32": MT_F32, "bf16": MT_BF16, "bf16m": MT_BF16_MASTER}
MT_STREAMED, MT_SERIALIZED, MT_RESIDENT, MT_SINGLE_SLOT = 0, 1, 2, 3
MODES = {"streamed": MT_STREAMED, "serialized": MT_SERIALIZED, "resident": MT_RESIDENT,
         "single_slot": MT_SINGLE_SLOT}
MT_BLOCK_EMBED, MT_BLOCK_LAYER, MT_BLOCK_HEAD = 0, 1, 2
MT_FLAG_TIME_KERNELS, MT_FLAG_POISON, MT_FLAG_DUPLEX_LINK, MT_FLAG_KEEP_DX, MT_FLAG_SDMA_QUEUES = 1, 2, 4, 8, 16
MT_FLAG_CKPT_BF16, MT_FLAG_DELAYS, MT_FLAG_PROGRESS = 32, 64, 128
MT_LANE_PREFETCH, MT_LANE_COMPUTE, MT_LANE_OFFLOAD, MT_LANE_HOST = 0, 1, 2, 3
MT_OP_FETCH, MT_OP_POISON, MT_OP_COMPUTE, MT_OP_OFFLOAD, MT_OP_ADAM, MT_OP_END = range(6)
MT_SCHED_MAX_WAITS = 8
EPI_STORE, EPI_F32, EPI_ADD_F32 = 0, 1, 2
GEMM_A_KMAJOR, GEMM_B_KMAJOR = 1, 2


class MtConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_layers", "d_model", "n_heads", "head_dim", "d_ff", "vocab", "batch", "seq_len", "store_dtype")] + \
               [(n, ctypes.c_double) for n in ("rms_eps", "rope_theta", "lr", "beta1", "beta2", "adam_eps")] + \
               [(n, ctypes.c_int32) for n in ("mode", "host_threads", "flags", "micro_batches", "head_chunk_tokens",
                                              "retain_layers", "token_chunk")]


class MtTensorDesc(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_uint64), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32)]


class MtBlockDesc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("layer", ctypes.c_int32), ("n_tensors", ctypes.c_int32),
                ("pad_", ctypes.c_int32)] + \
               [(n, ctypes.c_uint64) for n in ("base", "w_off", "g_off", "m_off", "v_off", "region_elems", "w_bytes",
                                               "mv_bytes")] + \
               [("tensors", MtTensorDesc * 8), ("p_off", ctypes.c_uint64), ("a_off", ctypes.c_uint64)]


class MtStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_double) for n in
                ("step_ms", "device_ms", "fwd_ms", "bwd_ms", "h2d_ms", "d2h_ms", "h2d_bytes", "d2h_bytes",
                 "stall_ms", "adam_ms", "adam_tail_ms", "gemm_ms", "gemm_flops", "attn_ms", "attn_flops")] + \
               [("gemm_launches", ctypes.c_int64), ("attn_launches", ctypes.c_int64), ("loss", ctypes.c_double),
                ("n_blocks", ctypes.c_int32), ("pad_", ctypes.c_int32), ("gemm_bytes", ctypes.c_double)]


class MtLayout(ctypes.Structure):
    _fields_ = [("dma_bytes", ctypes.c_uint64), ("opt_bytes", ctypes.c_uint64), ("n_blocks", ctypes.c_int32),
                ("pad_", ctypes.c_int32)]


class MtBlockStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_double) for n in
                ("fwd_ms", "bwd_ms", "h2d_fwd_ms", "h2d_bwd_ms", "d2h_ms", "stall_fwd_ms", "stall_bwd_ms",
                 "adam_ms")]


class MtKernelTime(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("kind", "m", "n", "k", "epi", "layout")] + \
               [(n, ctypes.c_double) for n in ("flops", "bytes", "ms")]


class MtGemmDesc(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("lda", ctypes.c_int64), ("B", ctypes.c_void_p), ("ldb", ctypes.c_int64),
                ("C", ctypes.c_void_p), ("ldc", ctypes.c_int64), ("M", ctypes.c_int32), ("N", ctypes.c_int32)]


class MtSchedOp(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("lane", "kind", "use", "block", "wslot", "gslot", "n_waits",
                                              "n_link")] + \
               [("waits", ctypes.c_int32 * MT_SCHED_MAX_WAITS), ("link", ctypes.c_int32 * 2)]


class MtError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (code {code})")
        self.code = code


_lib = None

_SIGS = {
    "mt_host_store_layout": (ctypes.c_int, [ctypes.POINTER(MtConfig), ctypes.POINTER(MtLayout),
                                            ctypes.POINTER(MtBlockDesc), ctypes.c_int32]),
    "mt_host_store_bytes": (ctypes.c_size_t, [ctypes.POINTER(MtConfig)]),
    "mt_host_opt_bytes": (ctypes.c_size_t, [ctypes.POINTER(MtConfig)]),
    "mt_alloc_host_opt": (ctypes.c_int, [ctypes.c_size_t, ctypes.POINTER(ctypes.c_void_p)]),
    "mt_free_host_opt": (None, [ctypes.c_void_p, ctypes.c_size_t]),
    "mt_block_count": (ctypes.c_int, [ctypes.POINTER(MtConfig)]),
    "mt_block_info": (ctypes.c_int, [ctypes.POINTER(MtConfig), ctypes.c_int, ctypes.POINTER(MtBlockDesc)]),
    "mt_device_bytes": (ctypes.c_size_t, [ctypes.POINTER(MtConfig)]),
    "mt_alloc_host_store": (ctypes.c_int, [ctypes.c_size_t, ctypes.POINTER(ctypes.c_void_p)]),
    "mt_free_host_store": (None, [ctypes.c_void_p]),
    "mt_init_store_header": (ctypes.c_int, [ctypes.POINTER(MtConfig), ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_void_p, ctypes.c_size_t]),
    "mt_store_step": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)]),
    "mt_store_save": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_char_p]),
    "mt_store_load": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_char_p]),
    "mt_create_model": (ctypes.c_int, [ctypes.POINTER(MtConfig), ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p)]),
    "mt_bind_host_store": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.c_size_t]),
    "mt_train_step": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p]),
    "mt_get_loss": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)]),
    "mt_get_stats": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(MtStats)]),
    "mt_get_block_stats": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(MtBlockStats)]),
    "mt_debug_buffers": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_void_p),
                                        ctypes.POINTER(ctypes.c_void_p)]),
    "mt_debug_grad": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_void_p)]),
    "mt_destroy_model": (None, [ctypes.c_void_p]),
    "mt_host_adam": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64, ctypes.c_double,
                                    ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_int32]),
    "mt_host_adam_master": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64, ctypes.c_double,
                                           ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_int32]),
    "mt_store_init_master": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t]),
    "mt_link_probe": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p),
                                     ctypes.POINTER(ctypes.c_double)]),
    "mt_rmsnorm_fwd": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p]),
    "mt_rmsnorm_fwd_res": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_float, ctypes.c_void_p]),
    "mt_rmsnorm_bwd_ws_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32]),
    "mt_rmsnorm_bwd": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]),
    "mt_swiglu_fwd": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]),
    "mt_swiglu_bwd": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]),
    "mt_rope_bwd_t": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]),
    "mt_xent": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p]),
    "mt_embed_fwd": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]),
    "mt_embed_bwd": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]),
    "mt_schedule": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]),
    "mt_get_kernel_times": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]),
    "mt_last_error": (ctypes.c_char_p, []),
    "mt_version": (ctypes.c_char_p, []),
    "mt_gemm": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                               ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                               ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]),
    "mt_gemm_ws": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                  ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p]),
    "mt_gemm_ws_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
    "mt_gemm_group_ws": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "mt_gemm_group_ws_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32]),
    "mt_gemm_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_void_p]),
    "mt_gemm_noalloc_max_ws": (ctypes.c_size_t, []),
    "mt_transpose": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                    ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]),
    "mt_rope_tables": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p,
                                      ctypes.c_void_p]),
    "mt_token_ld": (ctypes.c_int64, [ctypes.c_int64]),
    "mt_rope_qkv": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]),
    "mt_attention_fwd": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_void_p]),
    "mt_attention_bwd": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_void_p]),
}


def lib():
    """The loaded libmt.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        # torch ships its own HIP runtime under the same soname as the
        # system one this library links against: whichever is loaded first
        # serves the process, and torch finds no GPU under the other.  Load
        # torch's first.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(rc):
    if rc != MT_OK:
        raise MtError(rc, lib().mt_last_error().decode())
    return rc


def make_config(shape, mode="streamed", host_threads=0, flags=0, micro_batches=1, head_chunk_tokens=0,
                retain_layers=0, token_chunk=0) -> MtConfig:
    """mt_config from any object with the model-shape attributes
    (n_layers, d_model, n_heads, head_dim, d_ff, vocab, batch, seq_len,
    store_dtype 'f32'|'bf16'|'bf16m' (bf16 with an fp32 master copy), rms_eps, rope_theta, lr, beta1, beta2, adam_eps)."""
    c = MtConfig()
    for f in ("n_layers", "d_model", "n_heads", "head_dim", "d_ff", "vocab", "batch", "seq_len"):
        setattr(c, f, int(getattr(shape, f)))
    c.store_dtype = STORE_DTYPES[getattr(shape, "store_dtype", "bf16")]
    for f in ("rms_eps", "rope_theta", "lr", "beta1", "beta2", "adam_eps"):
        setattr(c, f, float(getattr(shape, f)))
    c.mode = MODES[mode] if isinstance(mode, str) else int(mode)
    c.host_threads = int(host_threads)
    c.flags = int(flags)
    c.micro_batches = int(micro_batches)
    c.head_chunk_tokens = int(head_chunk_tokens)
    c.retain_layers = int(retain_layers)
    c.token_chunk = int(token_chunk)
    return c


def host_store_bytes(cfg: MtConfig) -> int:
    n = lib().mt_host_store_bytes(ctypes.byref(cfg))
    if n == 0:
        raise MtError(MT_E_INVALID, lib().mt_last_error().decode())
    return n


def host_opt_bytes(cfg: MtConfig) -> int:
    n = lib().mt_host_opt_bytes(ctypes.byref(cfg))
    if n == 0:
        raise MtError(MT_E_INVALID, lib().mt_last_error().decode())
    return n


def device_bytes(cfg: MtConfig) -> int:
    n = lib().mt_device_bytes(ctypes.byref(cfg))
    if n == 0:
        raise MtError(MT_E_INVALID, lib().mt_last_error().decode())
    return n


def store_layout(cfg: MtConfig):
    """(mt_layout, [mt_block_desc per block]) of the host store of cfg."""
    lay = MtLayout()
    check(lib().mt_host_store_layout(ctypes.byref(cfg), ctypes.byref(lay), None, 0))
    blocks = (MtBlockDesc * lay.n_blocks)()
    check(lib().mt_host_store_layout(ctypes.byref(cfg), ctypes.byref(lay), blocks, lay.n_blocks))
    return lay, list(blocks)


def schedule(cfg: MtConfig) -> list:
    """The operations one streamed step of cfg issues (mt_schedule), as dicts
    with lane, kind, use, block, wslot, gslot, waits and link."""
    n = lib().mt_schedule(ctypes.byref(cfg), None, 0)
    if n < 0:
        check(n)
    ops = (MtSchedOp * n)()
    check(min(0, lib().mt_schedule(ctypes.byref(cfg), ops, n)))
    return [dict(lane=o.lane, kind=o.kind, use=o.use, block=o.block, wslot=o.wslot, gslot=o.gslot,
                 waits=list(o.waits[:o.n_waits]), link=list(o.link[:o.n_link])) for o in ops]


def block_infos(cfg: MtConfig) -> list:
    return store_layout(cfg)[1]


def _view(addr: int, nbytes: int, dtype) -> np.ndarray:
    buf = (ctypes.c_uint8 * nbytes).from_address(addr)
    return np.frombuffer(buf, dtype=dtype)


class HostStore:
    """Host store: pinned DMA part (header page + per-block [W | G]) and
    pageable optimizer part (per-block [m | v], then the fp32 master weights
    P of a 'bf16m' store, then the fp32 gradient accumulator A when the
    configuration has micro-batches)."""

    def __init__(self, cfg: MtConfig):
        self.cfg = cfg
        self.nbytes = host_store_bytes(cfg)
        self.opt_nbytes = host_opt_bytes(cfg)
        p = ctypes.c_void_p()
        check(lib().mt_alloc_host_store(self.nbytes, ctypes.byref(p)))
        self.ptr = p.value
        q = ctypes.c_void_p()
        rc = lib().mt_alloc_host_opt(self.opt_nbytes, ctypes.byref(q))
        if rc != MT_OK:
            lib().mt_free_host_store(self.ptr)
            check(rc)
        self.opt_ptr = q.value
        check(lib().mt_init_store_header(ctypes.byref(cfg), self.ptr, self.nbytes, self.opt_ptr, self.opt_nbytes))
        self.blocks = block_infos(cfg)
        self.wdtype = np.float32 if cfg.store_dtype == MT_F32 else np.uint16

    def region(self, block: int, which: str) -> np.ndarray:
        b = self.blocks[block]
        base = self.ptr if which in "wg" else self.opt_ptr
        if which == "p" and self.cfg.store_dtype != MT_BF16_MASTER:
            raise ValueError("the store has no fp32 master copy")
        if which == "a" and self.cfg.micro_batches <= 1:
            raise ValueError("the store has no gradient accumulator")
        off = {"w": b.w_off, "g": b.g_off, "m": b.m_off, "v": b.v_off, "p": b.p_off, "a": b.a_off}[which]
        dt = self.wdtype if which in "wg" else np.float32
        n = b.region_elems
        return _view(base + off, n * np.dtype(dt).itemsize, dt)

    def tensor(self, block: int, index: int, which: str = "w") -> np.ndarray:
        b = self.blocks[block]
        t = b.tensors[index]
        reg = self.region(block, which)
        return reg[t.offset:t.offset + t.rows * t.cols].reshape(t.rows, t.cols)

    def step_count(self) -> int:
        t = ctypes.c_int64()
        check(lib().mt_store_step(self.ptr, ctypes.byref(t)))
        return t.value

    def save(self, path: str):
        """Checkpoint: header, every block's W, and [m | v] (mt_store_save)."""
        check(lib().mt_store_save(self.ptr, self.nbytes, self.opt_ptr, self.opt_nbytes, str(path).encode()))

    def load(self, path: str):
        """Resume from a checkpoint of a store with the same layout (mt_store_load)."""
        check(lib().mt_store_load(self.ptr, self.nbytes, self.opt_ptr, self.opt_nbytes, str(path).encode()))

    def free(self):
        if self.ptr:
            lib().mt_free_host_store(self.ptr)
            self.ptr = None
        if self.opt_ptr:
            lib().mt_free_host_opt(self.opt_ptr, self.opt_nbytes)
            self.opt_ptr = None

    # Logical tensors of the decoder inside the store (weights are [out x in]).
    def logical(self, name: str, layer: int | None = None, which: str = "w") -> np.ndarray:
        c = self.cfg
        d, F, L = c.d_model, c.d_ff, c.n_layers
        if name == "E":
            return self.tensor(0, 0, which)
        if name == "wh":
            return self.tensor(L + 1, 0, which)
        if name == "final_norm":
            return self.tensor(L + 1, 1, which)[0]
        blk = layer + 1
        if name in ("wq", "wk", "wv"):
            i = "qkv".index(name[1])
            return self.tensor(blk, 0, which)[i * d:(i + 1) * d]
        if name == "wo":
            return self.tensor(blk, 1, which)
        if name in ("wg", "wu"):
            i = "gu".index(name[1])
            return self.tensor(blk, 2, which)[i * F:(i + 1) * F]
        if name == "wd":
            return self.tensor(blk, 3, which)
        if name == "attn_norm":
            return self.tensor(blk, 4, which)[0]
        if name == "ffn_norm":
            return self.tensor(blk, 5, which)[0]
        raise KeyError(name)

    def logical_names(self):
        names = [("E", None)]
        for l in range(self.cfg.n_layers):
            names += [("attn_norm", l), ("wq", l), ("wk", l), ("wv", l), ("wo", l), ("ffn_norm", l),
                      ("wg", l), ("wu", l), ("wd", l)]
        names += [("final_norm", None), ("wh", None)]
        return names


class Model:
    """A model handle bound to a host store; device arena and the prefetch,
    compute and offload streams (default priority) from torch."""

    def __init__(self, cfg: MtConfig, store: HostStore, device: str = "cuda:0"):
        import torch
        self.torch = torch
        self.cfg = cfg
        self.store = store
        self.device = torch.device(device)
        nbytes = device_bytes(cfg)
        self.arena = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.streams = [torch.cuda.Stream(device=self.device) for _ in range(3)]  # prefetch, compute, offload
        self.stream = self.streams[1]
        sv = (ctypes.c_void_p * 3)(*[s.cuda_stream for s in self.streams])
        h = ctypes.c_void_p()
        torch.cuda.synchronize(self.device)
        check(lib().mt_create_model(ctypes.byref(cfg), self.arena.data_ptr(), nbytes, sv, ctypes.byref(h)))
        self.handle = h.value
        check(lib().mt_bind_host_store(self.handle, store.ptr, store.nbytes, store.opt_ptr, store.opt_nbytes))

    def step(self, tokens: np.ndarray) -> float:
        tok = np.ascontiguousarray(tokens, dtype=np.int32).reshape(-1)
        if tok.size != max(1, self.cfg.micro_batches) * self.cfg.batch * self.cfg.seq_len:
            raise ValueError("tokens must hold micro_batches*batch*seq_len values")
        check(lib().mt_train_step(self.handle, tok.ctypes.data))
        return self.loss()

    def loss(self) -> float:
        v = ctypes.c_float()
        check(lib().mt_get_loss(self.handle, ctypes.byref(v)))
        return float(v.value)

    def stats(self) -> dict:
        s = MtStats()
        check(lib().mt_get_stats(self.handle, ctypes.byref(s)))
        return {f: getattr(s, f) for f, _ in MtStats._fields_ if f != "pad_"}

    def kernel_times(self) -> list:
        """Every timed launch of the last step (MT_FLAG_TIME_KERNELS), as dicts."""
        n = lib().mt_get_kernel_times(self.handle, None, 0)
        if n < 0:
            check(n)
        out = (MtKernelTime * n)()
        check(min(0, lib().mt_get_kernel_times(self.handle, out, n)))
        return [{f: getattr(o, f) for f, _ in MtKernelTime._fields_} for o in out]

    def block_stats(self, block: int) -> dict:
        s = MtBlockStats()
        check(lib().mt_get_block_stats(self.handle, block, ctypes.byref(s)))
        return {f: getattr(s, f) for f, _ in MtBlockStats._fields_}

    def _arena_view(self, ptr: int, nelem: int, dtype):
        torch = self.torch
        off = ptr - self.arena.data_ptr()
        esz = torch.tensor([], dtype=dtype).element_size()
        return self.arena[off:off + nelem * esz].view(dtype)

    def checkpoint(self, layer: int):
        """Layer-boundary activation x^layer [B*T x d] as float32 (a device view
        of the fp32 checkpoint, or the widened bf16 one with MT_FLAG_CKPT_BF16)."""
        p = ctypes.c_void_p()
        check(lib().mt_debug_buffers(self.handle, layer, ctypes.byref(p), None))
        c = self.cfg
        lp = bool(c.flags & MT_FLAG_CKPT_BF16)
        t = self._arena_view(p.value, c.batch * c.seq_len * c.d_model,
                             self.torch.bfloat16 if lp else self.torch.float32).view(c.batch * c.seq_len, c.d_model)
        return t.float() if lp else t

    def grad(self, layer: int):
        """fp32 gradient dl/dx^layer arriving at layer boundary `layer` [B*T x d]
        (device tensor view; needs MT_FLAG_KEEP_DX)."""
        p = ctypes.c_void_p()
        check(lib().mt_debug_grad(self.handle, layer, ctypes.byref(p)))
        c = self.cfg
        return self._arena_view(p.value, c.batch * c.seq_len * c.d_model, self.torch.float32).view(
            c.batch * c.seq_len, c.d_model)

    def row_loss(self):
        p = ctypes.c_void_p()
        check(lib().mt_debug_buffers(self.handle, 0, None, ctypes.byref(p)))
        c = self.cfg
        return self._arena_view(p.value, c.batch * c.seq_len, self.torch.float32)

    def close(self):
        """Destroy the model and drop its reference to the device arena."""
        if getattr(self, "handle", None):
            lib().mt_destroy_model(self.handle)
            self.handle = None
        self.arena = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def link_probe(sizes, reps=4, sdma=False, device="cuda:0") -> list:
    """Host-link GB/s (host->device, device->host, both at once) with the
    library's own copy path (mt_link_probe) at each byte count in `sizes`."""
    import torch
    n = max(sizes)
    ha, hb = ctypes.c_void_p(), ctypes.c_void_p()
    check(lib().mt_alloc_host_store(n, ctypes.byref(ha)))
    try:
        check(lib().mt_alloc_host_store(n, ctypes.byref(hb)))
    except MtError:
        lib().mt_free_host_store(ha.value)
        raise
    try:
        dev = torch.device(device)
        da = torch.empty(n, dtype=torch.uint8, device=dev)
        db = torch.empty(n, dtype=torch.uint8, device=dev)
        ss = [torch.cuda.Stream(device=dev) for _ in range(2)]
        sv = (ctypes.c_void_p * 2)(*[s.cuda_stream for s in ss])
        torch.cuda.synchronize(dev)
        out = []
        for b in sizes:
            r = (ctypes.c_double * 3)()
            check(lib().mt_link_probe(da.data_ptr(), db.data_ptr(), ha.value, hb.value, int(b), int(reps),
                                      MT_FLAG_SDMA_QUEUES if sdma else 0, sv, r))
            out.append({"bytes": int(b), "h2d_gbs": r[0], "d2h_gbs": r[1], "bidir_gbs": r[2]})
        del da, db
        return out
    finally:
        lib().mt_free_host_store(ha.value)
        lib().mt_free_host_store(hb.value)


def init_store_weights(store: HostStore, draw, threads: int = 0):
    """Fill every weight tensor from ``draw(name, layer, out, pool)``, which
    writes the initial value of a logical tensor into ``out`` (a flat uint16
    bf16 view or float32 view of the store).  Gains are set to 1.  G, m, v
    and the padding were zeroed when the store header was written.  A 'bf16m'
    store's fp32 master copy is then set to the widened bf16 weights."""
    from concurrent.futures import ThreadPoolExecutor
    one = np.float32(1.0)
    one_bits = np.uint16(0x3F80)
    jobs = []
    for name, layer in store.logical_names():
        view = store.logical(name, layer, "w")
        if name.endswith("norm"):
            view[...] = one_bits if view.dtype == np.uint16 else one
        else:
            jobs.append((name, layer, view))
    nthreads = threads or (len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 1)
    with ThreadPoolExecutor(max(1, nthreads)) as pool:
        for name, layer, view in jobs:
            draw(name, layer, view.reshape(-1), pool)
    if store.cfg.store_dtype == MT_BF16_MASTER:
        check(lib().mt_store_init_master(store.ptr, store.nbytes, store.opt_ptr, store.opt_nbytes))
