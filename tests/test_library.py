"""Host-side tests of the C-ABI library (no GPU calls): symbols, store
layout, configuration checks, and the host Adam against the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

import datagen
import host_memory_layer_amd as mt
from oracle import adam_update

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    names = set()
    for h in ("mt.h", "mt_kernels.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(mt_[a-z0-9_]+)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol():
    L = mt.lib()
    names = declared_symbols()
    assert len(names) >= 20
    for n in sorted(names):
        assert hasattr(L, n), n
    assert set(mt._SIGS) == names


def test_torch_runtime_loads_before_the_library():
    """torch's HIP runtime and the system one share a soname: the binding
    must load torch's first, or torch finds no GPU in that process."""
    import subprocess
    import sys
    code = ("import sys, host_memory_layer_amd as mt; assert 'torch' not in sys.modules; mt.lib(); "
            "assert 'torch' in sys.modules; print('ok')")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-2000:]


def test_struct_sizes_match_header():
    # layout of the C structs, mirrored by ctypes
    assert ctypes.sizeof(mt.MtConfig) == 9 * 4 + 4 + 6 * 8 + 7 * 4 + 4
    assert ctypes.sizeof(mt.MtTensorDesc) == 16
    assert ctypes.sizeof(mt.MtBlockDesc) == 16 + 8 * 8 + 8 * 16 + 2 * 8
    assert ctypes.sizeof(mt.MtStats) == 15 * 8 + 2 * 8 + 8 + 2 * 4 + 8
    assert ctypes.sizeof(mt.MtSchedOp) == (8 + mt.MT_SCHED_MAX_WAITS + 2) * 4
    assert ctypes.sizeof(mt.MtKernelTime) == 6 * 4 + 3 * 8


@pytest.mark.parametrize("name,dtype", [(n, None) for n in datagen.PRESETS] +
                         [("1.3b", datagen.BF16_MASTER), ("14b", datagen.BF16_MASTER)])
def test_store_layout(name, dtype):
    shape = datagen.PRESETS[name]
    if dtype:
        shape = shape.replace(store_dtype=dtype)
    master = shape.store_dtype == datagen.BF16_MASTER
    cfg = mt.make_config(shape)
    blocks = mt.block_infos(cfg)
    total = mt.host_store_bytes(cfg)
    opt_total = mt.host_opt_bytes(cfg)
    wb = 4 if shape.store_dtype == "f32" else 2
    d, F, V, L = shape.d_model, shape.d_ff, shape.vocab, shape.n_layers
    assert len(blocks) == L + 2
    prev_end = 4096
    prev_opt = 0
    n_params = 0
    for i, b in enumerate(blocks):
        assert b.kind == (mt.MT_BLOCK_EMBED if i == 0 else mt.MT_BLOCK_HEAD if i == L + 1 else mt.MT_BLOCK_LAYER)
        for off in (b.base, b.w_off, b.g_off, b.m_off, b.v_off):
            assert off % 4096 == 0
        # per block: W | G contiguous in the DMA part, m | v (| P) contiguous in the optimizer part
        assert b.base == prev_end == b.w_off
        assert b.g_off == b.w_off + b.w_bytes
        assert b.m_off == prev_opt and b.v_off == b.m_off + b.mv_bytes
        prev_end = b.g_off + b.w_bytes
        prev_opt = b.v_off + b.mv_bytes
        if master:
            assert b.p_off == prev_opt
            prev_opt += b.mv_bytes
        else:
            assert b.p_off == 0
        assert b.w_bytes == b.region_elems * wb and b.mv_bytes == b.region_elems * 4
        end = 0
        for t in range(b.n_tensors):
            tt = b.tensors[t]
            assert (tt.offset * wb) % 4096 == 0 and tt.offset >= end
            end = tt.offset + tt.rows * tt.cols
            n_params += tt.rows * tt.cols
        assert end <= b.region_elems
    assert total == prev_end and opt_total == prev_opt
    assert n_params == shape.n_params()
    b1 = blocks[1]
    shapes = [(b1.tensors[t].rows, b1.tensors[t].cols) for t in range(b1.n_tensors)]
    assert shapes == [(3 * d, d), (d, d), (2 * F, d), (d, F), (1, d), (1, d)]


def test_store_sizes_of_the_14b_shape():
    """Layer weight block 634.4 MB and 186.64 GB store at 12 bytes/param,
    of which 4 bytes/param (W and G) are pinned."""
    cfg = mt.make_config(datagen.PRESETS["14b"])
    blocks = mt.block_infos(cfg)
    assert abs(blocks[1].w_bytes / 1e6 - 634.4) < 0.1
    dma, opt = mt.host_store_bytes(cfg), mt.host_opt_bytes(cfg)
    assert abs((dma + opt) / 1e9 - 186.64) < 0.05
    assert abs(dma / (dma + opt) - 1 / 3) < 1e-3


def test_store_sizes_with_fp32_master():
    """The fp32 master copy adds 4 bytes/param to the pageable part only:
    16 bytes/param, the pinned (streamed) part unchanged."""
    base = mt.make_config(datagen.PRESETS["14b"])
    cfg = mt.make_config(datagen.PRESETS["14b"].replace(store_dtype=datagen.BF16_MASTER))
    assert mt.host_store_bytes(cfg) == mt.host_store_bytes(base)
    assert mt.host_opt_bytes(cfg) * 2 == mt.host_opt_bytes(base) * 3
    assert abs((mt.host_store_bytes(cfg) + mt.host_opt_bytes(cfg)) / 1e9 - 186.64 * 16 / 12) < 0.1


@pytest.mark.parametrize("name,dtype", [("1.3b", datagen.BF16), ("1.3b", datagen.BF16_MASTER), ("tiny", datagen.F32)])
def test_store_layout_with_gradient_accumulator(name, dtype):
    """micro_batches > 1 adds an fp32 accumulator A after m, v (and P) of
    every block in the pageable part; the pinned part is unchanged."""
    shape = datagen.PRESETS[name].replace(store_dtype=dtype)
    base = mt.make_config(shape)
    cfg = mt.make_config(shape, micro_batches=4)
    assert mt.host_store_bytes(cfg) == mt.host_store_bytes(base)
    regions = 3 if dtype == datagen.BF16_MASTER else 2
    assert mt.host_opt_bytes(cfg) * regions == mt.host_opt_bytes(base) * (regions + 1)
    prev = 0
    for b in mt.block_infos(cfg):
        assert b.m_off == prev and b.a_off % 4096 == 0
        last = b.p_off if dtype == datagen.BF16_MASTER else b.v_off
        assert b.a_off == last + b.mv_bytes
        prev = b.a_off + b.mv_bytes
    assert prev == mt.host_opt_bytes(cfg)
    assert all(b.a_off == 0 for b in mt.block_infos(mt.make_config(shape, micro_batches=1)))


def test_config_validation():
    shape = datagen.PRESETS["tiny"]
    bad = [shape.replace(n_heads=3), shape.replace(n_layers=0), shape.replace(vocab=1),
           datagen.PRESETS["1.3b"].replace(head_dim=64, n_heads=32), datagen.PRESETS["1.3b"].replace(d_ff=5500)]
    for s in bad:
        with pytest.raises(mt.MtError):
            mt.host_store_bytes(mt.make_config(s))
    c = mt.make_config(shape)
    c.mode = 7
    with pytest.raises(mt.MtError):
        mt.device_bytes(c)
    for k in (-1, 5000):
        with pytest.raises(mt.MtError):
            mt.host_store_bytes(mt.make_config(shape, micro_batches=k))


SMALL_T256 = datagen.ModelShape("small-bf16-T256", 2, 256, 2, 128, 512, 1000, 2, 256)


def test_token_passes_and_bf16_checkpoints_validation():
    """Token passes: evened out to multiples of 64, each at least 192 tokens;
    only with a bf16 store and without the resident schedule or retained
    layers.  bf16 checkpoints: the same schedule conditions."""
    with pytest.raises(mt.MtError, match="192 tokens"):
        mt.device_bytes(mt.make_config(SMALL_T256, token_chunk=192))  # passes of 192, 192, 128
    with pytest.raises(mt.MtError):
        mt.host_store_bytes(mt.make_config(SMALL_T256, token_chunk=-1))
    with pytest.raises(mt.MtError, match="bf16 store"):
        mt.device_bytes(mt.make_config(datagen.PRESETS["tiny"], token_chunk=64))
    for kw in (dict(mode="resident"), dict(retain_layers=1)):
        with pytest.raises(mt.MtError, match="token passes"):
            mt.device_bytes(mt.make_config(SMALL_T256, token_chunk=256, **kw))
        with pytest.raises(mt.MtError, match="bf16 checkpoints"):
            mt.device_bytes(mt.make_config(SMALL_T256, flags=mt.MT_FLAG_CKPT_BF16, **kw))
    with pytest.raises(mt.MtError, match="bf16 checkpoints"):
        mt.device_bytes(mt.make_config(datagen.PRESETS["tiny"], flags=mt.MT_FLAG_CKPT_BF16))
    # a chunk at least as long as the step, or 0 on a shape that needs no
    # passes, is one pass: the same arena as no chunk at all
    one = mt.device_bytes(mt.make_config(SMALL_T256))
    assert mt.device_bytes(mt.make_config(SMALL_T256, token_chunk=512)) == one
    assert mt.device_bytes(mt.make_config(SMALL_T256, token_chunk=320)) != one  # two passes of 256 (+ fp32 sums)


def test_long_context_arena_with_passes_and_bf16_checkpoints():
    """The 7B width over one sequence: token passes are taken automatically
    once the weight-gradient operands outgrow 32-bit addressing, and keep
    the per-layer workspace at about 76 GB at 512K tokens; bf16 checkpoints
    halve the rest, so 512K fits the device.  The 14B-shape step (one pass)
    holds one more bf16 [tokens x d] buffer than the pass form needs: the
    grouped weight gradients read bf16(dl/dx2) and bf16(dl/dx1) together."""
    GB = 1e9
    s7 = datagen.PRESETS["7b"]
    assert mt.device_bytes(mt.make_config(datagen.PRESETS["14b"])) == 54704961024 + 32768 * 5120 * 2
    for T, fp32_gb, bf16_gb in ((262144, 186.9, 124.6), (524288, 359.2, 234.6)):
        s = s7.replace(batch=1, seq_len=T)
        a = mt.device_bytes(mt.make_config(s)) / GB
        b = mt.device_bytes(mt.make_config(s, flags=mt.MT_FLAG_CKPT_BF16)) / GB
        assert abs(a - fp32_gb) < 0.1 and abs(b - bf16_gb) < 0.1, (T, a, b)
    assert mt.device_bytes(mt.make_config(s7.replace(batch=1, seq_len=524288), flags=mt.MT_FLAG_CKPT_BF16)) < 280 * GB


def test_device_bytes_fit_one_gpu():
    for name in ("1.3b", "7b", "14b"):
        nb = mt.device_bytes(mt.make_config(datagen.PRESETS[name]))
        assert 0 < nb < 200e9, (name, nb)


def test_host_adam_f32_bitwise_equals_oracle():
    rng = np.random.default_rng(1)
    n = 100003
    w = rng.standard_normal(n).astype(np.float32) * 0.02
    g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-9, -1, n)).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v = (rng.random(n) * 1e-5).astype(np.float32)
    for t in (1, 2, 7):
        ow, om, ov = adam_update(w, g, m, v, t, 1e-3, 0.9, 0.95, 1e-8)
        w2, m2, v2 = w.copy(), m.copy(), v.copy()
        mt.check(mt.lib().mt_host_adam(mt.MT_F32, w2.ctypes.data, g.ctypes.data, m2.ctypes.data, v2.ctypes.data, n,
                                       t, 1e-3, 0.9, 0.95, 1e-8, 4))
        assert np.array_equal(w2, ow) and np.array_equal(m2, om) and np.array_equal(v2, ov), t


def test_host_adam_bf16_rounds_the_fp32_update():
    """bf16 store: the fp32 update of the widened values, rounded to nearest
    even, for every one of the 65536 bf16 weight patterns that is finite."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    wf = datagen.bf16_bits_to_f32(bits)
    keep = np.isfinite(wf) & (np.abs(wf) < 1e30)
    bits = bits[keep]
    n = bits.size
    rng = np.random.default_rng(2)
    gbits = datagen.f32_to_bf16_bits((rng.standard_normal(n) * 1e-3).astype(np.float32))
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    w2 = bits.copy()
    mt.check(mt.lib().mt_host_adam(mt.MT_BF16, w2.ctypes.data, gbits.ctypes.data, m.ctypes.data, v.ctypes.data, n,
                                   1, 1e-3, 0.9, 0.95, 1e-8, 3))
    ow, om, ov = adam_update(datagen.bf16_bits_to_f32(bits), datagen.bf16_bits_to_f32(gbits), np.zeros(n, np.float32),
                             np.zeros(n, np.float32), 1, 1e-3, 0.9, 0.95, 1e-8)
    assert np.array_equal(w2, datagen.f32_to_bf16_bits(ow))
    assert np.array_equal(m, om) and np.array_equal(v, ov)


@pytest.mark.parametrize("n", [1, 15, 16, 20, 32, 33, 200, 4099])
@pytest.mark.parametrize("threads", [1, 3])
def test_host_adam_bf16_keeps_subnormal_results(n, threads):
    """Subnormal bf16 weights and results round like every other value,
    wherever the element falls in a vector chunk or the scalar tail: with
    g = 0 the update is exactly 0 and W is unchanged; with the fp32 master
    store, subnormal masters round to their nearest-even bf16 bits."""
    sub = np.concatenate([np.arange(1, 0x80), np.arange(0x8001, 0x8080), [0x0080, 0x8080, 0x0081, 0]])
    bits = np.resize(sub.astype(np.uint16), n)
    g = np.zeros(n, np.uint16)
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    w = bits.copy()
    mt.check(mt.lib().mt_host_adam(mt.MT_BF16, w.ctypes.data, g.ctypes.data, m.ctypes.data, v.ctypes.data, n,
                                   1, 1e-3, 0.9, 0.95, 1e-8, threads))
    assert np.array_equal(w, bits)
    # master: p holds fp32 subnormals between bf16 patterns (ties included)
    rng = np.random.default_rng(n)
    pu = (rng.integers(1, 1 << 23, n, dtype=np.uint32) | (rng.integers(0, 2, n, dtype=np.uint32) << 31))
    pu[::5] = (pu[::5] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)  # exact ties
    p = pu.view(np.float32).copy()
    wm = np.zeros(n, np.uint16)
    m[:] = 0
    v[:] = 0
    mt.check(mt.lib().mt_host_adam_master(wm.ctypes.data, p.ctypes.data, g.ctypes.data, m.ctypes.data,
                                          v.ctypes.data, n, 1, 1e-3, 0.9, 0.95, 1e-8, threads))
    assert np.array_equal(p.view(np.uint32), pu)
    assert np.array_equal(wm, datagen.f32_to_bf16_bits(p))


def _adam_master(w, p, g, m, v, t, lr):
    mt.check(mt.lib().mt_host_adam_master(w.ctypes.data, p.ctypes.data, g.ctypes.data, m.ctypes.data, v.ctypes.data,
                                          w.size, t, lr, 0.9, 0.95, 1e-8, 3))


def test_host_adam_master_is_the_fp32_iteration():
    """fp32 master store: over several steps the master p follows the
    oracle's float32 Adam on float32 weights bit for bit (gradients widened
    from bf16), and w is p rounded to nearest even after every step."""
    rng = np.random.default_rng(3)
    n = 70001
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    w = datagen.f32_to_bf16_bits(p0)
    p = datagen.bf16_bits_to_f32(w).copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    ow, om, ov = p.copy(), m.copy(), v.copy()
    for t in range(1, 6):
        gb = datagen.f32_to_bf16_bits((rng.standard_normal(n) * 10.0 ** rng.uniform(-7, -2, n)).astype(np.float32))
        _adam_master(w, p, gb, m, v, t, 1e-3)
        ow, om, ov = adam_update(ow, datagen.bf16_bits_to_f32(gb), om, ov, t, 1e-3, 0.9, 0.95, 1e-8)
        assert np.array_equal(p, ow) and np.array_equal(m, om) and np.array_equal(v, ov), t
        assert np.array_equal(w, datagen.f32_to_bf16_bits(p)), t


def test_master_keeps_updates_below_bf16_resolution():
    """A constant gradient makes every bias-corrected Adam step lr*g/(|g|+eps)
    (closed form).  At |w| = 0.02 (bf16 spacing 2^-13) steps of lr = 1e-5 are
    below half a bf16 spacing: a bf16 store never moves, while the fp32
    master advances by the sum of the steps and its rounding moves w."""
    n, k, lr = 4096, 60, 1e-5
    w0 = np.full(n, 0.02, np.float32)
    g = np.where(np.arange(n) % 2 == 0, 1e-3, -1e-3).astype(np.float32)
    gb = datagen.f32_to_bf16_bits(g)
    wb = datagen.f32_to_bf16_bits(w0)
    w_bf16 = wb.copy()
    m1, v1 = np.zeros(n, np.float32), np.zeros(n, np.float32)
    w_m, p = wb.copy(), datagen.bf16_bits_to_f32(wb).copy()
    m2, v2 = np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in range(1, k + 1):
        mt.check(mt.lib().mt_host_adam(mt.MT_BF16, w_bf16.ctypes.data, gb.ctypes.data, m1.ctypes.data,
                                       v1.ctypes.data, n, t, lr, 0.9, 0.95, 1e-8, 2))
        _adam_master(w_m, p, gb, m2, v2, t, lr)
    assert np.array_equal(w_bf16, wb)
    gw = datagen.bf16_bits_to_f32(gb).astype(np.float64)
    expect = datagen.bf16_bits_to_f32(wb).astype(np.float64) - k * lr * gw / (np.abs(gw) + 1e-8)
    assert np.max(np.abs(p - expect)) < 1e-7
    assert np.array_equal(w_m, datagen.f32_to_bf16_bits(p))
    assert np.all(w_m != wb)


def test_host_adam_rejects_bad_arguments():
    assert mt.lib().mt_host_adam(5, None, None, None, None, 0, 1, 1e-3, 0.9, 0.95, 1e-8, 1) == mt.MT_E_INVALID
    x = np.zeros(4, np.float32)
    assert mt.lib().mt_host_adam(mt.MT_F32, x.ctypes.data, x.ctypes.data, x.ctypes.data, x.ctypes.data, 4, 0,
                                 1e-3, 0.9, 0.95, 1e-8, 1) == mt.MT_E_INVALID


def test_api_errors_without_device():
    L = mt.lib()
    assert L.mt_train_step(None, None) == mt.MT_E_INVALID
    assert b"null" in L.mt_last_error()
    assert L.mt_get_loss(None, None) == mt.MT_E_INVALID
    cfg = mt.make_config(datagen.PRESETS["tiny"])
    h = ctypes.c_void_p()
    assert L.mt_create_model(ctypes.byref(cfg), None, 0, None, ctypes.byref(h)) == mt.MT_E_INVALID
    assert L.mt_create_model(ctypes.byref(cfg), 0x1001, 1 << 30, None, ctypes.byref(h)) == mt.MT_E_INVALID
    # stream handles are never dereferenced: every call below fails its checks first
    streams = (ctypes.c_void_p * 3)(1, 2, 3)
    one_missing = (ctypes.c_void_p * 3)(1, None, 3)
    repeated = (ctypes.c_void_p * 3)(1, 2, 1)
    assert L.mt_create_model(ctypes.byref(cfg), 0x1000, 1 << 30, one_missing, ctypes.byref(h)) == mt.MT_E_INVALID
    assert L.mt_create_model(ctypes.byref(cfg), 0x1000, 1 << 30, repeated, ctypes.byref(h)) == mt.MT_E_INVALID
    assert b"three different streams" in L.mt_last_error()
    assert L.mt_create_model(ctypes.byref(cfg), 0x1001, 1 << 30, streams, ctypes.byref(h)) == mt.MT_E_ALIGN
    assert L.mt_create_model(ctypes.byref(cfg), 0x1000, 16, streams, ctypes.byref(h)) == mt.MT_E_SIZE
    assert L.mt_debug_grad(None, 0, ctypes.byref(h)) == mt.MT_E_INVALID
    assert L.mt_get_kernel_times(None, None, 0) == mt.MT_E_INVALID
    out = (ctypes.c_double * 3)()
    assert L.mt_link_probe(None, None, None, None, 1 << 20, 2, 0, None, out) == mt.MT_E_INVALID
    assert L.mt_link_probe(0x1000, 0x2000, 0x3000, 0x4000, 0, 2, 0, None, out) == mt.MT_E_INVALID
    assert L.mt_link_probe(0x1000, 0x2000, 0x3000, 0x4000, 1 << 20, 2, 0, None, out) == mt.MT_E_INVALID


def test_host_store_layout_matches_block_info():
    """mt_host_store_layout reports both part sizes and every block's
    descriptor, the same as mt_host_store_bytes / mt_host_opt_bytes /
    mt_block_info; a short capacity fills only that many blocks."""
    for name in ("tiny", "1.3b", "14b"):
        cfg = mt.make_config(datagen.PRESETS[name])
        lay, blocks = mt.store_layout(cfg)
        assert lay.dma_bytes == mt.host_store_bytes(cfg) and lay.opt_bytes == mt.host_opt_bytes(cfg)
        assert lay.n_blocks == cfg.n_layers + 2 == len(blocks)
        for i, b in enumerate(blocks):
            ref = mt.MtBlockDesc()
            mt.check(mt.lib().mt_block_info(ctypes.byref(cfg), i, ctypes.byref(ref)))
            assert bytes(b) == bytes(ref), (name, i)
        few = (mt.MtBlockDesc * 2)()
        mt.check(mt.lib().mt_host_store_layout(ctypes.byref(cfg), ctypes.byref(lay), few, 1))
        assert bytes(few[0]) == bytes(blocks[0]) and not any(bytes(few[1]))
    bad = mt.make_config(datagen.PRESETS["tiny"])
    bad.n_heads = 3
    assert mt.lib().mt_host_store_layout(ctypes.byref(bad), ctypes.byref(mt.MtLayout()), None, 0) == mt.MT_E_INVALID
    assert mt.lib().mt_host_store_layout(ctypes.byref(cfg), None, None, 0) == mt.MT_E_INVALID


def _aligned(nbytes):
    """A 4 KiB-aligned host buffer (numpy-owned) and its address."""
    raw = np.zeros(nbytes + 4096, np.uint8)
    off = (-raw.ctypes.data) % 4096
    buf = raw[off:off + nbytes]
    return raw, buf, buf.ctypes.data


def _plain_store(cfg):
    """Store parts in ordinary host memory, header initialised (no GPU)."""
    n, no = mt.host_store_bytes(cfg), mt.host_opt_bytes(cfg)
    keep_d, dma, pd = _aligned(n)
    keep_o, opt, po = _aligned(no)
    mt.check(mt.lib().mt_init_store_header(ctypes.byref(cfg), pd, n, po, no))
    return (keep_d, keep_o), dma, opt, pd, po, n, no


SMALL_MASTER = datagen.ModelShape("small-bf16m", 2, 256, 2, 128, 512, 1000, 2, 128, store_dtype=datagen.BF16_MASTER)


def test_store_init_master_widens_w():
    cfg = mt.make_config(SMALL_MASTER)
    keep, dma, opt, pd, po, n, no = _plain_store(cfg)
    rng = np.random.default_rng(8)
    blocks = mt.block_infos(cfg)
    for b in blocks:
        dma[b.w_off:b.w_off + b.w_bytes] = rng.integers(0, 256, b.w_bytes, dtype=np.uint8)
    mt.check(mt.lib().mt_store_init_master(pd, n, po, no))
    for b in blocks:
        wbits = dma[b.w_off:b.w_off + b.w_bytes].view(np.uint16)
        pw = opt[b.p_off:b.p_off + b.mv_bytes].view(np.uint32)
        assert np.array_equal(pw, wbits.astype(np.uint32) << np.uint32(16))
        assert not opt[b.m_off:b.v_off + b.mv_bytes].any()
    plain = mt.make_config(SMALL_MASTER.replace(store_dtype=datagen.BF16))
    keep2, _, _, pd2, po2, n2, no2 = _plain_store(plain)
    assert mt.lib().mt_store_init_master(pd2, n2, po2, no2) == mt.MT_E_STATE


@pytest.mark.parametrize("shape", [datagen.PRESETS["tiny"], SMALL_MASTER], ids=["tiny-f32", "small-bf16m"])
def test_store_checkpoint_round_trip(shape, tmp_path):
    """mt_store_save / mt_store_load: W regions, the optimizer part ([m | v],
    with the fp32 master P when there is one) and the step count come back
    bit for bit into a fresh store; gradients are not part of the checkpoint;
    a store of another layout or a short file is rejected."""
    cfg = mt.make_config(shape)
    keep_a, dma_a, opt_a, pa, oa, n, no = _plain_store(cfg)
    rng = np.random.default_rng(5)
    dma_a[4096:] = rng.integers(0, 256, n - 4096, dtype=np.uint8)
    opt_a[:] = rng.integers(0, 256, no, dtype=np.uint8)
    # completed Adam steps: the int64 after magic, version, n_blocks and the config
    step_off = 16 + ctypes.sizeof(mt.MtConfig)
    step_off += (-step_off) % 8
    dma_a[step_off:step_off + 8] = np.frombuffer(np.int64(7).tobytes(), np.uint8)
    t = ctypes.c_int64()
    mt.check(mt.lib().mt_store_step(pa, ctypes.byref(t)))
    assert t.value == 7
    path = str(tmp_path / "ckpt.bin")
    mt.check(mt.lib().mt_store_save(pa, n, oa, no, path.encode()))
    blocks = mt.block_infos(cfg)
    assert os.path.getsize(path) == 8 + 4096 + sum(b.w_bytes for b in blocks) + no

    keep_b, dma_b, opt_b, pb, ob, _, _ = _plain_store(cfg)
    mt.check(mt.lib().mt_store_load(pb, n, ob, no, path.encode()))
    mt.check(mt.lib().mt_store_step(pb, ctypes.byref(t)))
    assert t.value == 7
    for b in blocks:
        assert np.array_equal(dma_b[b.w_off:b.w_off + b.w_bytes], dma_a[b.w_off:b.w_off + b.w_bytes])
        assert not dma_b[b.g_off:b.g_off + b.w_bytes].any()
    assert np.array_equal(opt_b, opt_a)

    other = mt.make_config(shape.replace(d_ff=shape.d_ff * 2))
    keep_c, _, _, pc, oc, nc, noc = _plain_store(other)
    assert mt.lib().mt_store_load(pc, nc, oc, noc, path.encode()) == mt.MT_E_INVALID
    with open(path, "r+b") as f:
        f.truncate(os.path.getsize(path) - 100)
    assert mt.lib().mt_store_load(pb, n, ob, no, path.encode()) == mt.MT_E_INVALID
    assert mt.lib().mt_store_load(pb, n, ob, no, str(tmp_path / "missing.bin").encode()) == mt.MT_E_INVALID


def test_retained_layers_grow_the_arena_by_one_intermediate_set_each():
    """retain_layers = R keeps R more sets of one layer's forward
    intermediates on the device (layer-boundary checkpoints only when 0);
    MT_RESIDENT keeps every layer's already, so R changes nothing there."""
    shape = datagen.PRESETS["14b"]
    b0 = mt.device_bytes(mt.make_config(shape))
    b1 = mt.device_bytes(mt.make_config(shape, retain_layers=1))
    per = b1 - b0
    # h, o, h2 (bf16 [M x d]), qkv (bf16 [M x 3d]), x1 (fp32 [M x d]), gu (bf16 [M x 2F]), y (bf16 [M x F])
    M, d, F = shape.batch * shape.seq_len, shape.d_model, shape.d_ff
    floor = M * d * 2 * 3 + M * 3 * d * 2 + M * d * 4 + M * 2 * F * 2 + M * F * 2
    assert floor <= per <= floor * 1.01, (per, floor)
    for R in (7, 30, shape.n_layers):
        assert mt.device_bytes(mt.make_config(shape, retain_layers=R)) == b0 + R * per
    res = mt.make_config(shape.replace(n_layers=2), mode="resident")
    assert mt.device_bytes(res) == mt.device_bytes(mt.make_config(shape.replace(n_layers=2), mode="resident",
                                                                  retain_layers=2))
    for R in (-1, shape.n_layers + 1):
        with pytest.raises(mt.MtError):
            mt.device_bytes(mt.make_config(shape, retain_layers=R))


def test_stream_k_plan_at_the_14b_shapes():
    """Which GEMMs of the 14B-shape step split their last round of tiles
    along K (planned for 256 persistent workgroups, the MI355X's compute
    units and the count assumed without a GPU): the down and gate/up weight
    gradients (1080 and 2160 tiles: last rounds of 0.22 and 0.44) do; the O
    and QKV weight gradients (tails of 0.56 and 0.69 of a round) and every
    GEMM whose tiles fill whole rounds do not."""
    L = mt.lib()
    M, d, F = 32768, 5120, 13824
    mib = 1 << 20
    assert L.mt_gemm_ws_bytes(d, F, M) == 128 * mib
    assert L.mt_gemm_ws_bytes(2 * F, d, M) == 128 * mib
    for shape in [(d, d, M), (3 * d, d, M), (M, 3 * d, d), (M, d, d), (M, 2 * F, d), (M, d, F), (M, F, d),
                  (M, d, 2 * F), (M, d, 3 * d), (300, 520, 256), (0, 5, 64)]:
        assert L.mt_gemm_ws_bytes(*shape) == 0, shape
