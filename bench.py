"""Benchmark of the layer-streamed training step on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 14b]

Runs W untimed and K timed training steps (forward, loss, backward with
recompute, gradient offload and host Adam: the whole step) of the selected
decoder shape with every weight and Adam moment in the pinned host store,
and prints one JSON line: model TFLOPS per step (model FLOPs exclude the
recompute; attention counted over the causal half), the host-link figures,
the GEMM roofline measured with HIP events around every GEMM launch, and
the oracle's throughput on the host cores for a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import datagen  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector

# HBM traffic of the bf16 GEMM at the 14B shape, bytes per launch averaged
# over the 627 launches of a step (the grouped weight-gradient launch counts once): rocprofv3 FETCH_SIZE and WRITE_SIZE,
# scaled by what each reads for a plain 1 GiB copy kernel in the same run
# (profiles/gemm_14b_pmc_traffic.md).  Valid only for the GEMM source it was
# measured on; reported as null once that file changes.
GEMM_TRAFFIC = {"source_sha256_16": "a1c148a5d1caa1b9", "config": "14b", "layers": 48,
                "bytes_per_launch": 10.553e9 + 0.848e9}


def gemm_traffic(shape_name, layers):
    """Measured bytes per GEMM launch, or None when the kernel has changed."""
    import hashlib
    src = os.path.join(ROOT, "host_memory_layer_amd", "csrc", "gemm.hip")
    try:
        h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    t = GEMM_TRAFFIC
    if h != t["source_sha256_16"] or shape_name != t["config"] or layers != t["layers"]:
        return None
    return t["bytes_per_launch"]
PEAK_HBM_GBS = 8000.0


def retained_variant(torch, mt, dev, shape, flags, K, store, tokens, warmup, steps, model_flops_step):
    """The same step with the forward intermediates of as many layers as fit
    in HBM kept on the device, so that their backward skips the recompute
    (results bit for bit those of the full recompute).  Runs on the same
    store after the main measurement."""
    import gc
    gc.collect()
    torch.cuda.empty_cache()
    free = torch.cuda.mem_get_info(dev)[0]
    base = mt.device_bytes(mt.make_config(shape, flags=flags, micro_batches=K))
    per = mt.device_bytes(mt.make_config(shape, flags=flags, micro_batches=K, retain_layers=1)) - base
    R = int(max(0, min(shape.n_layers, (free - base - (8 << 30)) // per)))
    if R == 0:
        return None
    model = mt.Model(mt.make_config(shape, flags=flags, micro_batches=K, retain_layers=R), store, "cuda:0")
    try:
        for _ in range(warmup):
            model.step(tokens)
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        for _ in range(steps):
            model.step(tokens)
            st = model.stats()
        torch.cuda.synchronize(dev)
        elapsed = time.perf_counter() - t0
    finally:
        model.close()
    log(f"retained variant: {R} layers, {elapsed / steps * 1e3:.0f} ms per step")
    return {"retain_layers": R, "arena_gb": (base + R * per) / 1e9, "ms_per_step": elapsed / steps * 1e3,
            "model_tflops": model_flops_step * steps / elapsed / 1e12, "stall_ms": st["stall_ms"],
            "gemm_tflops": st["gemm_flops"] / (st["gemm_ms"] / 1e3) / 1e12 if st["gemm_ms"] > 0 else None}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_shapes(times):
    """Per-shape rates of the last timed step's launches (HIP events around
    each launch on the compute stream; no profiler): GEMMs by (m, n, k,
    epilogue, operand layout), the grouped weight-gradient launches and the
    attention launches by their flop count."""
    groups = {}
    for t in times:
        if t["kind"] == 0:
            key = ("gemm", t["m"], t["n"], t["k"], t["epi"], t["layout"])
        elif t["kind"] == 2:  # the layer's grouped weight gradients (down, gate/up, output projection)
            key = ("gemm_group", t["flops"])
        else:
            key = ("attention", t["flops"])
        g = groups.setdefault(key, [0, 0.0, 0.0])
        g[0] += 1
        g[1] += t["ms"]
        g[2] += t["flops"]
    out = []
    for key, (n, ms, fl) in sorted(groups.items(), key=lambda kv: -kv[1][2]):
        row = {"kind": key[0], "launches": n, "avg_ms": ms / n, "tflops": fl / (ms / 1e3) / 1e12 if ms > 0 else None,
               "frac_of_peak": fl / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS if ms > 0 else None}
        if key[0] == "gemm":
            row.update(m=key[1], n=key[2], k=key[3], epi=key[4], layout=key[5])
        else:
            row.update(flops_per_launch=key[1])
        out.append(row)
    return out


def flops(shape, n_layers=None):
    """(forward flops of one layer, model flops per step, flops the device
    executes per step).  Model flops exclude the recompute and count
    attention over the causal half.  The recompute inside the backward sweep
    runs a layer's forward without its down projection (its output x^{l+1}
    is the checkpoint already held), so the device executes
    fwd_layer - 2*M*d*F more per layer."""
    L = shape.n_layers if n_layers is None else n_layers
    M, d, F, V, B, T = shape.tokens, shape.d_model, shape.d_ff, shape.vocab, shape.batch, shape.seq_len
    fwd_layer = 2.0 * M * (4 * d * d + 3 * d * F) + 2.0 * B * T * T * d
    model = 3.0 * (L * fwd_layer + 2.0 * M * d * V)
    recompute = fwd_layer - 2.0 * M * d * F
    return fwd_layer, model, model + L * recompute


ADAM_BYTES = {datagen.BF16: 22, datagen.BF16_MASTER: 28, datagen.F32: 28}


def host_triad(torch, reps=3):
    """Host DRAM bandwidth of a STREAM-style triad a = b + s*c (float32, 512 MiB
    per array, 12 bytes per element counted) on every core of the affinity
    mask, the threads the host Adam runs on."""
    n_thr = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    prev = torch.get_num_threads()
    torch.set_num_threads(n_thr)
    n = 1 << 27
    a, b, c = torch.empty(n), torch.ones(n), torch.ones(n)
    torch.add(b, c, alpha=0.5, out=a)
    t0 = time.perf_counter()
    for _ in range(reps):
        torch.add(b, c, alpha=0.5, out=a)
    dt = (time.perf_counter() - t0) / reps
    torch.set_num_threads(prev)
    return {"triad_gbs": 12.0 * n / dt / 1e9, "threads": n_thr}


# Layer-block burst sizes (bf16 W region of one layer) of the 1.3B, 7B, 14B
# and 120B shapes.
LINK_SIZES = (101_187_584, 404_774_912, 634_413_056, 2_537_619_456)


def link_peak(mt, reps=4):
    """Host-link GB/s with the library's own copies (mt_link_probe) at the
    layer-block sizes, on the three streams' hipMemcpyAsync and on the SDMA
    engine queues; the peak per direction is the best sustained rate over
    every size and both paths."""
    table = []
    for sdma in (False, True):
        for r in mt.link_probe(LINK_SIZES, reps=reps, sdma=sdma):
            r["path"] = "sdma_queues" if sdma else "hip_streams"
            table.append(r)
    peak = {k: max(r[k] for r in table) for k in ("h2d_gbs", "d2h_gbs", "bidir_gbs")}
    return {**peak, "table": table, "reps": reps}


def host_description():
    """CPU model, threads allowed, and the BLAS numpy uses."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        blas = f"{b.get('name')} {b.get('version', '')}".strip()
    except Exception:  # pragma: no cover - older numpy
        pass
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            blas = f"{blas} ({infos[0].get('internal_api')} {infos[0].get('version')}, " \
                   f"{infos[0].get('num_threads')} threads)"
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "blas": blas}


def cpu_tiny_single_thread():
    """The oracle's whole training step (forward, backward, Adam) of the tiny
    fp32 decoder on one core: seconds and model TFLOPS."""
    from threadpoolctl import threadpool_limits
    from oracle import Oracle
    shape = datagen.PRESETS["tiny"]
    P = datagen.init_params(shape)
    tok = datagen.tokens(shape)
    prev = os.sched_getaffinity(0)
    try:
        os.sched_setaffinity(0, {min(prev)})
        with threadpool_limits(1):
            Oracle(shape, np.float32).step(P, tok)
            t0 = time.perf_counter()
            Oracle(shape, np.float32).step(P, tok)
            dt = time.perf_counter() - t0
    finally:
        os.sched_setaffinity(0, prev)
    return {"seconds": dt, "model_tflops": flops(shape)[1] / dt / 1e12, "threads": 1,
            "workload": "tiny fp32 decoder, 2 x 64 tokens, whole step"}


def cpu_baseline(shape, tokens_sample, seconds_hint):
    """The oracle, as it stands, on one decoder layer of `shape` over one
    sequence of `tokens_sample` tokens: forward, recompute, backward and Adam
    of that layer (float32 NumPy, BLAS on every allowed core)."""
    from oracle import Oracle, adam_update
    sub = shape.replace(n_layers=1, batch=1, seq_len=tokens_sample)
    P = {}
    P["0.attn_norm"] = datagen.init_tensor(sub, "attn_norm")
    P["0.ffn_norm"] = datagen.init_tensor(sub, "ffn_norm")
    for nm in datagen.LAYER_TENSORS:
        P[f"0.{nm}"] = datagen.init_tensor(sub, nm, 0)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((tokens_sample, sub.d_model)).astype(np.float32)
    dx = (rng.standard_normal((tokens_sample, sub.d_model)) * 1e-3).astype(np.float32)
    o = Oracle(sub, np.float32)
    t0 = time.perf_counter()
    _, cache = o.layer_fwd(x, P, 0)          # forward (keeps only x^l in streamed mode)
    _, cache = o.layer_fwd(x, P, 0)          # recompute inside the backward sweep
    grads = {}
    o.layer_bwd(dx, cache, P, 0, grads)
    for k in P:
        adam_update(P[k], grads[k], np.zeros_like(P[k]), np.zeros_like(P[k]), 1, sub.lr, sub.beta1, sub.beta2,
                    sub.adam_eps)
    dt = time.perf_counter() - t0
    fwd_layer = 2.0 * tokens_sample * (4 * sub.d_model ** 2 + 3 * sub.d_model * sub.d_ff) + \
        2.0 * tokens_sample ** 2 * sub.d_model
    model_flops = 3.0 * fwd_layer
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count()
    return {"value": model_flops / dt / 1e12, "unit": "TFLOPS", "cores": cores, "kind": "oracle",
            **host_description(),
            "sample": f"one {shape.name}-shape decoder layer (d {sub.d_model}, F {sub.d_ff}, {sub.n_heads} heads) "
                      f"on 1 x {tokens_sample} tokens: forward + recompute + backward + Adam, float32 NumPy; "
                      f"{dt:.1f} s",
            "seconds": dt}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="14b", choices=list(datagen.PRESETS))
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (same per-layer shape)")
    ap.add_argument("--batch", type=int, default=0, help="override the batch size")
    ap.add_argument("--seq-len", type=int, default=0, help="override the sequence length (long context)")
    ap.add_argument("--mode", default="streamed", choices=["streamed", "serialized", "resident", "single_slot"])
    ap.add_argument("--micro-batches", type=int, default=1,
                    help="gradient accumulation: this many micro-batches of the configured batch per step")
    ap.add_argument("--fp32-master", action="store_true",
                    help="keep an fp32 master copy of the weights beside the Adam moments (bf16 still streamed)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--duplex-link", action="store_true",
                    help="let prefetches and offloads use the host link at the same time")
    ap.add_argument("--retain-layers", default="0",
                    help="layers that keep their forward intermediates on the device, so that their backward "
                         "skips the recompute (bit-identical results): a count, or 'auto' for as many as fit in "
                         "HBM; 0 (default) recomputes every layer from its layer-boundary checkpoint")
    ap.add_argument("--retained-variant", action="store_true",
                    help="after the measurement, run the same step with as many layers' forward intermediates kept "
                         "on the device as fit (their backward skips the recompute)")
    ap.add_argument("--sdma-queues", action="store_true",
                    help="prefetches and offloads on two SDMA engine queues fed by host threads instead of "
                         "hipMemcpyAsync on the prefetch and offload streams")
    ap.add_argument("--no-link-probe", action="store_true")
    ap.add_argument("--token-chunk", type=int, default=0,
                    help="tokens per pass of a layer's per-token work (0: automatic, passes only where needed)")
    ap.add_argument("--ckpt-bf16", action="store_true",
                    help="keep the layer-boundary checkpoints in bf16 (long contexts)")
    ap.add_argument("--progress", action="store_true",
                    help="print a line to stderr as each block use of a step finishes (steps that take minutes)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run a plain 1 GiB device copy kernel first (the reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; the multi-GPU path is design-only",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import host_memory_layer_amd as mt

    shape = datagen.PRESETS[args.config]
    if args.layers:
        shape = shape.replace(n_layers=args.layers)
    if args.batch:
        shape = shape.replace(batch=args.batch)
    if args.seq_len:
        shape = shape.replace(seq_len=args.seq_len)
    if args.fp32_master:
        shape = shape.replace(store_dtype=datagen.BF16_MASTER)
    dev = torch.device("cuda:0")
    flags = 0 if args.no_kernel_timing else mt.MT_FLAG_TIME_KERNELS
    if args.duplex_link:
        flags |= mt.MT_FLAG_DUPLEX_LINK
    if args.sdma_queues:
        flags |= mt.MT_FLAG_SDMA_QUEUES
    if args.ckpt_bf16:
        flags |= mt.MT_FLAG_CKPT_BF16
    if args.progress:
        flags |= mt.MT_FLAG_PROGRESS
    K = max(1, args.micro_batches)
    cfg = mt.make_config(shape, mode=args.mode, flags=flags, micro_batches=K, token_chunk=args.token_chunk)
    R = 0
    if args.retain_layers == "auto":
        # as many sets of one layer's intermediates as fit beside the arena,
        # with 8 GiB left for the runtime and torch
        free = torch.cuda.mem_get_info(dev)[0]
        base = mt.device_bytes(cfg)
        per = mt.device_bytes(mt.make_config(shape, mode=args.mode, flags=flags, micro_batches=K,
                                             retain_layers=1)) - base
        R = int(max(0, min(shape.n_layers, (free - base - (8 << 30)) // per)))
    elif int(args.retain_layers):
        R = int(args.retain_layers)
    if R:
        cfg = mt.make_config(shape, mode=args.mode, flags=flags, micro_batches=K, retain_layers=R)
        log(f"retaining the forward intermediates of {R} of {shape.n_layers} layers on the device")

    t0 = time.perf_counter()
    store = mt.HostStore(cfg)
    log(f"host store: pinned W|G part {store.nbytes / 1e9:.2f} GB, pageable m|v part "
        f"{store.opt_nbytes / 1e9:.2f} GB, in {time.perf_counter() - t0:.1f} s")
    t0 = time.perf_counter()
    mt.init_store_weights(store, datagen.store_filler(shape))
    log(f"initialised weights in {time.perf_counter() - t0:.1f} s")
    model = mt.Model(cfg, store, "cuda:0")
    log(f"device arena {model.arena.numel() / 1e9:.2f} GB")
    link = None if args.no_link_probe else link_peak(mt)
    if link:
        for r in link["table"]:
            log(f"host link {r['path']:11s} {r['bytes'] / 1e6:8.1f} MB: H2D {r['h2d_gbs']:.2f} D2H {r['d2h_gbs']:.2f} "
                f"both {r['bidir_gbs']:.2f} GB/s")
    dram = host_triad(torch)
    log(f"host DRAM: {dram}")
    tokens = datagen.tokens(shape.replace(batch=K * shape.batch))
    if args.copy_probe:
        # 1 GiB read + 1 GiB written per launch: what FETCH_SIZE / WRITE_SIZE
        # read for this kernel calibrates those counters to bytes
        a = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize(dev)
        del a, b
        log("copy probe: 3 x torch.neg over 1 GiB")

    for i in range(args.warmup):
        t0 = time.perf_counter()
        loss = model.step(tokens)
        log(f"warmup step {i}: loss {loss:.4f} {time.perf_counter() - t0:.2f} s")
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    gemm_ms = gemm_fl = gemm_by = attn_ms = attn_fl = 0.0
    gemm_n = 0
    st_acc = []
    for i in range(args.steps):
        loss = model.step(tokens)
        st = model.stats()
        st_acc.append(st)
        gemm_ms += st["gemm_ms"]
        gemm_fl += st["gemm_flops"]
        gemm_by += st["gemm_bytes"]
        gemm_n += st["gemm_launches"]
        attn_ms += st["attn_ms"]
        attn_fl += st["attn_flops"]
        log(f"step {i}: loss {loss:.4f} step {st['step_ms']:.0f} ms device {st['device_ms']:.0f} ms "
            f"stall {st['stall_ms']:.1f} ms adam {st['adam_ms']:.0f} ms (tail {st['adam_tail_ms']:.0f})")
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    kshapes = kernel_shapes(model.kernel_times()) if flags & mt.MT_FLAG_TIME_KERNELS else None

    fwd_layer, model_flops, hw_flops = flops(shape)
    hw_flops -= R * (fwd_layer - 2.0 * shape.tokens * shape.d_model * shape.d_ff)  # retained layers skip their recompute
    value = K * model_flops * args.steps / elapsed / 1e12
    last = st_acc[-1]
    L = shape.n_layers
    per_layer = [model.block_stats(j) for j in range(1, L + 1)]
    mid = per_layer[1:-1] or per_layer
    comp_f = float(np.mean([b["fwd_ms"] for b in mid]))
    comp_b = float(np.mean([b["bwd_ms"] for b in mid]))
    h2d_f = float(np.mean([b["h2d_fwd_ms"] for b in mid]))
    h2d_b = float(np.mean([b["h2d_bwd_ms"] for b in mid]))
    d2h = float(np.mean([b["d2h_ms"] for b in mid]))
    h2d_gbs = last["h2d_bytes"] / (last["h2d_ms"] / 1e3) / 1e9 if last["h2d_ms"] > 0 else None
    d2h_gbs = last["d2h_bytes"] / (last["d2h_ms"] / 1e3) / 1e9 if last["d2h_ms"] > 0 else None
    bf = shape.store_dtype != datagen.F32
    roof = None
    if gemm_ms > 0:
        achieved = gemm_fl / (gemm_ms / 1e3) / 1e12
        peak = PEAK_BF16_TFLOPS if bf else PEAK_F32_TFLOPS
        roof = {"bound": "mfma" if bf else "alu", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": gemm_traffic(args.config, L), "kernel": "k_gemm_bf16 (all launches)",
                "launches_per_step": gemm_n / args.steps,
                "flops_per_launch": gemm_fl / max(gemm_n, 1),
                "algorithmic_bytes_per_launch": gemm_by / max(gemm_n, 1),
                "avg_launch_ms": gemm_ms / max(gemm_n, 1)}
    cpu = None
    if not args.no_cpu_baseline:
        log("oracle CPU baseline ...")
        cpu = cpu_baseline(shape, args.cpu_tokens, 20)
        cpu["tiny_step_single_thread"] = cpu_tiny_single_thread()
        log(f"oracle: {cpu}")
    out = {
        "metric": "model TFLOPS/step on 1 MI355X (14B-shape) + H2D GB/s vs host-link peak",
        "value": value,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic",
        "config": {"workload": f"{shape.name}-shape decoder: {L} layers, d {shape.d_model}, "
                               f"{shape.n_heads}x{shape.head_dim} heads, SwiGLU {shape.d_ff}, vocab {shape.vocab}; "
                               f"batch {shape.batch} x seq {shape.seq_len}"
                               f"{f' x {K} micro-batches' if K > 1 else ''}; {args.mode} from the host store"
                               f"{f', forward intermediates of {R} layers kept on the device' if R else ''}"
                               f"{', bf16 layer-boundary checkpoints' if args.ckpt_bf16 else ''} "
                               f"({store.nbytes / 1e9:.1f} GB pinned W/G + {store.opt_nbytes / 1e9:.1f} GB "
                               f"Adam m/v{' + fp32 master W' if args.fp32_master else ''})",
                   "global_batch": K * shape.batch, "seq_len": shape.seq_len, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "detail": {
            "retain_layers": R,
            "model_flops_per_step": K * model_flops, "hw_flops_per_step": K * hw_flops,
            "hw_tflops": K * hw_flops * args.steps / elapsed / 1e12,
            "device_ms": last["device_ms"], "step_ms": last["step_ms"], "loss": loss,
            "h2d_gbs_achieved": h2d_gbs, "d2h_gbs_achieved": d2h_gbs,
            "transfers": "sdma_queues" if args.sdma_queues else "hip_streams",
            "link_peak": link,
            "h2d_frac_of_link_peak": h2d_gbs / link["h2d_gbs"] if h2d_gbs and link else None,
            "d2h_frac_of_link_peak": d2h_gbs / link["d2h_gbs"] if d2h_gbs and link else None,
            "stall_ms": last["stall_ms"], "adam_ms": last["adam_ms"], "adam_tail_ms": last["adam_tail_ms"],
            "host_dram": dram,
            # bytes the host Adam moves per parameter: bf16 store W, G, m, v in and W, m, v out (22);
            # fp32 master or fp32 store 28 (gradient accumulation adds more and is not counted here)
            "adam_gbs": (ADAM_BYTES[shape.store_dtype] * shape.n_params() / (last["adam_ms"] / 1e3) / 1e9
                         if K == 1 and last["adam_ms"] > 0 else None),
            "per_layer_ms": {"fwd_compute": comp_f, "bwd_compute": comp_b, "h2d_fwd": h2d_f, "h2d_bwd": h2d_b,
                             "d2h": d2h},
            "attention": {"ms_per_step": attn_ms / args.steps,
                          "tflops": attn_fl / (attn_ms / 1e3) / 1e12 if attn_ms > 0 else None},
            "kernel_shapes": kshapes,
        },
    }
    model.close()
    if R == 0 and args.mode == "streamed" and args.retained_variant and not args.copy_probe:
        out["detail"]["retained_variant"] = retained_variant(torch, mt, dev, shape, flags, K, store, tokens,
                                                             args.warmup, args.steps, K * model_flops)
    store.free()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
