"""Kernel parity on the GPU through the C ABI (include/mt_kernels.h).

References: the definitions the oracle uses (a projection is x @ W.T;
attention, RoPE as in oracle.model), evaluated in float64 on exactly the
bf16 values the kernel reads.  Shapes span several tiles with ragged tails,
and the full 14B-shape projections are checked on sampled outputs.
"""
import ctypes

import numpy as np
import pytest

import datagen
import host_memory_layer_amd as mt
from oracle import attention_bwd, attention_fwd, attention_key_tail, attention_rows, rope_apply, rope_tables

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def bf16_tensor(x_f32):
    """float32 array -> (device uint16 tensor of bf16 bits, float64 values)."""
    bits = datagen.f32_to_bf16_bits(np.ascontiguousarray(x_f32, np.float32))
    t = torch.from_numpy(bits.view(np.int16)).to(dev())
    return t, datagen.bf16_bits_to_f32(bits).astype(np.float64)


def to_f32(t_bits):
    return datagen.bf16_bits_to_f32(t_bits.cpu().numpy().view(np.uint16)).astype(np.float64)


def gemm(dtype, A, lda, B, ldb, C, ldc, M, N, K, epi, R=None, ldr=0, layout=0):
    mt.check(mt.lib().mt_gemm(dtype, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc,
                              R.data_ptr() if R is not None else None, ldr, M, N, K, epi, layout, None))


def acc_bound(a, b):
    """Worst-case fp32 accumulation error of a @ b.T: K * 2^-24 * |a| @ |b|.T."""
    K = a.shape[1]
    return K * 2.0 ** -24 * (np.abs(a) @ np.abs(b).T)


@pytest.mark.parametrize("M,N,K", [(300, 520, 200), (64, 8, 8), (513, 257, 1032), (1, 1, 8),
                                   (300, 520, 256), (513, 257, 1024), (70, 1000, 64), (256, 256, 640)])
def test_gemm_bf16_small(M, N, K):
    rng = np.random.default_rng(M * 7 + N)
    A, a = bf16_tensor(rng.standard_normal((M, K)).astype(np.float32))
    B, b = bf16_tensor(rng.standard_normal((N, K)).astype(np.float32))
    ref = a @ b.T
    bound = acc_bound(a, b)
    # fp32 output
    C = torch.empty((M, N), dtype=torch.float32, device=dev())
    gemm(mt.MT_BF16, A, K, B, K, C, N, M, N, K, mt.EPI_F32)
    torch.cuda.synchronize()
    c = C.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(c - ref) <= bound + 1e-30)
    # bf16 output: the fp32 result rounded to nearest even
    Cb = torch.empty((M, N), dtype=torch.int16, device=dev())
    gemm(mt.MT_BF16, A, K, B, K, Cb, N, M, N, K, mt.EPI_STORE)
    # residual add
    R = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).to(dev())
    Cr = torch.empty((M, N), dtype=torch.float32, device=dev())
    gemm(mt.MT_BF16, A, K, B, K, Cr, N, M, N, K, mt.EPI_ADD_F32, R, N)
    torch.cuda.synchronize()
    cb = Cb.cpu().numpy().view(np.uint16)
    assert np.array_equal(cb, datagen.f32_to_bf16_bits(C.cpu().numpy()))
    cr = Cr.cpu().numpy().astype(np.float64)
    r = R.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(cr - (r + ref)) <= bound + np.abs(r + ref) * 2.0 ** -23 + 1e-30)


@pytest.mark.parametrize("layout", [mt.GEMM_A_KMAJOR, mt.GEMM_B_KMAJOR, mt.GEMM_A_KMAJOR | mt.GEMM_B_KMAJOR])
@pytest.mark.parametrize("M,N,K,pad", [(300, 520, 192, 0), (513, 257, 1024, 8), (256, 256, 640, 0), (70, 1000, 256, 24)])
def test_gemm_bf16_kmajor_operands(layout, M, N, K, pad):
    """K-major operands ([K x M], [K x N], row stride a multiple of 8 >= M
    (N), padding filled with NaN) give the same contraction; ragged M, N leave
    the columns a last tile reads past M (N) out of the stored result."""
    rng = np.random.default_rng(M + 3 * N + K + layout)
    a32 = rng.standard_normal((M, K)).astype(np.float32)
    b32 = rng.standard_normal((N, K)).astype(np.float32)
    up8 = lambda x: (x + 7) // 8 * 8
    if layout & mt.GEMM_A_KMAJOR:
        lda = up8(M) + pad
        buf = np.full((K, lda), np.nan, np.float32)
        buf[:, :M] = a32.T
        A, aw = bf16_tensor(buf)
        a = aw[:, :M].T
    else:
        A, a = bf16_tensor(a32)
        lda = K
    if layout & mt.GEMM_B_KMAJOR:
        ldb = up8(N) + pad
        buf = np.full((K, ldb), np.nan, np.float32)
        buf[:, :N] = b32.T
        B, bw = bf16_tensor(buf)
        b = bw[:, :N].T
    else:
        B, b = bf16_tensor(b32)
        ldb = K
    ref = a @ b.T
    bound = acc_bound(a, b)
    C = torch.full((M, N), np.nan, dtype=torch.float32, device=dev())
    gemm(mt.MT_BF16, A, lda, B, ldb, C, N, M, N, K, mt.EPI_F32, layout=layout)
    Cb = torch.empty((M, N), dtype=torch.int16, device=dev())
    gemm(mt.MT_BF16, A, lda, B, ldb, Cb, N, M, N, K, mt.EPI_STORE, layout=layout)
    torch.cuda.synchronize()
    c = C.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(c - ref) <= bound + 1e-30)
    assert np.array_equal(Cb.cpu().numpy().view(np.uint16), datagen.f32_to_bf16_bits(C.cpu().numpy()))


def test_gemm_kmajor_rejects_unsupported_shapes():
    A = torch.zeros((256, 256), dtype=torch.int16, device=dev())
    C = torch.zeros((256, 256), dtype=torch.float32, device=dev())
    rc = mt.lib().mt_gemm(mt.MT_BF16, A.data_ptr(), 256, A.data_ptr(), 256, C.data_ptr(), 256, None, 0, 256, 256, 128,
                          mt.EPI_F32, mt.GEMM_A_KMAJOR, None)
    assert rc != 0


def test_gemm_bf16_strided_operands():
    """Row strides larger than K (views into wider matrices)."""
    rng = np.random.default_rng(5)
    M, N, K, lda, ldb, ldc = 260, 300, 136, 200, 144, 320
    A, a = bf16_tensor(rng.standard_normal((M, lda)).astype(np.float32))
    B, b = bf16_tensor(rng.standard_normal((N, ldb)).astype(np.float32))
    C = torch.full((M, ldc), 7.0, dtype=torch.float32, device=dev())
    gemm(mt.MT_BF16, A, lda, B, ldb, C, ldc, M, N, K, mt.EPI_F32)
    torch.cuda.synchronize()
    c = C.cpu().numpy().astype(np.float64)
    ref = a[:, :K] @ b[:, :K].T
    assert np.all(np.abs(c[:, :N] - ref) <= acc_bound(a[:, :K], b[:, :K]) + 1e-30)
    assert np.all(c[:, N:] == 7.0)


def test_gemm_f32_small():
    rng = np.random.default_rng(9)
    M, N, K = 130, 77, 45
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((N, K)).astype(np.float32)
    A = torch.from_numpy(a).to(dev())
    B = torch.from_numpy(b).to(dev())
    C = torch.empty((M, N), dtype=torch.float32, device=dev())
    gemm(mt.MT_F32, A, K, B, K, C, N, M, N, K, mt.EPI_STORE)
    torch.cuda.synchronize()
    ref = a.astype(np.float64) @ b.astype(np.float64).T
    assert np.all(np.abs(C.cpu().numpy() - ref) <= acc_bound(a, b) + 1e-30)


# Full-size projections of the 14B shape (32768 tokens, d 5120, F 13824):
# forward QKV, down-projection data gradient, and a weight gradient with
# K = 32768 tokens; 4096 sampled outputs each.
@pytest.mark.parametrize("M,N,K", [(32768, 15360, 5120), (32768, 5120, 13824), (5120, 5120, 32768)])
def test_gemm_bf16_14b_shapes_sampled(M, N, K):
    print(f"gemm {M}x{N}x{K}", flush=True)
    g = torch.Generator(device=dev()).manual_seed(M + N + K)
    A = torch.randn((M, K), generator=g, device=dev(), dtype=torch.float32).to(torch.bfloat16).view(torch.int16)
    B = torch.randn((N, K), generator=g, device=dev(), dtype=torch.float32).to(torch.bfloat16).view(torch.int16)
    C = torch.empty((M, N), dtype=torch.float32, device=dev())
    gemm(mt.MT_BF16, A, K, B, K, C, N, M, N, K, mt.EPI_F32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = rng.integers(0, M, 4096)
    cols = rng.integers(0, N, 4096)
    ri = torch.from_numpy(rows).to(dev())
    ci = torch.from_numpy(cols).to(dev())
    a = to_f32(A[ri])
    b = to_f32(B[ci])
    got = C[ri, ci].cpu().numpy().astype(np.float64)
    ref = np.einsum("ij,ij->i", a, b)
    bound = K * 2.0 ** -24 * np.einsum("ij,ij->i", np.abs(a), np.abs(b))
    assert np.all(np.abs(got - ref) <= bound)
    # typical error far below the worst case
    assert np.sqrt(np.mean((got - ref) ** 2)) < 1e-3 * np.sqrt(np.mean(ref ** 2))


# ---------------------------------------------------------------- attention --
def run_attention(dtype, B, T, H, hd, seed, theta=10000.0):
    rng = np.random.default_rng(seed)
    d = H * hd
    M = B * T
    qkv = (rng.standard_normal((M, 3 * d)) * 1.5).astype(np.float32)
    dO = rng.standard_normal((M, d)).astype(np.float32)
    cos = np.empty((T, hd // 2), np.float32)
    sin = np.empty((T, hd // 2), np.float32)
    mt.check(mt.lib().mt_rope_tables(T, hd, theta, cos.ctypes.data, sin.ctypes.data))
    cos_t = torch.from_numpy(cos).to(dev())
    sin_t = torch.from_numpy(sin).to(dev())
    if dtype == mt.MT_BF16:
        q_dev, qkv64 = bf16_tensor(qkv)
        do_dev, do64 = bf16_tensor(dO)
        et = torch.int16
    else:
        q_dev = torch.from_numpy(qkv).to(dev())
        do_dev = torch.from_numpy(dO).to(dev())
        qkv64, do64 = qkv.astype(np.float64), dO.astype(np.float64)
        et = torch.float32
    ldT = int(mt.lib().mt_token_ld(M))
    assert ldT >= M and ldT % 128 == 0 and (ldT // 128) % 2 == 1
    mt.check(mt.lib().mt_rope_qkv(dtype, q_dev.data_ptr(), cos_t.data_ptr(), sin_t.data_ptr(), B, T, H, hd, None))
    o = torch.empty((M, d), dtype=et, device=dev())
    lse = torch.empty((B * H, T), dtype=torch.float32, device=dev())
    mt.check(mt.lib().mt_attention_fwd(dtype, q_dev.data_ptr(), o.data_ptr(), lse.data_ptr(), B, T, H, hd, None))
    Dsum = torch.empty((B * H, T), dtype=torch.float32, device=dev())
    dqkvT = torch.empty((3 * d, ldT), dtype=et, device=dev())
    mt.check(mt.lib().mt_attention_bwd(dtype, q_dev.data_ptr(), o.data_ptr(), do_dev.data_ptr(), lse.data_ptr(),
                                       Dsum.data_ptr(), dqkvT.data_ptr(), ldT, B, T, H, hd, None))
    torch.cuda.synchronize()
    conv = to_f32 if dtype == mt.MT_BF16 else (lambda t: t.cpu().numpy().astype(np.float64))
    out = dict(qkv=conv(q_dev), qkv_in=qkv64, o=conv(o), lse=lse.cpu().numpy(), dqkvT=conv(dqkvT[:, :M]))
    # oracle in float64 on the values the kernel read
    c64, s64 = rope_tables(T, hd, theta, np.float64)
    heads = lambda x: x.reshape(B, T, H, hd).transpose(0, 2, 1, 3)
    q = rope_apply(heads(qkv64[:, :d]), c64, s64)
    k = rope_apply(heads(qkv64[:, d:2 * d]), c64, s64)
    v = heads(qkv64[:, 2 * d:])
    ref = dict(q=q, k=k, v=v, o=np.empty_like(q), dq=np.empty_like(q), dk=np.empty_like(q), dv=np.empty_like(q))
    dOh = heads(do64)
    for bb in range(B):
        ob, p = attention_fwd(q[bb], k[bb], v[bb])
        ref["o"][bb] = ob
        ref["dq"][bb], ref["dk"][bb], ref["dv"][bb] = attention_bwd(dOh[bb], q[bb], k[bb], v[bb], p)
    return out, ref, heads


def close(got, ref, cos_min, rel_max):
    from tests.harness import cosine, maxnorm_rel
    c, r = cosine(got, ref), maxnorm_rel(got, ref)
    assert c >= cos_min and r <= rel_max, (c, r)


@pytest.mark.parametrize("B,T,H", [(2, 192, 2), (1, 64, 1), (1, 512, 3)])
def test_attention_bf16(B, T, H):
    hd = 128
    d = H * hd
    out, ref, heads = run_attention(mt.MT_BF16, B, T, H, hd, seed=T + H)
    # rotated q, k stored back in qkv; v untouched
    close(heads(out["qkv"][:, :d]), ref["q"], 0.99999, 1e-2)
    close(heads(out["qkv"][:, d:2 * d]), ref["k"], 0.99999, 1e-2)
    assert np.array_equal(out["qkv"][:, 2 * d:], out["qkv_in"][:, 2 * d:])
    close(heads(out["o"]), ref["o"], 0.9999, 2e-2)
    dq = heads(out["dqkvT"][:d].T)
    dk = heads(out["dqkvT"][d:2 * d].T)
    dv = heads(out["dqkvT"][2 * d:].T)
    close(dq, ref["dq"], 0.999, 3e-2)
    close(dk, ref["dk"], 0.999, 3e-2)
    close(dv, ref["dv"], 0.999, 3e-2)


def test_attention_f32():
    B, T, H, hd = 2, 64, 4, 32
    d = H * hd
    out, ref, heads = run_attention(mt.MT_F32, B, T, H, hd, seed=3)
    close(heads(out["o"]), ref["o"], 0.9999999, 1e-5)
    close(heads(out["dqkvT"][:d].T), ref["dq"], 0.9999999, 1e-4)
    close(heads(out["dqkvT"][d:2 * d].T), ref["dk"], 0.9999999, 1e-4)
    close(heads(out["dqkvT"][2 * d:].T), ref["dv"], 0.9999999, 1e-4)


def test_attention_bf16_14b_head_sampled():
    """One (batch, head) pair at the 14B shape's sequence length, T = 4096."""
    out, ref, heads = run_attention(mt.MT_BF16, 1, 4096, 1, 128, seed=11)
    close(heads(out["o"]), ref["o"], 0.9999, 2e-2)
    close(heads(out["dqkvT"][:128].T), ref["dq"], 0.999, 3e-2)
    close(heads(out["dqkvT"][128:256].T), ref["dk"], 0.999, 3e-2)
    close(heads(out["dqkvT"][256:].T), ref["dv"], 0.999, 3e-2)


# Long context: one layer of the 7B shape (32 heads of 128) over a single
# sequence of 65536 or 131072 tokens, so every offset and stride is the real
# one (at 131072 a key row's byte offset inside its head column exceeds 2^31).  Heads 0
# and 31 (the first and the last column block) carry random data, the others
# zeros; the oracle evaluates single query rows and the last keys exactly,
# and two identities cover every key: sum_j dv_j = sum_i dO_i (each
# probability row sums to 1) and sum_j dk_j = 0 (each dS row sums to 0).
@pytest.mark.parametrize("T", [65536, 131072])
def test_attention_bf16_long_context_7b_layer(T):
    B, H, hd = 1, 32, 128
    d = H * hd
    live = (0, 31)
    print(f"attention long context T={T} H={H}", flush=True)
    rng = np.random.default_rng(T)
    qkv = torch.zeros((T, 3 * d), dtype=torch.int16, device=dev())
    dO = torch.zeros((T, d), dtype=torch.int16, device=dev())
    x64, do64 = {}, {}
    for h in live:
        cols = [slice(j * d + h * hd, j * d + (h + 1) * hd) for j in range(3)]
        for j, c in enumerate(cols):
            t, x64[h, j] = bf16_tensor((rng.standard_normal((T, hd)) * 1.5).astype(np.float32))
            qkv[:, c] = t
        t, do64[h] = bf16_tensor(rng.standard_normal((T, hd)).astype(np.float32))
        dO[:, h * hd:(h + 1) * hd] = t
    cos = np.empty((T, hd // 2), np.float32)
    sin = np.empty((T, hd // 2), np.float32)
    mt.check(mt.lib().mt_rope_tables(T, hd, 10000.0, cos.ctypes.data, sin.ctypes.data))
    cos_t, sin_t = torch.from_numpy(cos).to(dev()), torch.from_numpy(sin).to(dev())
    ldT = int(mt.lib().mt_token_ld(T))
    o = torch.empty((T, d), dtype=torch.int16, device=dev())
    lse = torch.empty((H, T), dtype=torch.float32, device=dev())
    Dsum = torch.empty((H, T), dtype=torch.float32, device=dev())
    dqkvT = torch.empty((3 * d, ldT), dtype=torch.int16, device=dev())
    mt.check(mt.lib().mt_rope_qkv(mt.MT_BF16, qkv.data_ptr(), cos_t.data_ptr(), sin_t.data_ptr(), B, T, H, hd, None))
    mt.check(mt.lib().mt_attention_fwd(mt.MT_BF16, qkv.data_ptr(), o.data_ptr(), lse.data_ptr(), B, T, H, hd, None))
    mt.check(mt.lib().mt_attention_bwd(mt.MT_BF16, qkv.data_ptr(), o.data_ptr(), dO.data_ptr(), lse.data_ptr(),
                                       Dsum.data_ptr(), dqkvT.data_ptr(), ldT, B, T, H, hd, None))
    torch.cuda.synchronize()
    # a zero head stays zero: nothing leaks across the column blocks
    quiet = 15
    assert not torch.any(o[:, quiet * hd:(quiet + 1) * hd]).item()
    for j in range(3):
        assert not torch.any(dqkvT[j * d + quiet * hd:j * d + (quiet + 1) * hd, :T]).item()
    c64, s64 = rope_tables(T, hd, 10000.0, np.float64)
    rows = [0, 1, 2, 63, 64, 127, 128, 4095, 4096, 16383, 16384, 32767, 32768, 49151, 65535, 65536, 87381,
            T - 300, T - 1]
    rows = sorted(set(r for r in rows if r < T))
    rows += sorted(np.random.default_rng(1).integers(0, T, 16).tolist())
    tail = 128
    for h in live:
        q = rope_apply(x64[h, 0], c64, s64)
        k = rope_apply(x64[h, 1], c64, s64)
        v = x64[h, 2]
        ro, rdq = attention_rows(q, k, v, do64[h], rows)
        tk, tv = attention_key_tail(q, k, v, do64[h], tail)
        got_o = to_f32(o[:, h * hd:(h + 1) * hd])
        g = [to_f32(dqkvT[j * d + h * hd:j * d + (h + 1) * hd, :T]).T for j in range(3)]
        close(got_o[rows], ro, 0.9999, 2e-2)
        close(g[0][rows], rdq, 0.999, 3e-2)
        close(g[0][T - tail:], attention_rows(q, k, v, do64[h], range(T - tail, T))[1], 0.999, 3e-2)
        close(g[1][T - tail:], tk, 0.999, 3e-2)
        close(g[2][T - tail:], tv, 0.999, 3e-2)
        dv_sum, do_sum = g[2].sum(0), do64[h].sum(0)
        tol = 0.02 * (np.sqrt(np.sum(do64[h] ** 2)) + np.sqrt(np.sum(g[2] ** 2)))
        assert np.linalg.norm(dv_sum - do_sum) <= tol, (np.linalg.norm(dv_sum - do_sum), tol)
        assert np.linalg.norm(g[1].sum(0)) <= 0.02 * np.sqrt(np.sum(g[1] ** 2))


def test_gemm_bf16_kmajor_long_context_sampled():
    """Weight gradient of the 7B QKV projection over 65536 tokens: both
    operands token-major ([K x M] and [K x N]), the first at the largest row
    stride the 32-bit buffer offsets allow (K * lda * 2 < 2^31); one stride
    past the limit is refused."""
    K, M, N = 65536, 12288, 4096
    print(f"gemm kmajor {M}x{N}x{K}", flush=True)
    g = torch.Generator(device=dev()).manual_seed(K + M + N)
    A = torch.randn((K, M), generator=g, device=dev(), dtype=torch.float32).to(torch.bfloat16).view(torch.int16)
    B = torch.randn((K, N), generator=g, device=dev(), dtype=torch.float32).to(torch.bfloat16).view(torch.int16)
    C = torch.empty((M, N), dtype=torch.float32, device=dev())
    gemm(mt.MT_BF16, A, M, B, N, C, N, M, N, K, mt.EPI_F32, layout=mt.GEMM_A_KMAJOR | mt.GEMM_B_KMAJOR)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    ri = torch.from_numpy(rng.integers(0, M, 512)).to(dev())
    ci = torch.from_numpy(rng.integers(0, N, 512)).to(dev())
    a = to_f32(A[:, ri]).T
    b = to_f32(B[:, ci]).T
    got = C[ri, ci].cpu().numpy().astype(np.float64)
    ref = np.einsum("ij,ij->i", a, b)
    bound = K * 2.0 ** -24 * np.einsum("ij,ij->i", np.abs(a), np.abs(b))
    assert np.all(np.abs(got - ref) <= bound)
    assert np.sqrt(np.mean((got - ref) ** 2)) < 1e-3 * np.sqrt(np.mean(ref ** 2))
    del A
    wide = 2 ** 30 // K + 8  # K * wide * 2 >= 2^31
    Aw = torch.zeros((K, wide), dtype=torch.int16, device=dev())
    rc = mt.lib().mt_gemm(mt.MT_BF16, Aw.data_ptr(), wide, B.data_ptr(), N, C.data_ptr(), N, None, 0, 256, N, K,
                          mt.EPI_F32, mt.GEMM_A_KMAJOR | mt.GEMM_B_KMAJOR, None)
    assert rc != 0


# ------------------------------------------------------------ stream-K tail --
def gemm_ws(A, lda, B, ldb, C, ldc, M, N, K, epi, ws, ws_bytes, R=None, ldr=0, layout=0):
    mt.check(mt.lib().mt_gemm_ws(A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc,
                                 R.data_ptr() if R is not None else None, ldr, M, N, K, epi, layout,
                                 ws.data_ptr() if ws is not None else None, ws_bytes, None))


@pytest.mark.parametrize("M,N,K,layout", [(5000, 13800, 32768, 3), (5120, 13824, 32768, 3), (8192, 2304, 8192, 0),
                                          (11008, 2048, 8192, 2)])
def test_gemm_stream_k_tail(M, N, K, layout):
    """A last round of tiles that would leave workgroups idle is split along
    K over every workgroup and summed in K order by a fix-up kernel.  Every
    output stays within the fp32 accumulation bound of the exact contraction
    (float64 on sampled outputs; against the unsplit GEMM everywhere), the
    tiles outside the tail are bit-identical to the unsplit GEMM, the bf16
    and residual epilogues are those of the fp32 sum, and a workspace that
    is too small gives the unsplit GEMM."""
    print(f"stream-K gemm {M}x{N}x{K} layout {layout}", flush=True)
    need = int(mt.lib().mt_gemm_ws_bytes(M, N, K))
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("tile rounds are planned for 256 compute units")
    assert need > 0
    # a tail of more than 0.45 of a round is not split (the 14B O and QKV
    # weight gradients: 400 and 1200 tiles on 256 workgroups)
    assert mt.lib().mt_gemm_ws_bytes(5120, 5120, 32768) == 0 and mt.lib().mt_gemm_ws_bytes(15360, 5120, 32768) == 0
    g = torch.Generator(device=dev()).manual_seed(M + N + K)
    akm, bkm = layout & mt.GEMM_A_KMAJOR, layout & mt.GEMM_B_KMAJOR
    A = torch.randn((K, M) if akm else (M, K), generator=g, device=dev()).to(torch.bfloat16)
    B = torch.randn((K, N) if bkm else (N, K), generator=g, device=dev()).to(torch.bfloat16)
    lda, ldb = (M if akm else K), (N if bkm else K)
    Ai, Bi = A.view(torch.int16), B.view(torch.int16)
    ws = torch.empty(need // 4, dtype=torch.float32, device=dev())
    plain = torch.empty((M, N), dtype=torch.float32, device=dev())
    split = torch.empty((M, N), dtype=torch.float32, device=dev())
    gemm(mt.MT_BF16, Ai, lda, Bi, ldb, plain, N, M, N, K, mt.EPI_F32, layout=layout)
    gemm_ws(Ai, lda, Bi, ldb, split, N, M, N, K, mt.EPI_F32, ws, need, layout=layout)
    # bf16 and residual epilogues of the split sums
    sb = torch.empty((M, N), dtype=torch.int16, device=dev())
    gemm_ws(Ai, lda, Bi, ldb, sb, N, M, N, K, mt.EPI_STORE, ws, need, layout=layout)
    R = torch.randn((M, N), generator=g, device=dev())
    sr = torch.empty((M, N), dtype=torch.float32, device=dev())
    gemm_ws(Ai, lda, Bi, ldb, sr, N, M, N, K, mt.EPI_ADD_F32, ws, need, R=R, ldr=N, layout=layout)
    # too small a workspace: the unsplit GEMM
    small = torch.empty((M, N), dtype=torch.float32, device=dev())
    gemm_ws(Ai, lda, Bi, ldb, small, N, M, N, K, mt.EPI_F32, ws, need - 4, layout=layout)
    torch.cuda.synchronize()
    assert torch.equal(small, plain)
    # |A| |B|^T (fp32 on the device; used only as the error bound)
    a_abs = A.float().abs()
    b_abs = B.float().abs()
    absprod = torch.mm(a_abs.t().contiguous() if akm else a_abs, b_abs if bkm else b_abs.t().contiguous())
    bound = K * 2.0 ** -24 * absprod * 1.001
    diff = (split - plain).abs()
    assert bool((diff <= 2 * bound).all())
    same = float((split == plain).float().mean())
    assert 0.3 < same < 0.999, same  # the tail tiles differ by rounding, the rest is identical
    assert np.array_equal(sb.cpu().numpy().view(np.uint16), datagen.f32_to_bf16_bits(split.cpu().numpy()))
    assert torch.equal(sr, R + split)
    # float64 on sampled outputs
    rng = np.random.default_rng(1)
    rows = torch.from_numpy(rng.integers(0, M, 2048)).to(dev())
    cols = torch.from_numpy(rng.integers(0, N, 2048)).to(dev())
    a = (A[:, rows].t() if akm else A[rows]).float().cpu().numpy().astype(np.float64)
    b = (B[:, cols].t() if bkm else B[cols]).float().cpu().numpy().astype(np.float64)
    ref = np.einsum("ij,ij->i", a, b)
    bnd = K * 2.0 ** -24 * np.einsum("ij,ij->i", np.abs(a), np.abs(b))
    got = split[rows, cols].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= bnd)


# --------------------------------------------------------- grouped GEMM --
def test_gemm_group_is_each_gemm():
    """mt_gemm_group_ws at the 14B weight-gradient shapes (gate/up, down,
    output projection; K = 32768 tokens, both operands K-major): without a
    workspace every product is bit for bit its own mt_gemm_ws; with one, the
    group's last partial round (tiles of the last product) is split along K,
    those outputs stay within the fp32 accumulation bound of the unsplit
    product and the rest is bit-identical; the split result repeats exactly;
    the bf16 epilogue is the fp32 sum rounded."""
    dev()
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("tile rounds are planned for 256 compute units")
    K, d, F = 32768, 5120, 13824
    shapes = [(2 * F, d), (d, F), (d, d)]
    print("grouped gemm " + ", ".join(f"{m}x{n}" for m, n in shapes) + f" K {K}", flush=True)
    g = torch.Generator(device=dev()).manual_seed(7)
    A = [torch.randn((K, m), generator=g, device=dev()).to(torch.bfloat16).view(torch.int16) for m, _ in shapes]
    B = [torch.randn((K, n), generator=g, device=dev()).to(torch.bfloat16).view(torch.int16) for _, n in shapes]
    lay = mt.GEMM_A_KMAJOR | mt.GEMM_B_KMAJOR

    def group(outs, ws, ws_bytes, epi):
        descs = (mt.MtGemmDesc * 3)(*[mt.MtGemmDesc(A[i].data_ptr(), shapes[i][0], B[i].data_ptr(), shapes[i][1],
                                                     outs[i].data_ptr(), shapes[i][1], shapes[i][0], shapes[i][1])
                                      for i in range(3)])
        mt.check(mt.lib().mt_gemm_group_ws(3, descs, K, epi, lay, ws.data_ptr() if ws is not None else None,
                                           ws_bytes, None))
        return descs

    plain = [torch.empty(s, dtype=torch.float32, device=dev()) for s in shapes]
    for i, (m, n) in enumerate(shapes):
        gemm_ws(A[i], m, B[i], n, plain[i], n, m, n, K, mt.EPI_F32, None, 0, layout=lay)
    whole = [torch.empty(s, dtype=torch.float32, device=dev()) for s in shapes]
    descs = group(whole, None, 0, mt.EPI_F32)
    need = int(mt.lib().mt_gemm_group_ws_bytes(3, descs, K))
    assert need > 0  # 3640 tiles: a last round of 56 on 256 workgroups is split
    ws = torch.empty(need // 4, dtype=torch.float32, device=dev())
    split = [torch.empty(s, dtype=torch.float32, device=dev()) for s in shapes]
    again = [torch.empty(s, dtype=torch.float32, device=dev()) for s in shapes]
    group(split, ws, need, mt.EPI_F32)
    group(again, ws, need, mt.EPI_F32)
    sb = [torch.empty(s, dtype=torch.int16, device=dev()) for s in shapes]
    group(sb, ws, need, mt.EPI_STORE)
    torch.cuda.synchronize()
    for i in range(3):
        assert torch.equal(whole[i], plain[i]), i
        assert torch.equal(split[i], again[i]), i
        assert np.array_equal(sb[i].cpu().numpy().view(np.uint16), datagen.f32_to_bf16_bits(split[i].cpu().numpy()))
    assert torch.equal(split[0], plain[0]) and torch.equal(split[1], plain[1])
    absprod = torch.mm(A[2].view(torch.bfloat16).float().abs().t().contiguous(), B[2].view(torch.bfloat16).float().abs())
    diff = (split[2] - plain[2]).abs()
    assert bool((diff <= 2 * K * 2.0 ** -24 * absprod * 1.001).all())
    same = float((split[2] == plain[2]).float().mean())
    assert 0.5 < same < 1.0, same  # 56 of the product's 400 tiles are split
    bad = (mt.MtGemmDesc * 1)(mt.MtGemmDesc(A[0].data_ptr(), 2 * F, B[0].data_ptr(), d, whole[0].data_ptr(), d, 2 * F, d))
    assert mt.lib().mt_gemm_group_ws(0, bad, K, 0, lay, None, 0, None) == mt.MT_E_INVALID
    assert mt.lib().mt_gemm_group_ws(1, bad, K, 2, lay, None, 0, None) == mt.MT_E_INVALID
