"""Memory-bound kernels against the oracle's definitions, through the C ABI
(transpose) and through whole-step parity (RMSNorm, SwiGLU, RoPE run inside
every layer; their own checks are in test_gpu_step and test_gpu_kernels)."""
import numpy as np
import pytest

import host_memory_layer_amd as mt

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.mark.parametrize("R,C,ld_in,ld_out", [(64, 64, 64, 64), (200, 136, 144, 208), (8, 8, 8, 8),
                                              (130, 70, 70, 130), (4096, 5120, 5120, 4224)])
def test_transpose_exact(R, C, ld_in, ld_out):
    rng = np.random.default_rng(R + C)
    a = rng.integers(0, 65535, (R, ld_in), dtype=np.uint16)
    A = torch.from_numpy(a.view(np.int16)).to(dev())
    O = torch.full((C, ld_out), -1, dtype=torch.int16, device=dev())
    mt.check(mt.lib().mt_transpose(mt.MT_BF16, A.data_ptr(), ld_in, O.data_ptr(), ld_out, R, C, None))
    torch.cuda.synchronize()
    o = O.cpu().numpy().view(np.uint16)
    assert np.array_equal(o[:, :R], a[:, :C].T)
    assert np.all(o[:, R:] == 0xFFFF)


# --------------------------------------------------------------------------
# The memory-bound kernels of a layer at the 14B shape (32768 tokens, d 5120,
# F 13824, V 32000, sequences of 4096) and at small ragged shapes, through
# the C ABI, against the oracle's functions evaluated in float64 on exactly
# the values the kernel read.  Bounds follow from fp32 arithmetic: a sum of
# n terms is within n * 2^-24 of its exact value relative to the sum of
# magnitudes, and a bf16 result within one bf16 unit (2^-8 relative) of the
# exact value, since the fp32 value it rounds may sit on either side of a
# rounding boundary.
import datagen  # noqa: E402
from oracle import rmsnorm_bwd, rmsnorm_fwd, rope_apply, rope_tables, silu, silu_grad  # noqa: E402

U = 2.0 ** -24   # fp32 unit roundoff
UB = 2.0 ** -8   # one bf16 unit, relative


def _bits_to_f64(t):
    return datagen.bf16_bits_to_f32(t.cpu().numpy().view(np.uint16)).astype(np.float64)


def _bf16_dev(a_f32):
    """(device bf16 tensor, host bf16 bits) of a float32 array."""
    bits = datagen.f32_to_bf16_bits(np.ascontiguousarray(a_f32, np.float32))
    return torch.from_numpy(bits.view(np.int16)).to(dev()), bits


def _f64(bits):
    return datagen.bf16_bits_to_f32(bits).astype(np.float64)


def _rows(M, n, seed):
    """n sampled rows of M: both ends and random ones."""
    rng = np.random.default_rng(seed)
    r = np.concatenate([[0, 1, M - 2, M - 1], rng.integers(0, M, n)])
    return np.unique(r[(r >= 0) & (r < M)])


def _tiled_normal(rows, cols, period, seed, scale=1.0):
    """[rows x cols] float32: `period` random rows repeated, each repeat
    scaled by its own factor (so rows differ in magnitude)."""
    rng = np.random.default_rng(seed)
    base = rng.standard_normal((period, cols), dtype=np.float32) * np.float32(scale)
    reps = -(-rows // period)
    f = rng.uniform(0.25, 4.0, reps).astype(np.float32)
    return (base[None] * f[:, None, None]).reshape(-1, cols)[:rows]


@pytest.mark.parametrize("M,d", [(32768, 5120), (37, 136), (1, 4096)])
def test_rmsnorm_fwd_bwd_against_oracle(M, d):
    eps = 1e-5
    x = _tiled_normal(M, d, 512, 1)
    g_dev, g = _bf16_dev(1.0 + 0.1 * np.random.default_rng(2).standard_normal(d).astype(np.float32))
    g = _f64(g)
    X = torch.from_numpy(x).to(dev())
    Y = torch.empty((M, d), dtype=torch.int16, device=dev())
    R = torch.empty(M, dtype=torch.float32, device=dev())
    mt.check(mt.lib().mt_rmsnorm_fwd(mt.MT_BF16, X.data_ptr(), g_dev.data_ptr(), Y.data_ptr(), R.data_ptr(), M, d,
                                     eps, None))
    dy = _tiled_normal(M, d, 384, 3, 1e-3)
    res = _tiled_normal(M, d, 256, 4)
    DY, RES = torch.from_numpy(dy).to(dev()), torch.from_numpy(res).to(dev())
    DX = torch.empty((M, d), dtype=torch.float32, device=dev())
    DXL = torch.empty((M, d), dtype=torch.int16, device=dev())
    DG = torch.empty(d, dtype=torch.int16, device=dev())
    WS = torch.empty(mt.lib().mt_rmsnorm_bwd_ws_bytes(M, d) // 4, dtype=torch.float32, device=dev())
    mt.check(mt.lib().mt_rmsnorm_bwd(mt.MT_BF16, DY.data_ptr(), X.data_ptr(), g_dev.data_ptr(), R.data_ptr(),
                                     RES.data_ptr(), DX.data_ptr(), DXL.data_ptr(), DG.data_ptr(), WS.data_ptr(), M, d,
                                     None))
    torch.cuda.synchronize()
    r_gpu = R.cpu().numpy().astype(np.float64)
    rows = _rows(M, 300, M + d)
    x64 = x[rows].astype(np.float64)
    y_ref, r_ref = rmsnorm_fwd(x64, g, eps)
    # rstd: mean of d squares in fp32, then 1/sqrt
    assert np.all(np.abs(r_gpu[rows] - r_ref[:, 0]) <= r_ref[:, 0] * (0.5 * (d + 2) * U + 4 * U))
    y = _bits_to_f64(Y)[rows]
    assert np.all(np.abs(y - y_ref) <= UB * np.abs(y_ref) + 1e-30)
    # backward with the kernel's own rstd as input (the forward's output)
    dy64, res64 = dy[rows].astype(np.float64), res[rows].astype(np.float64)
    r64 = r_gpu[rows][:, None]
    dx_ref, _ = rmsnorm_bwd(dy64, x64, g, r64)
    dx_ref = dx_ref + res64
    xh = np.abs(x64 * r64)
    mean_abs = np.mean(np.abs(dy64 * g) * xh, axis=-1, keepdims=True)
    bound = r64 * (4 * U * np.abs(dy64 * g) + xh * (d + 4) * U * mean_abs) + 2 * U * np.abs(dx_ref) + 1e-30
    dx = DX.cpu().numpy()
    assert np.all(np.abs(dx[rows] - dx_ref) <= bound)
    assert np.array_equal(DXL.cpu().numpy().view(np.uint16), datagen.f32_to_bf16_bits(dx))
    # gain gradient: sum over every row of dy * x * rstd
    terms = dy.astype(np.float64) * (x.astype(np.float64) * r_gpu[:, None])
    dg_ref = terms.sum(axis=0)
    dg = _bits_to_f64(DG)
    assert np.all(np.abs(dg - dg_ref) <= UB * np.abs(dg_ref) + (M + 8) * 2 * U * np.abs(terms).sum(axis=0) + 1e-30)


@pytest.mark.parametrize("M,d", [(32768, 5120), (37, 136), (1, 4096)])
def test_rmsnorm_fwd_with_residual_is_the_add_then_the_norm(M, d):
    """mt_rmsnorm_fwd_res: x becomes res + x, the fp32 add, bit for bit; y and
    rstd are bit for bit those of mt_rmsnorm_fwd on that sum (whose parity
    with the oracle the test above checks)."""
    eps = 1e-5
    res = _tiled_normal(M, d, 512, 7)
    prod = _tiled_normal(M, d, 384, 8, 0.3)
    g_dev, _ = _bf16_dev(1.0 + 0.1 * np.random.default_rng(9).standard_normal(d).astype(np.float32))
    RES, X = torch.from_numpy(res).to(dev()), torch.from_numpy(prod).to(dev())
    Y, Y2 = (torch.empty((M, d), dtype=torch.int16, device=dev()) for _ in range(2))
    R, R2 = (torch.empty(M, dtype=torch.float32, device=dev()) for _ in range(2))
    mt.check(mt.lib().mt_rmsnorm_fwd_res(mt.MT_BF16, RES.data_ptr(), X.data_ptr(), g_dev.data_ptr(), Y.data_ptr(),
                                         R.data_ptr(), M, d, eps, None))
    SUM = torch.from_numpy(res + prod).to(dev())  # numpy float32 add: round to nearest
    mt.check(mt.lib().mt_rmsnorm_fwd(mt.MT_BF16, SUM.data_ptr(), g_dev.data_ptr(), Y2.data_ptr(), R2.data_ptr(), M, d,
                                     eps, None))
    torch.cuda.synchronize()
    assert np.array_equal(X.cpu().numpy().view(np.uint32), (res + prod).view(np.uint32))
    assert torch.equal(Y, Y2)
    assert torch.equal(R.view(torch.int32), R2.view(torch.int32))


@pytest.mark.parametrize("M,F", [(32768, 13824), (33, 520), (3, 12)])
def test_swiglu_fwd_bwd_against_oracle(M, F):
    GU, gu_bits = _bf16_dev(_tiled_normal(M, 2 * F, 64, 5, 2.0))
    DYb, dy_bits = _bf16_dev(_tiled_normal(M, F, 48, 6, 1e-2))
    Y = torch.empty((M, F), dtype=torch.int16, device=dev())
    DGU = torch.empty((M, 2 * F), dtype=torch.int16, device=dev())
    mt.check(mt.lib().mt_swiglu_fwd(mt.MT_BF16, GU.data_ptr(), Y.data_ptr(), M, F, None))
    mt.check(mt.lib().mt_swiglu_bwd(mt.MT_BF16, DYb.data_ptr(), GU.data_ptr(), DGU.data_ptr(), M, F, None))
    torch.cuda.synchronize()
    rows = _rows(M, 200, M + F) if M > 8 else np.arange(M)
    gu64, e = _f64(gu_bits[rows]), _f64(dy_bits[rows])
    g, u = gu64[:, :F], gu64[:, F:]
    y_ref = silu(g) * u
    y = _bits_to_f64(Y)[rows]
    # fp32 exponential and division: a few units of 2^-24; then bf16 rounding
    assert np.all(np.abs(y - y_ref) <= UB * np.abs(y_ref) + 16 * U * np.abs(silu(g) * u) + 1e-30)
    s = 1 / (1 + np.exp(-g))
    dg_ref = e * u * silu_grad(g)
    du_ref = e * silu(g)
    dgu = _bits_to_f64(DGU)[rows]
    # silu'(g) = s (1 + g (1 - s)) cancels near g = -1.28: bound by its terms
    scale_g = np.abs(e * u) * s * (1 + np.abs(g) * (1 - s))
    assert np.all(np.abs(dgu[:, :F] - dg_ref) <= UB * np.abs(dg_ref) + 32 * U * scale_g + 1e-30)
    assert np.all(np.abs(dgu[:, F:] - du_ref) <= UB * np.abs(du_ref) + 16 * U * np.abs(du_ref) + 1e-30)


@pytest.mark.parametrize("B,T,H", [(8, 4096, 40), (3, 64, 2)])
def test_rope_bwd_transposed_against_oracle(B, T, H):
    """Inverse rotation of the dq, dk rows of dqkvT [3d x ldT] at the
    attention backward's padded row stride; dv rows and the padding columns
    untouched.  Each output is a_i cos +- b_i sin in fp32 (error within
    2 * 2^-24 (|a_i| + |b_i|)), then rounded to bf16."""
    hd = 128
    d, M, h = H * hd, B * T, hd // 2
    ldT = mt.lib().mt_token_ld(M)
    cos, sin = rope_tables(T, hd, 10000.0, np.float32)
    cosT = torch.from_numpy(np.ascontiguousarray(cos.T)).to(dev())
    sinT = torch.from_numpy(np.ascontiguousarray(sin.T)).to(dev())
    A, a_bits = _bf16_dev(_tiled_normal(3 * d, ldT, 96, 7))
    before = A.clone()
    mt.check(mt.lib().mt_rope_bwd_t(mt.MT_BF16, A.data_ptr(), ldT, cosT.data_ptr(), sinT.data_ptr(), B, T, H, hd,
                                    None))
    torch.cuda.synchronize()
    cols = _rows(M, 64, B * H)
    got = _bits_to_f64(A[:, torch.as_tensor(cols, device=dev())])   # [3d x n]
    a = _f64(a_bits[:, cols])
    t = cols % T
    c64, s64 = cos[t].astype(np.float64), sin[t].astype(np.float64)  # [n x hd/2]
    for part in (0, 1):                           # dq rows, then dk rows
        x = a[part * d:(part + 1) * d].T.reshape(len(cols), H, hd).transpose(1, 0, 2)   # [H, n, hd]
        ref = rope_apply(x, c64, s64, inverse=True)
        mag = np.abs(x[..., :h]) + np.abs(x[..., h:])
        mag = np.concatenate([mag, mag], axis=-1)
        out = got[part * d:(part + 1) * d].T.reshape(len(cols), H, hd).transpose(1, 0, 2)
        assert np.all(np.abs(out - ref) <= UB * np.abs(ref) + 4 * U * mag + 1e-30), part
    assert torch.equal(A[2 * d:], before[2 * d:])
    if ldT > M:
        assert torch.equal(A[:, M:], before[:, M:])


@pytest.mark.parametrize("rows,row0,T,V", [(8192, 8000, 4096, 32000), (300, 7, 64, 1000)])
def test_xent_rows_against_oracle(rows, row0, T, V):
    """Loss rows and bf16 logit gradients of a pass of `rows` token rows
    starting at row0 (sequence ends inside the pass)."""
    from oracle import cross_entropy
    M = row0 + rows + 1
    rng = np.random.default_rng(rows + V)
    tok = rng.integers(0, V, M, dtype=np.int32)
    z = _tiled_normal(rows, V, 128, 8, 3.0)
    Z = torch.from_numpy(z).to(dev())
    TOK = torch.from_numpy(tok).to(dev())
    RL = torch.full((M,), -1.0, dtype=torch.float32, device=dev())
    DL = torch.empty((rows, V), dtype=torch.int16, device=dev())
    inv_n = np.float32(1.0 / (M - M // T))
    mt.check(mt.lib().mt_xent(mt.MT_BF16, Z.data_ptr(), TOK.data_ptr(), RL.data_ptr(), DL.data_ptr(), rows, row0, T,
                              V, float(inv_n), None))
    torch.cuda.synchronize()
    rl = RL.cpu().numpy()
    assert np.all(rl[:row0] == -1.0) and np.all(rl[row0 + rows:] == -1.0)
    ends = [i for i in range(rows) if (row0 + i) % T == T - 1]
    assert ends, "the pass must hold a sequence end"
    pick = np.unique(np.concatenate([[0, rows - 1], ends, np.array(ends) - 1, rng.integers(0, rows, 40)]))
    pick = pick[(pick >= 0) & (pick < rows)]
    dl = DL[torch.as_tensor(pick, device=dev())]
    dl = _bits_to_f64(dl)
    for k, i in enumerate(pick):
        m = row0 + i
        if m % T == T - 1:
            assert rl[m] == 0.0 and not np.any(dl[k])
            continue
        # the oracle's loss of one labelled row: a two-position window whose
        # second position carries no label
        loss, g = cross_entropy(z[i][None, None].astype(np.float64).repeat(2, axis=1),
                                np.array([[tok[m], tok[m + 1]]]))
        assert abs(rl[m] - loss) <= 1e-5 * abs(loss) + 64 * U * np.log(V), (m, rl[m], loss)
        ref = g[0, 0] * np.float64(inv_n)
        # the softmax sum over V terms (fp32, per-thread runs then a tree)
        # carries a relative error of a few hundred 2^-24; p - 1 on the label
        # makes it absolute
        assert np.all(np.abs(dl[k] - ref) <= UB * np.abs(ref) + 512 * U * float(inv_n)), m


@pytest.mark.parametrize("M,V,d", [(32768, 32000, 5120), (40, 17, 8)])
def test_embedding_fwd_bwd_exact(M, V, d):
    rng = np.random.default_rng(M + d)
    tok = rng.integers(0, V, M, dtype=np.int32)
    tok[: min(M, 64)] = tok[0]  # a token repeated many times
    Eb, E_bits = _bf16_dev(_tiled_normal(V, d, 97, 9, 0.02))
    TOK = torch.from_numpy(tok).to(dev())
    X = torch.empty((M, d), dtype=torch.float32, device=dev())
    mt.check(mt.lib().mt_embed_fwd(mt.MT_BF16, TOK.data_ptr(), Eb.data_ptr(), X.data_ptr(), M, d, None))
    dx = _tiled_normal(M, d, 211, 10, 1e-3)
    order = np.argsort(tok, kind="stable").astype(np.int32)
    seg = np.searchsorted(tok[order], np.arange(V + 1)).astype(np.int32)
    DX = torch.from_numpy(dx).to(dev())
    ORD = torch.from_numpy(order).to(dev())
    SEG = torch.from_numpy(seg).to(dev())
    DE = torch.full((V, d), -1, dtype=torch.int16, device=dev())
    mt.check(mt.lib().mt_embed_bwd(mt.MT_BF16, DX.data_ptr(), ORD.data_ptr(), SEG.data_ptr(), DE.data_ptr(), V, d,
                                   None))
    torch.cuda.synchronize()
    assert np.array_equal(X.cpu().numpy(), datagen.bf16_bits_to_f32(E_bits[tok]))
    ref = np.zeros((V, d), np.float32)
    np.add.at(ref, tok, dx)   # float32, positions in increasing order
    assert np.array_equal(DE.cpu().numpy().view(np.uint16), datagen.f32_to_bf16_bits(ref))
