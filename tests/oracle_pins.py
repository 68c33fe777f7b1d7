"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each check takes an ``OracleLibrary`` so that the same checks can be run on a
deliberately broken copy of the oracle (see test_oracle_mutants.py) to show that
they would catch a plausible mistake.  Expected values never come from the GPU.

Independent decoders used for comparison: numpy's float16 and torch's bfloat16
conversions (library routines), and Python's ``float``/``fractions``.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch

import workloads


def to_f64(storage: np.ndarray, dtype: str) -> np.ndarray:
    """Decode storage with numpy/torch (not with the oracle's own decoders)."""
    if dtype == "f32":
        return storage.astype(np.float64)
    if dtype == "f16":
        return storage.view(np.float16).astype(np.float64)
    t = torch.from_numpy(storage.view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def from_f64(values: np.ndarray, dtype: str) -> np.ndarray:
    """Encode exactly representable values into storage."""
    if dtype == "f32":
        out = values.astype(np.float32)
    elif dtype == "f16":
        out = values.astype(np.float16).view(np.uint16)
    else:
        out = torch.from_numpy(values.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    back = to_f64(np.ascontiguousarray(out), dtype)
    assert np.array_equal(back, values.astype(np.float64)), "value not representable"
    return np.ascontiguousarray(out).reshape(-1)


def dense(p, which):
    """(batch, rows, cols) float64 view of A or B of a Problem."""
    if which == "A":
        rows, cols, ld, st, buf = p.M, p.K, p.lda, p.strideA, p.A
    else:
        rows, cols, ld, st, buf = p.K, p.N, p.ldb, p.strideB, p.B
    out = np.zeros((p.batch, rows, cols))
    full = to_f64(buf, p.dtype)
    for b in range(p.batch):
        if rows and cols:
            out[b] = full[b * st: b * st + rows * ld].reshape(rows, ld)[:, :cols]
    return out


def run(lib, p, with_absden=False):
    return lib.gemm(p.M, p.N, p.K, p.dtype, p.A, p.lda, p.B, p.ldb, C0=p.C0, ldc=p.ldc,
                    alpha=p.alpha, beta=p.beta, batch=p.batch, strideA=p.strideA,
                    strideB=p.strideB, strideC=p.strideC, with_absden=with_absden)


def pin_decode(lib):
    """Every bf16 and f16 bit pattern decodes as the library conversions do."""
    bits = np.arange(65536, dtype=np.uint16)
    for dt in ("f16", "bf16"):
        mine = lib.decode(bits, dt)
        ref = to_f64(bits, dt)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(mine), nan), dt
        assert np.array_equal(mine[~nan], ref[~nan]), dt
        assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan])), dt


def pin_identity_permutation(lib):
    """A = I or a permutation: every output has one nonzero term, so C = alpha*P.B exactly."""
    rng = np.random.default_rng(7)
    for dt in ("f32", "bf16", "f16"):
        for alpha in (1.0, 1.5, -2.0):
            M = K = 29
            N = 19
            p = workloads.custom(dt, M, N, K, ldb_pad=3, alpha=alpha, seed=3)
            Bd = dense(p, "B")[0]
            perm = rng.permutation(M)
            P = np.zeros((M, K))
            P[np.arange(M), perm] = 1.0
            for mat in (np.eye(M), P):
                p.A = from_f64(mat, dt)
                p.lda = K
                p.strideA = M * K
                got = run(lib, p)[0]
                exp = alpha * (mat @ Bd)      # one nonzero term per output: exact
                assert np.array_equal(got, exp), (dt, alpha)
            # B a permutation: column permutation of A
            p2 = workloads.custom(dt, 23, 31, 31, lda_pad=2, alpha=alpha, seed=4)
            Ad = dense(p2, "A")[0]
            perm = rng.permutation(31)
            Pb = np.zeros((31, 31))
            Pb[perm, np.arange(31)] = 1.0
            p2.B = from_f64(Pb, dt)
            p2.ldb = 31
            p2.strideB = 31 * 31
            got = run(lib, p2)[0]
            assert np.array_equal(got, alpha * Ad[:, perm]), (dt, alpha)


def pin_bruteforce_python(lib):
    """Tiny shapes: a Python float loop in k order is bitwise equal; exact Fraction sums are within gamma_K."""
    for dt in ("f32", "bf16", "f16"):
        for (M, N, K) in [(1, 1, 1), (1, 5, 3), (4, 1, 7), (3, 7, 2), (9, 8, 9), (5, 3, 13), (2, 2, 0)]:
            p = workloads.custom(dt, M, N, K, lda_pad=2, ldb_pad=1, ldc_pad=3, alpha=1.25, beta=-0.75,
                                 seed=M * 100 + N * 10 + K)
            A, B = dense(p, "A")[0], dense(p, "B")[0]
            C0 = np.zeros((M, N))
            if p.C0 is not None and M:
                C0 = p.C0[: M * p.ldc].reshape(M, p.ldc)[:, :N].astype(np.float64)
            got = run(lib, p)[0]
            for i in range(M):
                for j in range(N):
                    s = 0.0
                    for k in range(K):
                        s += float(A[i, k]) * float(B[k, j])
                    exp = 1.25 * s + (-0.75) * float(C0[i, j])
                    assert got[i, j] == exp, (dt, M, N, K, i, j)
                    # exact rational sum; binary64 k-ordered sum error <= (K-1) u sum|ab|
                    fs = sum((Fraction(float(A[i, k])) * Fraction(float(B[k, j])) for k in range(K)), Fraction(0))
                    den = sum(abs(float(A[i, k]) * float(B[k, j])) for k in range(K))
                    s_or = (got[i, j] - (-0.75) * float(C0[i, j])) / 1.25
                    bound = max(K - 1, 0) * 2.0 ** -53 * den + 4 * 2.0 ** -53 * abs(float(fs)) + 1e-300
                    assert abs(float(Fraction(s_or) - fs)) <= bound + 2.0 ** -52 * (abs(s_or) + abs(C0[i, j])), (dt, i, j)


def pin_numpy_matmul(lib):
    """Medium shapes: numpy's float64 matmul (a library routine) agrees to 1e-12 relative to sum|a||b|."""
    for dt, (M, N, K) in [("f32", (70, 90, 150)), ("bf16", (129, 65, 257)), ("f16", (64, 130, 99))]:
        p = workloads.custom(dt, M, N, K, lda_pad=5, ldb_pad=7, alpha=0.5, beta=2.0, seed=11)
        A, B = dense(p, "A")[0], dense(p, "B")[0]
        C0 = p.C0[: M * p.ldc].reshape(M, p.ldc)[:, :N].astype(np.float64)
        got, den = run(lib, p, with_absden=True)
        exp = 0.5 * (A @ B) + 2.0 * C0
        den_ref = np.abs(A) @ np.abs(B)
        assert np.all(np.abs(got[0] - exp) <= 1e-12 * (0.5 * den_ref + 2.0 * np.abs(C0) + 1e-300)), dt
        assert np.allclose(den[0], den_ref, rtol=1e-12, atol=0), dt


def pin_padding_invariance(lib):
    """Zero-padding M, N, K (any amount) and NaN in the ld padding leave C bit-exactly unchanged."""
    for dt in ("f32", "bf16", "f16"):
        M, N, K = 37, 41, 53
        p = workloads.custom(dt, M, N, K, lda_pad=3, ldb_pad=5, ldc_pad=2, alpha=1.5, beta=0.5, seed=21)
        base = run(lib, p)[0]
        A, B = dense(p, "A")[0], dense(p, "B")[0]
        C0 = p.C0[: M * p.ldc].reshape(M, p.ldc)[:, :N]
        for (Mp, Np, Kp) in [(64, 64, 64), (40, 48, 56), (37, 41, 128), (96, 41, 53)]:
            lda, ldb, ldc = Kp + 4, Np + 3, Np + 1
            Ap = np.zeros((Mp, lda))
            Ap[:, Kp:] = np.nan
            Ap[:M, :K] = A
            Bp = np.zeros((Kp, ldb))
            Bp[:, Np:] = np.nan
            Bp[:K, :N] = B
            Cp = np.zeros((Mp, ldc), dtype=np.float32)
            Cp[:, Np:] = np.nan
            Cp[:M, :N] = C0
            q = workloads.Problem("pad", dt, Mp, Np, Kp, lda=lda, ldb=ldb, ldc=ldc, alpha=1.5, beta=0.5)
            q.A = _encode_with_nan(Ap, dt)
            q.B = _encode_with_nan(Bp, dt)
            q.C0 = Cp.reshape(-1)
            got = run(lib, q)[0][:M, :N]
            assert np.array_equal(got, base), (dt, Mp, Np, Kp)


def _encode_with_nan(x, dt):
    fin = np.where(np.isnan(x), 0.0, x)
    enc = from_f64(fin, dt)
    nanbits = {"bf16": 0x7FC0, "f16": 0x7E00}
    if dt == "f32":
        enc = enc.copy()
        enc[np.isnan(x).reshape(-1)] = np.nan
    else:
        enc = enc.copy()
        enc[np.isnan(x).reshape(-1)] = nanbits[dt]
    return enc


def pin_closed_forms(lib):
    """All-ones, rank-1, K = 0 and beta = 0 with NaN C0."""
    for dt in ("f32", "bf16", "f16"):
        M, N, K = 13, 17, 40
        ones = workloads.Problem("ones", dt, M, N, K, alpha=1.5, beta=0.5)
        ones.A = from_f64(np.ones((M, K)), dt)
        ones.B = from_f64(np.ones((K, N)), dt)
        c0 = np.arange(M * N, dtype=np.float32).reshape(M, N) - 100
        ones.C0 = c0.reshape(-1)
        got = run(lib, ones)[0]
        assert np.array_equal(got, 1.5 * K + 0.5 * c0.astype(np.float64)), dt
        # rank one: A = u 1^T, B = 1 v^T  ->  C_ij = alpha K u_i v_j
        u = np.arange(1, M + 1, dtype=np.float64) / 4
        v = -np.arange(1, N + 1, dtype=np.float64) / 8
        r1 = workloads.Problem("rank1", dt, M, N, K, alpha=2.0)
        r1.A = from_f64(np.repeat(u[:, None], K, axis=1), dt)
        r1.B = from_f64(np.repeat(v[None, :], K, axis=0), dt)
        got = run(lib, r1)[0]
        assert np.array_equal(got, 2.0 * K * np.outer(u, v)), dt
        # K = 0: C = beta C0
        k0 = workloads.custom(dt, 9, 7, 0, alpha=3.0, beta=0.5, seed=5)
        got = run(lib, k0)[0]
        c0 = k0.C0.reshape(9, 7).astype(np.float64)
        assert np.array_equal(got, 0.5 * c0), dt
        # beta = 0: C0 is not read (NaN stays out)
        nb = workloads.custom(dt, 9, 7, 5, alpha=1.0, beta=0.0, seed=6)
        nb_c0 = np.full(9 * 7, np.nan, dtype=np.float32)
        got = lib.gemm(9, 7, 5, dt, nb.A, nb.lda, nb.B, nb.ldb, C0=nb_c0, ldc=7, alpha=1.0, beta=0.0)
        assert not np.isnan(got).any(), dt
        A, B = dense(nb, "A")[0], dense(nb, "B")[0]
        assert np.allclose(got[0], A @ B, rtol=0, atol=1e-12)


def pin_batched_and_points(lib):
    """A strided batch equals separate problems; sampled points equal the full result bitwise."""
    for dt in ("bf16", "f16"):
        p = workloads.custom(dt, 19, 23, 31, batch=4, alpha=0.75, beta=1.0, seed=8)
        full, den = run(lib, p, with_absden=True)
        for b in range(p.batch):
            A, B = dense(p, "A")[b], dense(p, "B")[b]
            C0 = p.C0[b * p.strideC: b * p.strideC + p.M * p.ldc].reshape(p.M, p.ldc)[:, :p.N].astype(np.float64)
            exp = 0.75 * (A @ B) + C0
            assert np.all(np.abs(full[b] - exp) <= 1e-12 * (0.75 * (np.abs(A) @ np.abs(B)) + np.abs(C0)))
        pts = workloads.sample_points(p, 200)
        v, d = lib.gemm_points(p.M, p.N, p.K, dt, p.A, p.lda, p.B, p.ldb, pts, C0=p.C0, ldc=p.ldc,
                               alpha=p.alpha, beta=p.beta, batch=p.batch, strideA=p.strideA,
                               strideB=p.strideB, strideC=p.strideC)
        assert np.array_equal(v, full[pts[:, 0], pts[:, 1], pts[:, 2]])
        assert np.array_equal(d, den[pts[:, 0], pts[:, 1], pts[:, 2]])


def pin_fused_tail(lib):
    """The fused tail act(alpha A.B + bias) + beta C0 against values fixed outside the oracle.

    * GELU is x Phi(x) with Phi the standard normal CDF: at the normal quantiles
      z(0.975) = 1.959963984540054 and z(0.75) = 0.6744897501960817 (fp32-rounded
      as the bias stores them) it is z times 0.975 and 0.75 to within Phi's slope
      times the rounding; GELU(0) = 0; and GELU(x) - GELU(-x) = x, since Phi(x) +
      Phi(-x) = 1;
    * ReLU keeps x > 0 and zeroes x < 0, so relu(x) - relu(-x) = x;
    * the residual is added after the activation: with K = 0, bias -1, ReLU,
      beta 1 and C0 = 2 every output is 2 (inside the activation it would be 1);
    * a per-column bias varies along a row, a per-row bias down a column;
    * K > 0: against numpy's product and scipy's normal CDF (ndtr) on the decoded
      operands; a strided batch with a bias stride equals its separate problems;
      sampled points equal the full result bitwise.
    """
    from scipy.special import ndtr
    empty = np.zeros(0, np.float32)
    # quantiles: K = 0, so the output is act(bias)
    z = np.array([1.959963984540054, 0.6744897501960817, 0.0, -1.959963984540054, -0.6744897501960817],
                 dtype=np.float32)
    got = lib.gemm(1, 5, 0, "f32", empty, 1, empty, 5, bias=z, bias_mode=1, activation=2)[0, 0]
    zq = z.astype(np.float64)
    phi = np.array([0.975, 0.75, 0.5, 0.025, 0.25])
    slack = np.abs(zq) * 0.4 * 1e-7 * np.abs(zq)      # |z| * pdf * |z - z_exact|, pdf < 0.4
    assert np.all(np.abs(got - zq * phi) <= slack + 1e-15), got
    assert got[2] == 0.0
    # odd part of GELU and ReLU
    x = np.linspace(-6, 6, 97).astype(np.float32)
    for act in (1, 2):
        pos = lib.gemm(1, 97, 0, "f32", empty, 1, empty, 97, bias=x, bias_mode=1, activation=act)[0, 0]
        neg = lib.gemm(1, 97, 0, "f32", empty, 1, empty, 97, bias=-x, bias_mode=1, activation=act)[0, 0]
        assert np.allclose(pos - neg, x.astype(np.float64), rtol=0, atol=1e-15), act
    relu = lib.gemm(1, 97, 0, "f32", empty, 1, empty, 97, bias=x, bias_mode=1, activation=1)[0, 0]
    assert np.array_equal(relu, np.where(x > 0, x, 0).astype(np.float64))
    # the residual after the activation
    c0 = np.full(6, 2.0, np.float32)
    got = lib.gemm(2, 3, 0, "f32", empty, 1, empty, 3, C0=c0, ldc=3, beta=1.0, bias=np.full(3, -1.0, np.float32),
                   bias_mode=1, activation=1)
    assert np.array_equal(got, np.full((1, 2, 3), 2.0))
    # bias orientation
    col = np.array([1.0, 2.0, 3.0], np.float32)
    row = np.array([10.0, 20.0], np.float32)
    assert np.array_equal(lib.gemm(2, 3, 0, "f32", empty, 1, empty, 3, bias=col, bias_mode=1)[0],
                          np.array([[1.0, 2.0, 3.0], [1.0, 2.0, 3.0]]))
    assert np.array_equal(lib.gemm(2, 3, 0, "f32", empty, 1, empty, 3, bias=row, bias_mode=2)[0],
                          np.array([[10.0, 10.0, 10.0], [20.0, 20.0, 20.0]]))
    # K > 0 against numpy and scipy
    rng = np.random.default_rng(21)
    for dt in ("f32", "bf16", "f16"):
        p = workloads.custom(dt, 21, 19, 37, batch=3, ldc_pad=2, alpha=0.5, beta=-0.75, seed=22)
        A, B = dense(p, "A"), dense(p, "B")
        C0 = np.stack([p.C0[b * p.strideC: b * p.strideC + p.M * p.ldc].reshape(p.M, p.ldc)[:, :p.N]
                       for b in range(p.batch)]).astype(np.float64)
        for mode, length in ((1, p.N), (2, p.M)):
            stride = length + 4
            bias = rng.standard_normal(p.batch * stride).astype(np.float32)
            for act in (0, 1, 2):
                got = lib.gemm(p.M, p.N, p.K, dt, p.A, p.lda, p.B, p.ldb, C0=p.C0, ldc=p.ldc, alpha=p.alpha,
                               beta=p.beta, batch=p.batch, strideA=p.strideA, strideB=p.strideB,
                               strideC=p.strideC, bias=bias, bias_stride=stride, bias_mode=mode, activation=act)
                for b in range(p.batch):
                    bv = bias[b * stride: b * stride + length].astype(np.float64)
                    y = p.alpha * (A[b] @ B[b]) + (bv[None, :] if mode == 1 else bv[:, None])
                    y = y if act == 0 else np.maximum(y, 0.0) if act == 1 else y * ndtr(y)
                    exp = y + p.beta * C0[b]
                    scale = p.alpha * (np.abs(A[b]) @ np.abs(B[b])) + np.abs(bv).max() + abs(p.beta) * np.abs(C0[b])
                    assert np.all(np.abs(got[b] - exp) <= 1e-12 * scale), (dt, mode, act, b)
                pts = workloads.sample_points(p, 60)
                v, _ = lib.gemm_points(p.M, p.N, p.K, dt, p.A, p.lda, p.B, p.ldb, pts, C0=p.C0, ldc=p.ldc,
                                       alpha=p.alpha, beta=p.beta, batch=p.batch, strideA=p.strideA,
                                       strideB=p.strideB, strideC=p.strideC, bias=bias, bias_stride=stride,
                                       bias_mode=mode, activation=act)
                assert np.array_equal(v, got[pts[:, 0], pts[:, 1], pts[:, 2]]), (dt, mode, act)


ALL_PINS = [pin_decode, pin_identity_permutation, pin_bruteforce_python, pin_numpy_matmul,
            pin_padding_invariance, pin_closed_forms, pin_batched_and_points, pin_fused_tail]
