"""GPU-test helpers: upload seeded problems, call the C ABI, compare with the oracle.

Expected values come only from the oracle (CPU) or, for GPU-vs-GPU invariants,
from another run of the GPU path under a different schedule.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import tile_scheduled_dense_amd as tg
import workloads

TOL = {"f32": 1e-5, "bf16": 4e-3, "f16": 4e-3}
GUARD = 4096          # sentinel floats before and after C
SENTINEL = -1234.5    # not a value any test problem produces


def need_gpu():
    if torch.cuda.device_count() == 0:
        pytest.skip("no GPU visible")


def device_tensor(storage: np.ndarray) -> torch.Tensor:
    if storage.dtype == np.uint16:
        t = torch.from_numpy(storage.view(np.int16))
    else:
        t = torch.from_numpy(storage)
    if t.numel() == 0:
        t = torch.zeros(8, dtype=t.dtype)
    return t.to("cuda")


class GpuProblem:
    """A Problem resident on the GPU, with a guarded C buffer."""

    def __init__(self, p: workloads.Problem):
        self.p = p
        self.A = device_tensor(p.A)
        self.B = device_tensor(p.B)
        n = p.sizeC()
        self.cbuf = torch.full((n + 2 * GUARD,), SENTINEL, dtype=torch.float32, device="cuda")
        self.C = self.cbuf[GUARD:GUARD + n]

    def reset_c(self, fill=None):
        """C <- C0 (beta != 0), else NaN, so an unread C is visible; ldc padding stays sentinel."""
        p = self.p
        self.cbuf.fill_(SENTINEL)
        if p.beta != 0:
            c0 = torch.from_numpy(p.C0).to("cuda")
            pad = torch.isnan(c0)           # ldc padding of C0 is NaN in the generator
            self.C.copy_(torch.where(pad, torch.full_like(c0, SENTINEL), c0))
        else:
            view = self.c_view()
            view.fill_(float("nan") if fill is None else fill)

    def c_view(self) -> torch.Tensor:
        """(batch, M, N) strided view of C inside the buffer."""
        p = self.p
        return torch.as_strided(self.C, (p.batch, p.M, p.N), (p.strideC, p.ldc, 1))

    def run(self, stream=None, **opts):
        p = self.p
        tg.tile_gemm_ex(p.batch, p.M, p.N, p.K, p.dtype, self.A, p.lda, p.strideA, self.B, p.ldb, p.strideB,
                        self.C, p.ldc, p.strideC, p.alpha, p.beta, stream, **opts)

    def result(self) -> np.ndarray:
        torch.cuda.synchronize()
        return self.c_view().cpu().numpy().astype(np.float64)

    def check_guards(self):
        """Nothing outside [0, M) x [0, N) of each batch entry was written."""
        torch.cuda.synchronize()
        p = self.p
        buf = self.cbuf.cpu().numpy()
        mask = np.ones(buf.shape, dtype=bool)
        for b in range(p.batch):
            for i in range(p.M):
                s = GUARD + b * p.strideC + i * p.ldc
                mask[s:s + p.N] = False
        outside = buf[mask]
        assert np.all(outside == SENTINEL), "a write landed outside C's M x N window"


def oracle_full(p: workloads.Problem):
    return oracle.gemm(p.M, p.N, p.K, p.dtype, p.A, p.lda, p.B, p.ldb, C0=p.C0, ldc=p.ldc, alpha=p.alpha,
                       beta=p.beta, batch=p.batch, strideA=p.strideA, strideB=p.strideB, strideC=p.strideC,
                       with_absden=True)


def oracle_points(p: workloads.Problem, pts):
    return oracle.gemm_points(p.M, p.N, p.K, p.dtype, p.A, p.lda, p.B, p.ldb, pts, C0=p.C0, ldc=p.ldc,
                              alpha=p.alpha, beta=p.beta, batch=p.batch, strideA=p.strideA,
                              strideB=p.strideB, strideC=p.strideC)


def parity_error(got, ref, den):
    """max |C_gpu - C_ref| / (sum_k |a||b| + 1e-30) where the sum is nonzero;
    where it is zero (K == 0, zero rows) C must equal the oracle exactly."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.asarray(den, dtype=np.float64)
    assert not np.isnan(got).any(), "NaN in the GPU result"
    zero = den == 0
    if zero.any():
        assert np.array_equal(got[zero], ref[zero]), "empty-sum outputs must equal beta*C0 exactly"
    if (~zero).any():
        return float(np.max(np.abs(got[~zero] - ref[~zero]) / (den[~zero] + 1e-30)))
    return 0.0


def c0_at(p: workloads.Problem, pts=None) -> np.ndarray:
    """C0 as float64, (batch, M, N) or at the points; zeros when beta == 0."""
    if p.beta == 0 or p.C0 is None:
        return np.zeros(len(pts) if pts is not None else (p.batch, p.M, p.N))
    if pts is not None:
        idx = pts[:, 0] * p.strideC + pts[:, 1] * p.ldc + pts[:, 2]
        return p.C0[idx].astype(np.float64)
    out = np.zeros((p.batch, p.M, p.N))
    for b in range(p.batch):
        out[b] = p.C0[b * p.strideC: b * p.strideC + p.M * p.ldc].reshape(p.M, p.ldc)[:, :p.N]
    return out


def half_ulp32(x) -> np.ndarray:
    """Half the fp32 spacing at |x|: the rounding of one fp32 operation that yields x."""
    return 0.5 * np.spacing(np.abs(np.asarray(x, dtype=np.float64)).astype(np.float32)).astype(np.float64)


def check_parity(p: workloads.Problem, got_full: np.ndarray, points=None, stated=False):
    """Compare with the oracle: full result, or at sampled points for big problems.

    The metric is the stated one, max |C_gpu - C_ref| / (sum_k |a||b| + 1e-30).  Unless
    `stated`, the two roundings an fp32 output of alpha * acc + beta * C0 cannot avoid are
    taken off |C_gpu - C_ref| first: half an ulp of the result (the epilogue's fma) and half
    an ulp of beta * C0 (its product, exact when beta is a power of two).  With small K and a
    large C0 those roundings alone exceed 1e-5 of sum |a||b| (K = 1, fp32: 2.1e-5).
    """
    if points is None:
        ref, den = oracle_full(p)
        got = got_full
        c0 = c0_at(p)
    else:
        ref, den = oracle_points(p, points)
        got = got_full[points[:, 0], points[:, 1], points[:, 2]]
        c0 = c0_at(p, points)
    err = parity_error(got, ref, den) if stated else parity_error_rounded(got, ref, den, p.beta, c0)
    assert err <= TOL[p.dtype], f"parity error {err:.3e} > {TOL[p.dtype]:.0e}"
    return err


def parity_error_rounded(got, ref, den, beta, c0):
    """parity_error after taking off |C_gpu - C_ref| the output's unavoidable fp32 roundings,
    half an ulp of the result and half an ulp of beta * C0; where sum |a||b| is zero the
    comparison stays exact."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.asarray(den, dtype=np.float64)
    slack = np.where(den > 0, half_ulp32(ref) + half_ulp32(beta * np.asarray(c0, dtype=np.float64)), 0.0)
    diff = np.abs(got - ref)
    # move got toward ref by the unavoidable rounding, never past it
    got = np.where(diff <= slack, ref, got - np.sign(got - ref) * slack)
    return parity_error(got, ref, den)


def result_points(gp: GpuProblem, pts) -> np.ndarray:
    torch.cuda.synchronize()
    idx = torch.from_numpy(np.ascontiguousarray(pts)).to("cuda")
    v = gp.c_view()[idx[:, 0], idx[:, 1], idx[:, 2]]
    return v.cpu().numpy().astype(np.float64)
