"""tile_scheduled_dense_amd -- Python binding of the gfx950 tiled GEMM library.

C = alpha * A . B + beta * C, row-major, any extents; A/B fp32, bf16 or fp16,
C fp32.  Every step runs in the HIP kernels of ``libtile_gemm.so`` (built
in-tree by ``build_lib.py``); this module only marshals arguments into its C
ABI (``include/tile_gemm.h``), with the same entry-point names.  There is no
CPU fallback: if the library is missing, every call raises.

Pointers are device addresses (ints) or torch tensors (their ``data_ptr()``);
``stream`` is a ``hipStream_t`` as an int, a ``torch.cuda.Stream``, or None for
torch's current stream on the current device.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtile_gemm.so")

TG_F32, TG_BF16, TG_F16 = 0, 1, 2
DTYPES = {"f32": TG_F32, "bf16": TG_BF16, "f16": TG_F16}

TG_OK, TG_ERR_INVALID_ARG, TG_ERR_UNSUPPORTED, TG_ERR_LAUNCH, TG_ERR_INTERNAL, TG_ERR_SCRATCH_LIMIT = range(6)
STATUS_NAMES = {0: "TG_OK", 1: "TG_ERR_INVALID_ARG", 2: "TG_ERR_UNSUPPORTED", 3: "TG_ERR_LAUNCH",
                4: "TG_ERR_INTERNAL", 5: "TG_ERR_SCRATCH_LIMIT"}
ABI_VERSION = 11
# bytes of the library's own scratch that tile_gemm_ex_noalloc works in (TILE_GEMM_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20

TG_CFG_AUTO, TG_CFG_256x256, TG_CFG_128x128, TG_CFG_64x64, TG_CFG_F32_64x64, TG_CFG_288x160 = range(6)
# layout-introspection ids of the thin fringe-strip blocks of TG_CFG_256x256, and of the
# fp32 ring tiles (TG_CFG_256x256, TG_CFG_128x128 and the strips with fp32 inputs)
LAYOUT_CFG_STRIP_N, LAYOUT_CFG_STRIP_M = 101, 102
LAYOUT_CFG_F32_256, LAYOUT_CFG_F32_128, LAYOUT_CFG_F32_STRIP_N, LAYOUT_CFG_F32_STRIP_M = 103, 104, 105, 106
SWZ_DEFAULT, SWZ_NONE, SWZ_PAD, SWZ_XOR = 0, 1, 2, 3
BIAS_NONE, BIAS_PER_COLUMN, BIAS_PER_ROW = 0, 1, 2
ACT_NONE, ACT_RELU, ACT_GELU = 0, 1, 2

LAYOUT_LDS_A, LAYOUT_LDS_B, LAYOUT_ACC, LAYOUT_COPY_A = range(4)
AXIS_M, AXIS_LANE, AXIS_WAVE, AXIS_PID, AXIS_TLANE, AXIS_TCOL = range(6)
AXIS_COUNT = 6
LAYOUT_MAX_ITERS = 12
LAYOUT_MAX_RANK = 6
LAYOUT_MAX_SWIZZLES = 2

# every symbol include/tile_gemm.h declares
EXPORTED = ["tile_gemm", "tile_gemm_strided_batched", "tile_gemm_ex", "tile_gemm_plan",
            "tile_gemm_workspace_size", "tg_layout_eval", "tile_gemm_describe_layout", "tile_gemm_lds_offset",
            "tile_gemm_acc_coord", "tile_gemm_status_string", "tile_gemm_abi_version", "tile_gemm_packed_b_ld",
            "tile_gemm_packed_b_size", "tile_gemm_pack_b", "tile_gemm_ex_noalloc"]


class TileGemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class Options(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_int), ("force_cfg", ctypes.c_int), ("pipeline_depth", ctypes.c_int),
                ("swizzle", ctypes.c_int), ("block_order", ctypes.c_int), ("split_k", ctypes.c_int),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
                ("pack_a", ctypes.c_int), ("pad0_", ctypes.c_int), ("plan_lda", ctypes.c_int64),
                ("tail_gemm", ctypes.c_int), ("persistent", ctypes.c_int),
                ("bias", ctypes.c_void_p), ("bias_stride", ctypes.c_int64), ("bias_mode", ctypes.c_int),
                ("activation", ctypes.c_int), ("pack_b", ctypes.c_int), ("pad1_", ctypes.c_int),
                ("plan_ldb", ctypes.c_int64)]


# size of the options struct in ABI version 1 (the first five ints)
OPTIONS_V1_SIZE = 5 * ctypes.sizeof(ctypes.c_int)


class PlanInfo(ctypes.Structure):
    _fields_ = [("config", ctypes.c_int), ("block_m", ctypes.c_int), ("block_n", ctypes.c_int),
                ("block_k", ctypes.c_int), ("waves", ctypes.c_int), ("threads", ctypes.c_int),
                ("pipeline_depth", ctypes.c_int), ("swizzle", ctypes.c_int), ("block_order", ctypes.c_int),
                ("tiles_m", ctypes.c_int64), ("tiles_n", ctypes.c_int64), ("grid", ctypes.c_int64),
                ("interior_blocks", ctypes.c_int64), ("fringe_blocks", ctypes.c_int64),
                ("k_tiles", ctypes.c_int64), ("k_tail", ctypes.c_int64), ("lds_bytes", ctypes.c_int),
                ("split_k", ctypes.c_int), ("k_slice", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("mfma_m", ctypes.c_int), ("mfma_n", ctypes.c_int), ("mfma_k", ctypes.c_int), ("pack_a", ctypes.c_int),
                ("strip_blocks", ctypes.c_int64), ("tail_n_splits", ctypes.c_int),
                ("tail_m_splits", ctypes.c_int), ("persistent", ctypes.c_int), ("per_cu", ctypes.c_int),
                ("pack_b", ctypes.c_int), ("strip_splits", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class Iter(ctypes.Structure):
    _fields_ = [("extent", ctypes.c_int64), ("stride", ctypes.c_int64), ("axis", ctypes.c_int32),
                ("pad_", ctypes.c_int32)]


class Swizzle(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int32), ("b", ctypes.c_int32), ("s", ctypes.c_int32)]


class Layout(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32), ("n_shard", ctypes.c_int32), ("n_replica", ctypes.c_int32),
                ("n_swizzle", ctypes.c_int32), ("shape", ctypes.c_int64 * LAYOUT_MAX_RANK),
                ("shard", Iter * LAYOUT_MAX_ITERS), ("replica", Iter * LAYOUT_MAX_ITERS),
                ("offset", ctypes.c_int64 * AXIS_COUNT), ("swizzle", Swizzle * LAYOUT_MAX_SWIZZLES),
                ("pad_", ctypes.c_int32)]


_lib_handle = None


def library_path() -> str:
    return LIB_PATH


def _lib():
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m tile_scheduled_dense_amd.build_lib` "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    i64, f32, vp, ci = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int
    lib.tile_gemm.argtypes = [i64, i64, i64, ci, vp, i64, vp, i64, vp, i64, f32, f32, vp]
    lib.tile_gemm.restype = ci
    lib.tile_gemm_strided_batched.argtypes = [i64, i64, i64, i64, ci, vp, i64, i64, vp, i64, i64,
                                              vp, i64, i64, f32, f32, vp]
    lib.tile_gemm_strided_batched.restype = ci
    lib.tile_gemm_ex.argtypes = [i64, i64, i64, i64, ci, vp, i64, i64, vp, i64, i64, vp, i64, i64,
                                 f32, f32, vp, ctypes.POINTER(Options)]
    lib.tile_gemm_ex.restype = ci
    lib.tile_gemm_ex_noalloc.argtypes = [i64, i64, i64, i64, ci, vp, i64, i64, vp, i64, i64, vp, i64, i64,
                                         f32, f32, vp, ctypes.POINTER(Options)]
    lib.tile_gemm_ex_noalloc.restype = ci
    lib.tile_gemm_plan.argtypes = [i64, i64, i64, i64, ci, ctypes.POINTER(Options), ctypes.POINTER(PlanInfo)]
    lib.tile_gemm_plan.restype = ci
    lib.tile_gemm_workspace_size.argtypes = [i64, i64, i64, i64, ci, ctypes.POINTER(Options), ctypes.POINTER(i64)]
    lib.tile_gemm_workspace_size.restype = ci
    lib.tg_layout_eval.argtypes = [ctypes.POINTER(Layout), ctypes.POINTER(i64), ctypes.POINTER(i64), i64]
    lib.tg_layout_eval.restype = i64
    lib.tile_gemm_describe_layout.argtypes = [ci, ci, ci, ctypes.POINTER(Layout)]
    lib.tile_gemm_describe_layout.restype = ci
    lib.tile_gemm_lds_offset.argtypes = [ci, ci, ci, i64, i64]
    lib.tile_gemm_lds_offset.restype = i64
    lib.tile_gemm_acc_coord.argtypes = [ci, ci, ci, ci, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.tile_gemm_acc_coord.restype = ci
    lib.tile_gemm_status_string.argtypes = [ci]
    lib.tile_gemm_status_string.restype = ctypes.c_char_p
    lib.tile_gemm_abi_version.restype = ci
    lib.tile_gemm_packed_b_ld.argtypes = [i64, ci]
    lib.tile_gemm_packed_b_ld.restype = i64
    lib.tile_gemm_packed_b_size.argtypes = [i64, i64, i64, ci, ctypes.POINTER(i64)]
    lib.tile_gemm_packed_b_size.restype = ci
    lib.tile_gemm_pack_b.argtypes = [i64, i64, i64, ci, vp, i64, i64, ci, vp, i64, vp]
    lib.tile_gemm_pack_b.restype = ci
    _lib_handle = lib
    return lib


def _addr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    raise TypeError(f"expected a device address or a tensor, got {type(x)!r}")


def _stream(s) -> int:
    if s is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream) if torch.cuda.is_available() else 0
    if isinstance(s, int):
        return s
    if hasattr(s, "cuda_stream"):
        return int(s.cuda_stream)
    raise TypeError(f"expected a stream, got {type(s)!r}")


def _dtype(d) -> int:
    return DTYPES[d] if isinstance(d, str) else int(d)


def _options(config=0, pipeline_depth=0, swizzle=0, block_order=0, split_k=0, workspace=None,
             workspace_bytes=None, pack_a=0, plan_lda=0, tail_gemm=0, persistent=0, bias=None, bias_stride=0,
             bias_mode=0, activation=0, pack_b=0, plan_ldb=0, force_cfg=None) -> Options:
    """tg_options from keyword arguments (`force_cfg` may also be given as `config`)."""
    ws = _addr(workspace)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0
    cfg = config if force_cfg is None else force_cfg
    return Options(ctypes.sizeof(Options), int(cfg), int(pipeline_depth), int(swizzle), int(block_order),
                   int(split_k), ws, int(workspace_bytes), int(pack_a), 0, int(plan_lda), int(tail_gemm),
                   int(persistent), _addr(bias), int(bias_stride), int(bias_mode), int(activation), int(pack_b), 0,
                   int(plan_ldb))


def _check(status: int, where: str):
    if status != TG_OK:
        raise TileGemmError(status, where)


def status_string(status: int) -> str:
    return _lib().tile_gemm_status_string(int(status)).decode()


def abi_version() -> int:
    return int(_lib().tile_gemm_abi_version())


def tile_gemm(M, N, K, dtype, A, lda, B, ldb, C, ldc, alpha=1.0, beta=0.0, stream=None) -> None:
    _check(_lib().tile_gemm(M, N, K, _dtype(dtype), _addr(A), lda, _addr(B), ldb, _addr(C), ldc,
                            alpha, beta, _stream(stream)), "tile_gemm")


def tile_gemm_strided_batched(batch, M, N, K, dtype, A, lda, strideA, B, ldb, strideB, C, ldc, strideC,
                              alpha=1.0, beta=0.0, stream=None) -> None:
    _check(_lib().tile_gemm_strided_batched(batch, M, N, K, _dtype(dtype), _addr(A), lda, strideA,
                                            _addr(B), ldb, strideB, _addr(C), ldc, strideC, alpha, beta,
                                            _stream(stream)), "tile_gemm_strided_batched")


def tile_gemm_ex(batch, M, N, K, dtype, A, lda, strideA, B, ldb, strideB, C, ldc, strideC,
                 alpha=1.0, beta=0.0, stream=None, **options) -> None:
    """tg_options as keywords (see _options): `workspace` is a device tensor or address for
    split-K partials or the aligned copies of A and B (its byte size is taken from the tensor
    unless `workspace_bytes` is given)."""
    opt = _options(**options)
    _check(_lib().tile_gemm_ex(batch, M, N, K, _dtype(dtype), _addr(A), lda, strideA, _addr(B), ldb, strideB,
                               _addr(C), ldc, strideC, alpha, beta, _stream(stream), ctypes.byref(opt)),
           "tile_gemm_ex")


def tile_gemm_ex_noalloc(batch, M, N, K, dtype, A, lda, strideA, B, ldb, strideB, C, ldc, strideC,
                         alpha=1.0, beta=0.0, stream=None, **options) -> None:
    """tile_gemm_ex in the library's own scratch (no workspace argument, nothing allocated)."""
    opt = _options(**options)
    _check(_lib().tile_gemm_ex_noalloc(batch, M, N, K, _dtype(dtype), _addr(A), lda, strideA, _addr(B), ldb,
                                       strideB, _addr(C), ldc, strideC, alpha, beta, _stream(stream),
                                       ctypes.byref(opt)), "tile_gemm_ex_noalloc")


def tile_gemm_status(fn: str, *args) -> int:
    """Call an entry point and return its raw status instead of raising (argument-error tests)."""
    return int(getattr(_lib(), fn)(*args))


def tile_gemm_plan(batch, M, N, K, dtype, **options) -> dict:
    """The plan a call would launch; bias_mode / activation shape it, the bias itself is not read."""
    info = PlanInfo()
    opt = _options(**options)
    _check(_lib().tile_gemm_plan(batch, M, N, K, _dtype(dtype), ctypes.byref(opt), ctypes.byref(info)),
           "tile_gemm_plan")
    return info.as_dict()


def tile_gemm_workspace_size(batch, M, N, K, dtype, **options) -> int:
    """Bytes of workspace a call with these arguments would use (split-K partials, the
    aligned copies of A and B and the remainder GEMMs' partials; 0: none)."""
    n = ctypes.c_int64(0)
    options = {k: v for k, v in options.items() if k not in ("workspace", "workspace_bytes")}
    opt = _options(**options)
    _check(_lib().tile_gemm_workspace_size(batch, M, N, K, _dtype(dtype), ctypes.byref(opt), ctypes.byref(n)),
           "tile_gemm_workspace_size")
    return int(n.value)


def tile_gemm_packed_b_ld(N, dtype) -> int:
    """Row length (elements) of B packed by tile_gemm_pack_b: rows of a multiple of 16 bytes."""
    ld = int(_lib().tile_gemm_packed_b_ld(N, _dtype(dtype)))
    if ld < 0:
        raise TileGemmError(TG_ERR_INVALID_ARG, "tile_gemm_packed_b_ld")
    return ld


def tile_gemm_packed_b_size(batch, K, N, dtype) -> int:
    n = ctypes.c_int64(0)
    _check(_lib().tile_gemm_packed_b_size(batch, K, N, _dtype(dtype), ctypes.byref(n)), "tile_gemm_packed_b_size")
    return int(n.value)


def tile_gemm_pack_b(batch, K, N, dtype, B, ldb, strideB, packed, packed_bytes=None, transposed=0,
                     stream=None) -> None:
    """Pack B (K x N, or stored transposed as N x K with transposed=1) into `packed` once; later
    calls pass `packed` as B with ldb = tile_gemm_packed_b_ld(N, dtype) and strideB = K * ldb."""
    if packed_bytes is None:
        packed_bytes = packed.numel() * packed.element_size() if hasattr(packed, "numel") else 0
    _check(_lib().tile_gemm_pack_b(batch, K, N, _dtype(dtype), _addr(B), ldb, strideB, int(transposed),
                                   _addr(packed), int(packed_bytes), _stream(stream)), "tile_gemm_pack_b")


def make_layout(shape, shard, replica=(), offset=None, swizzle=None) -> Layout:
    """Build a tg_layout: shard/replica are (extent, stride, axis) triples; swizzle is
    one (M, B, S) triple or a list of them, applied in order."""
    L = Layout()
    L.rank = len(shape)
    for d, e in enumerate(shape):
        L.shape[d] = e
    L.n_shard = len(shard)
    for k, (e, s, a) in enumerate(shard):
        L.shard[k] = Iter(e, s, a, 0)
    L.n_replica = len(replica)
    for k, (e, s, a) in enumerate(replica):
        L.replica[k] = Iter(e, s, a, 0)
    for a, v in (offset or {}).items():
        L.offset[a] = v
    if swizzle is not None:
        chain = [swizzle] if isinstance(swizzle[0], int) else list(swizzle)
        L.n_swizzle = len(chain)
        for z, (m, b, sh) in enumerate(chain):
            L.swizzle[z] = Swizzle(m, b, sh)
    return L


def tg_layout_eval(layout: Layout, x) -> list:
    """All coordinates of L(x), each a tuple of AXIS_COUNT ints."""
    xs = (ctypes.c_int64 * len(x))(*x)
    n = _lib().tg_layout_eval(ctypes.byref(layout), xs, None, 0)
    if n < 0:
        raise ValueError("invalid layout or coordinate")
    out = (ctypes.c_int64 * (AXIS_COUNT * max(n, 1)))()
    _lib().tg_layout_eval(ctypes.byref(layout), xs, out, n)
    return [tuple(out[r * AXIS_COUNT:(r + 1) * AXIS_COUNT]) for r in range(n)]


def tile_gemm_describe_layout(config, swizzle, kind) -> Layout:
    L = Layout()
    _check(_lib().tile_gemm_describe_layout(config, swizzle, kind, ctypes.byref(L)), "tile_gemm_describe_layout")
    return L


def tile_gemm_lds_offset(config, swizzle, operand, row, k) -> int:
    return int(_lib().tile_gemm_lds_offset(config, swizzle, operand, row, k))


def tile_gemm_acc_coord(config, wave, lane, slot):
    r, c = ctypes.c_int64(), ctypes.c_int64()
    rc = _lib().tile_gemm_acc_coord(config, wave, lane, slot, ctypes.byref(r), ctypes.byref(c))
    if rc != 0:
        raise ValueError("invalid accumulator slot")
    return int(r.value), int(c.value)
