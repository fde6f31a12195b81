"""Python binding of libkqmv.so, the MI355X k-quant decode matvec library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/kqmv.h.  The functions keep the
C names.  Tensors are torch tensors on the GPU (PyTorch supplies device
memory and streams); plain integers are accepted as raw device pointers.
If the library has not been built the calls raise -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkqmv.so")

KQ_Q4_K, KQ_Q5_K, KQ_Q6_K = 12, 13, 14
KQ_MAX_SET = 16
KQ_MAX_NTOK = 8
STATUS = {
    0: "KQ_OK", -1: "KQ_ERR_FORMAT", -2: "KQ_ERR_COLS", -3: "KQ_ERR_ROWS", -4: "KQ_ERR_NTOK",
    -5: "KQ_ERR_NULL", -6: "KQ_ERR_ALIGN", -7: "KQ_ERR_STRIDE", -8: "KQ_ERR_OVERLAP",
    -9: "KQ_ERR_SET_SIZE", -10: "KQ_ERR_HIP", -11: "KQ_ERR_TOO_LARGE", -12: "KQ_ERR_SCRATCH",
}
EXPORTS = ("kq_block_bytes", "kq_row_bytes", "kq_matvec", "kq_matvec_set", "kq_matvec_set_noalloc",
           "kq_validate_set", "kq_release_workspace", "kq_debug_set_pipeline", "kq_debug_plan_kernel",
           "kq_debug_set_plane_groups", "kq_debug_plan_plane_groups",
           "kq_matvec16", "kq_matmul", "kq_embed_rows", "kq_unpack_blocks", "kq_dequant", "kq_debug_read_probe", "kq_strerror",
           "kq_version")


class KqError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__("%s failed: %s (%s)" % (what, STATUS.get(code, code), kq_strerror(code)))


class kq_tensor(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("reserved", ctypes.c_int32), ("w", ctypes.c_void_p),
                ("x", ctypes.c_void_p), ("y", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("ldx", ctypes.c_int64), ("ldy", ctypes.c_int64)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libkqmv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkqmv.so is not built (%s); run `python -m quant_matvec_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.kq_block_bytes.argtypes = [i32]
        L.kq_block_bytes.restype = i32
        L.kq_row_bytes.argtypes = [i32, i64]
        L.kq_row_bytes.restype = i64
        L.kq_matvec.argtypes = [i32, vp, i64, i64, vp, i64, vp, i64, i32, vp]
        L.kq_matvec.restype = ctypes.c_int
        L.kq_matvec_set.argtypes = [ctypes.POINTER(kq_tensor), i32, i32, vp]
        L.kq_matvec_set.restype = ctypes.c_int
        L.kq_validate_set.argtypes = [ctypes.POINTER(kq_tensor), i32, i32]
        L.kq_validate_set.restype = ctypes.c_int
        L.kq_matvec_set_noalloc.argtypes = [ctypes.POINTER(kq_tensor), i32, i32, vp]
        L.kq_matvec_set_noalloc.restype = ctypes.c_int
        L.kq_debug_set_pipeline.argtypes = [i32]
        L.kq_debug_set_pipeline.restype = ctypes.c_int
        L.kq_debug_plan_kernel.argtypes = [ctypes.POINTER(kq_tensor), i32, i32]
        L.kq_debug_plan_kernel.restype = ctypes.c_int
        L.kq_debug_set_plane_groups.argtypes = [i32]
        L.kq_debug_set_plane_groups.restype = ctypes.c_int
        L.kq_debug_plan_plane_groups.argtypes = [ctypes.POINTER(kq_tensor), i32, i32]
        L.kq_debug_plan_plane_groups.restype = ctypes.c_int
        L.kq_release_workspace.argtypes = [vp]
        L.kq_release_workspace.restype = ctypes.c_int
        L.kq_unpack_blocks.argtypes = [i32, vp, i64, vp, vp, vp, vp, vp, vp]
        L.kq_unpack_blocks.restype = ctypes.c_int
        L.kq_dequant.argtypes = [i32, vp, i64, i64, vp, i64, vp]
        L.kq_dequant.restype = ctypes.c_int
        L.kq_matvec16.argtypes = [i32, vp, i64, i64, vp, i64, vp, i64, i32, vp]
        L.kq_matvec16.restype = ctypes.c_int
        L.kq_matmul.argtypes = [i32, vp, i64, i64, vp, i64, vp, i64, i32, vp]
        L.kq_matmul.restype = ctypes.c_int
        L.kq_embed_rows.argtypes = [i32, vp, i64, i64, vp, i32, vp, i64, vp]
        L.kq_embed_rows.restype = ctypes.c_int
        L.kq_debug_read_probe.argtypes = [vp, i64, vp, vp]
        L.kq_debug_read_probe.restype = ctypes.c_int
        L.kq_strerror.argtypes = [ctypes.c_int]
        L.kq_strerror.restype = ctypes.c_char_p
        L.kq_version.argtypes = []
        L.kq_version.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, what: str) -> int:
    if rc < 0:
        raise KqError(rc, what)
    return rc


def kq_block_bytes(fmt: int) -> int:
    return _check(load().kq_block_bytes(fmt), "kq_block_bytes")


def kq_row_bytes(fmt: int, cols: int) -> int:
    return _check(load().kq_row_bytes(fmt, cols), "kq_row_bytes")


def kq_strerror(code: int) -> str:
    return load().kq_strerror(code).decode()


def kq_version() -> int:
    return load().kq_version()


def kq_debug_read_probe(buf, sink, stream=None) -> int:
    """One trivial streaming-read launch over the whole of `buf` (a GPU
    tensor, 16-byte multiple); `sink` a GPU int32 tensor (calibration)."""
    nbytes = buf.numel() * buf.element_size()
    return _check(load().kq_debug_read_probe(_ptr(buf), nbytes, _ptr(sink), _stream(stream)),
                  "kq_debug_read_probe")


def _plane_stride(t, default: int) -> int:
    if isinstance(t, int) or t is None or t.dim() < 2:
        return default
    return t.shape[-1]


def kq_matvec(fmt: int, w, rows: int, cols: int, x, y, ntok: int = 1, ldx: int | None = None,
              ldy: int | None = None, stream=None) -> None:
    """y[t][i] = sum_j W[i,j] x[t][j], t < ntok (x: [ntok, ldx], y: [ntok, ldy])."""
    ldx = _plane_stride(x, cols) if ldx is None else ldx
    ldy = _plane_stride(y, rows) if ldy is None else ldy
    rc = load().kq_matvec(fmt, _ptr(w), rows, cols, _ptr(x), ldx, _ptr(y), ldy, ntok, _stream(stream))
    _check(rc, "kq_matvec")


def make_set(tensors) -> ctypes.Array:
    """tensors: iterable of dicts with fmt, w, x, y, rows, cols (and optional ldx, ldy)."""
    tensors = list(tensors)
    arr = (kq_tensor * max(1, len(tensors)))()
    for i, d in enumerate(tensors):
        arr[i].fmt = d["fmt"]
        arr[i].reserved = d.get("reserved", 0)
        arr[i].w = _ptr(d["w"])
        arr[i].x = _ptr(d["x"])
        arr[i].y = _ptr(d["y"])
        arr[i].rows = d["rows"]
        arr[i].cols = d["cols"]
        arr[i].ldx = d.get("ldx") or _plane_stride(d["x"], d["cols"])
        arr[i].ldy = d.get("ldy") or _plane_stride(d["y"], d["rows"])
    return arr


def kq_matvec_set(tensors, ntok: int = 1, stream=None, n: int | None = None) -> None:
    """One grid-split launch over a set of tensors (list of dicts or a kq_tensor array)."""
    arr = tensors if isinstance(tensors, ctypes.Array) else make_set(tensors)
    count = len(arr) if n is None else n
    _check(load().kq_matvec_set(arr, count, ntok, _stream(stream)), "kq_matvec_set")


def kq_validate_set(tensors, ntok: int = 1, n: int | None = None) -> int:
    """Host-only checks of a set; returns the status code (no HIP call)."""
    arr = tensors if isinstance(tensors, ctypes.Array) else make_set(tensors)
    count = len(arr) if n is None else n
    return load().kq_validate_set(arr, count, ntok)


def kq_matvec_set_noalloc(tensors, ntok: int = 1, stream=None, n: int | None = None) -> None:
    """kq_matvec_set with the library's fixed scratch instead of a workspace:
    allocates nothing (raises KqError with KQ_ERR_SCRATCH for a plan that
    needs more than the scratch holds)."""
    arr = tensors if isinstance(tensors, ctypes.Array) else make_set(tensors)
    count = len(arr) if n is None else n
    _check(load().kq_matvec_set_noalloc(arr, count, ntok, _stream(stream)), "kq_matvec_set_noalloc")


def kq_debug_set_pipeline(mode) -> None:
    """Debug/test: which launches may take the pipelined kernel: False or 0
    none, True or 1 large enough ones (the default), 2 any that fit."""
    _check(load().kq_debug_set_pipeline(int(mode)), "kq_debug_set_pipeline")


def kq_debug_plan_kernel(tensors, ntok: int = 1, n: int | None = None) -> str:
    """Debug/test: the kernel kq_matvec_set would launch for this set on the
    current device, "kq_pc_kernel<ntok>" (pipelined) or "kq_matvec_kernel<ntok>"."""
    arr = tensors if isinstance(tensors, ctypes.Array) else make_set(tensors)
    count = len(arr) if n is None else n
    rc = load().kq_debug_plan_kernel(arr, count, ntok)
    _check(rc, "kq_debug_plan_kernel")
    return ("kq_pc_kernel<%d>" if rc == 1 else "kq_matvec_kernel<%d>") % ntok


def kq_debug_set_plane_groups(groups: int) -> None:
    """Debug/test: token-plane groups of the matvec launches: 0 chosen per
    launch (the default), G >= 1 forced wherever it divides ntok."""
    _check(load().kq_debug_set_plane_groups(int(groups)), "kq_debug_set_plane_groups")


def kq_debug_plan_plane_groups(tensors, ntok: int = 1, n: int | None = None) -> int:
    """Debug/test: the token-plane groups kq_matvec_set would use for this
    set on the current device."""
    arr = tensors if isinstance(tensors, ctypes.Array) else make_set(tensors)
    count = len(arr) if n is None else n
    rc = load().kq_debug_plan_plane_groups(arr, count, ntok)
    _check(rc, "kq_debug_plan_plane_groups")
    return rc


def kq_release_workspace(stream=None) -> None:
    """Free the library's workspaces for `stream` on the current device
    (synchronize the stream first)."""
    _check(load().kq_release_workspace(_stream(stream)), "kq_release_workspace")


def kq_unpack_blocks(fmt: int, w, nblocks: int, codes=None, scales=None, mins=None, d=None, dmin=None,
                     stream=None) -> None:
    rc = load().kq_unpack_blocks(fmt, _ptr(w), nblocks, _ptr(codes), _ptr(scales), _ptr(mins), _ptr(d),
                                 _ptr(dmin), _stream(stream))
    _check(rc, "kq_unpack_blocks")


def kq_matvec16(fmt: int, w, rows: int, cols: int, x, y, ntok: int = 16, ldx: int | None = None,
                ldy: int | None = None, stream=None) -> None:
    """y[t][i] = sum_j W[i,j] x[t][j] for t < ntok <= 16, on the matrix cores."""
    ldx = _plane_stride(x, cols) if ldx is None else ldx
    ldy = _plane_stride(y, rows) if ldy is None else ldy
    rc = load().kq_matvec16(fmt, _ptr(w), rows, cols, _ptr(x), ldx, _ptr(y), ldy, ntok, _stream(stream))
    _check(rc, "kq_matvec16")


def kq_matmul(fmt: int, w, rows: int, cols: int, x, y, ntok: int, ldx: int | None = None,
              ldy: int | None = None, stream=None) -> None:
    """y[t][i] = sum_j W[i,j] x[t][j] for a batch of t < ntok planes."""
    ldx = _plane_stride(x, cols) if ldx is None else ldx
    ldy = _plane_stride(y, rows) if ldy is None else ldy
    rc = load().kq_matmul(fmt, _ptr(w), rows, cols, _ptr(x), ldx, _ptr(y), ldy, ntok, _stream(stream))
    _check(rc, "kq_matmul")


def kq_embed_rows(fmt: int, table, rows: int, cols: int, ids, out, ldo: int | None = None,
                  stream=None) -> None:
    """out[t] = row ids[t] of the dequantized Q4_K table (device int32 ids,
    device float32 out [n][ldo])."""
    n = int(ids.numel()) if hasattr(ids, "numel") else len(ids)
    ldo = _plane_stride(out, cols) if ldo is None else ldo
    rc = load().kq_embed_rows(fmt, _ptr(table), rows, cols, _ptr(ids), n, _ptr(out), ldo, _stream(stream))
    _check(rc, "kq_embed_rows")


def kq_dequant(fmt: int, w, rows: int, cols: int, out, ldw: int | None = None, stream=None) -> None:
    ldw = _plane_stride(out, cols) if ldw is None else ldw
    rc = load().kq_dequant(fmt, _ptr(w), rows, cols, _ptr(out), ldw, _stream(stream))
    _check(rc, "kq_dequant")
