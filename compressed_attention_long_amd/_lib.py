"""ctypes binding of libcsa.so (the C ABI declared in include/csa.h).

Argument marshalling only: torch tensors supply device pointers and the current
stream; every step of the path runs in the library's HIP kernels.  There is no
fallback: if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcsa.so")

CSA_OK, CSA_EINVAL, CSA_ENOTSUP, CSA_EWORKSPACE, CSA_EHIP = 0, -1, -2, -3, -4
CSA_BF16, CSA_FP8_E4M3, CSA_FP32, CSA_FP4_E2M1 = 0, 1, 2, 3
CSA_NOALLOC_SCRATCH_BYTES = 32 << 20   # include/csa.h

# Entry points declared in include/csa.h, in declaration order.
EXPORTS = (
    "csa_compress",
    "csa_compress_batch",
    "csa_index_topk",
    "csa_index_topk_workspace_bytes",
    "csa_index_topk_compress",
    "csa_attend",
    "csa_attend_workspace_bytes",
    "csa_attend_noalloc",
    "hca_attend",
    "hca_attend_workspace_bytes",
    "csa_out_proj",
    "csa_out_proj_workspace_bytes",
    "csa_last_error",
    "csa_abi_version",
)


class CsaError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


class CCache(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("n_valid", ctypes.c_void_p),
        ("pos0", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("cap", ctypes.c_int32),
        ("C", ctypes.c_int32),
        ("scale_block", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("stride", ctypes.c_int32),
    ]


class CCompressCall(ctypes.Structure):
    _fields_ = [
        ("kv", ctypes.c_void_p),
        ("logits", ctypes.c_void_p),
        ("ld_tok", ctypes.c_int64),
        ("ld_seq", ctypes.c_int64),
        ("B", ctypes.c_int32),
        ("T_raw", ctypes.c_int32),
        ("first_row", ctypes.c_int32),
        ("n_new", ctypes.c_int32),
        ("out", ctypes.POINTER(CCache)),
        ("inv_freq", ctypes.c_void_p),
        ("rope_dim", ctypes.c_int32),
    ]


_lib = None

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_PC = ctypes.POINTER(CCache)

_SIGS = {
    "csa_compress": (_i32, [_vp, _vp, _i64, _i64, _i32, _i32, _i32, _i32, _PC, _vp, _i32, _vp]),
    "csa_compress_batch": (_i32, [ctypes.POINTER(CCompressCall), _i32, _vp]),
    "csa_index_topk": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _PC, _i32, _vp, _vp, _vp, _sz, _vp]),
    "csa_index_topk_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "csa_index_topk_compress": (_i32, [ctypes.POINTER(CCompressCall), _i32, _vp, _vp, _vp, _i32, _i32, _i32, _PC,
                                       _i32, _vp, _vp, _vp, _sz, _vp]),
    "csa_attend": (_i32, [_vp, _vp, _i32, _i32, _i32, _PC, _vp, _i32, _PC, _i32, _vp, _vp, _i32, _f32,
                          _vp, _i32, _vp, _vp, _sz, _vp]),
    "csa_attend_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "csa_attend_noalloc": (_i32, [_vp, _vp, _i32, _i32, _i32, _PC, _vp, _i32, _PC, _i32, _vp, _vp, _i32, _f32,
                                  _vp, _i32, _vp, _vp]),
    "hca_attend": (_i32, [_vp, _vp, _i32, _i32, _i32, _PC, _PC, _i32, _vp, _vp, _i32, _f32,
                          _vp, _i32, _vp, _vp, _sz, _vp]),
    "hca_attend_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "csa_out_proj": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _i32, _vp, _i32, _vp, _sz, _vp]),
    "csa_out_proj_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "csa_last_error": (ctypes.c_char_p, []),
    "csa_abi_version": (_i32, []),
}


def load(path: str = LIB_PATH):
    """Load libcsa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m compressed_attention_long_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def last_error() -> str:
    return load().csa_last_error().decode()


def _check(fn: str, rc: int):
    if rc != CSA_OK:
        raise CsaError(fn, rc, last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    return torch.cuda.current_stream().cuda_stream


@dataclasses.dataclass
class Cache:
    """A per-layer row cache (see csa_cache_t): tensors plus row geometry.

    data     [B, cap, C] torch.bfloat16, or torch.uint8 holding E4M3FN codes, or with
             fmt=CSA_FP4_E2M1 [B, cap, C // 2] torch.uint8 holding two E2M1 codes per byte
    scales   [B, cap, C // scale_block] float32 (fp8 and fp4; fp4 blocks are 32 channels)
    n_valid  [B] int32     rows holding data
    pos0     [B] int64     position of raw token 0 of row 0
    """

    data: torch.Tensor
    n_valid: torch.Tensor
    pos0: torch.Tensor
    window: int
    stride: int
    scales: Optional[torch.Tensor] = None
    scale_block: int = 0
    fmt: Optional[int] = None      # storage code; None: bf16 or fp8 from data's dtype

    @property
    def dtype_code(self) -> int:
        if self.fmt is not None:
            return self.fmt
        return CSA_FP8_E4M3 if self.data.dtype == torch.uint8 else CSA_BF16

    @property
    def B(self) -> int:
        return self.data.shape[0]

    @property
    def cap(self) -> int:
        return self.data.shape[1]

    @property
    def C(self) -> int:
        return self.data.shape[2] * (2 if self.dtype_code == CSA_FP4_E2M1 else 1)

    def struct(self) -> CCache:
        assert self.data.is_contiguous()
        assert self.n_valid.dtype == torch.int32 and self.pos0.dtype == torch.int64
        if self.scales is not None:
            assert self.scales.dtype == torch.float32 and self.scales.is_contiguous()
        return CCache(self.data.data_ptr(), _ptr(self.scales), self.n_valid.data_ptr(),
                      self.pos0.data_ptr(), self.dtype_code, self.cap, self.C,
                      self.scale_block, self.window, self.stride)


def compress(kv: torch.Tensor, logits: Optional[torch.Tensor], out: Cache, first_row: int, n_new: int,
             inv_freq: Optional[torch.Tensor], rope_dim: int, stream=None):
    """csa_compress: pool raw rows kv/logits [B, T, C] (bf16) into out rows [first_row, +n_new)."""
    assert kv.dtype == torch.bfloat16 and kv.stride(-1) == 1
    if logits is not None:
        assert logits.dtype == torch.bfloat16 and logits.stride() == kv.stride()
    B, T, _ = kv.shape
    c = out.struct()
    rc = load().csa_compress(kv.data_ptr(), _ptr(logits), kv.stride(1), kv.stride(0), B, T, first_row, n_new,
                             ctypes.byref(c), _ptr(inv_freq), rope_dim, _stream(stream))
    _check("csa_compress", rc)


def _compress_calls(calls):
    """csa_compress_call_t array (and the cache structs it points to, kept alive) for calls =
    [(kv, logits, out, first_row, n_new, inv_freq, rope_dim), ...]."""
    n = len(calls)
    arr = (CCompressCall * max(n, 1))()
    keep = []
    for i, (kv, logits, out, first_row, n_new, inv_freq, rope_dim) in enumerate(calls):
        assert kv.dtype == torch.bfloat16 and kv.stride(-1) == 1
        if logits is not None:
            assert logits.dtype == torch.bfloat16 and logits.stride() == kv.stride()
        c = out.struct()
        keep.append(c)
        B, T, _ = kv.shape
        arr[i] = CCompressCall(kv.data_ptr(), _ptr(logits), kv.stride(1), kv.stride(0), B, T, first_row, n_new,
                               ctypes.pointer(c), _ptr(inv_freq), rope_dim)
    return arr, keep


def compress_batch(calls, stream=None):
    """csa_compress_batch: calls = [(kv, logits, out, first_row, n_new, inv_freq, rope_dim), ...],
    each as for compress(); one launch when every call is small."""
    arr, keep = _compress_calls(calls)
    rc = load().csa_compress_batch(arr, len(calls), _stream(stream))
    _check("csa_compress_batch", rc)


def index_topk_workspace_bytes(B, Tq, Hi, cap, topk) -> int:
    return load().csa_index_topk_workspace_bytes(B, Tq, Hi, cap, topk)


def index_topk(q_idx: torch.Tensor, w: torch.Tensor, q_pos: torch.Tensor, keys: Cache, topk: int,
               idx_out: torch.Tensor, scores_out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None, stream=None):
    """csa_index_topk: q_idx [B, Tq, Hi, Di] bf16, w [B, Tq, Hi] fp32, q_pos [B, Tq] int64."""
    assert q_idx.dtype == torch.bfloat16 and q_idx.is_contiguous()
    assert w.dtype == torch.float32 and w.is_contiguous() and q_pos.dtype == torch.int64
    assert idx_out.dtype == torch.int32 and idx_out.is_contiguous()
    B, Tq, Hi, _ = q_idx.shape
    c = keys.struct()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load().csa_index_topk(q_idx.data_ptr(), w.data_ptr(), q_pos.data_ptr(), B, Tq, Hi, ctypes.byref(c),
                               topk, idx_out.data_ptr(), _ptr(scores_out), _ptr(workspace), ws_bytes,
                               _stream(stream))
    _check("csa_index_topk", rc)


def index_topk_compress(calls, q_idx: torch.Tensor, w: torch.Tensor, q_pos: torch.Tensor, keys: Cache, topk: int,
                        idx_out: torch.Tensor, scores_out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None):
    """csa_index_topk_compress: compress_batch(calls) and index_topk(...) with fewer launches."""
    assert q_idx.dtype == torch.bfloat16 and q_idx.is_contiguous()
    assert w.dtype == torch.float32 and w.is_contiguous() and q_pos.dtype == torch.int64
    assert idx_out.dtype == torch.int32 and idx_out.is_contiguous()
    arr, keep = _compress_calls(calls)
    B, Tq, Hi, _ = q_idx.shape
    c = keys.struct()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load().csa_index_topk_compress(arr, len(calls), q_idx.data_ptr(), w.data_ptr(), q_pos.data_ptr(), B, Tq,
                                        Hi, ctypes.byref(c), topk, idx_out.data_ptr(), _ptr(scores_out),
                                        _ptr(workspace), ws_bytes, _stream(stream))
    _check("csa_index_topk_compress", rc)


def csa_attend_workspace_bytes(B, Tq, H, topk, W) -> int:
    return load().csa_attend_workspace_bytes(B, Tq, H, topk, W)


def hca_attend_workspace_bytes(B, Tq, H, cap, W) -> int:
    return load().hca_attend_workspace_bytes(B, Tq, H, cap, W)


def _out_code(out: torch.Tensor) -> int:
    if out.dtype == torch.float32:
        return CSA_FP32
    if out.dtype == torch.bfloat16:
        return CSA_BF16
    raise TypeError(f"unsupported output dtype {out.dtype}")


def csa_attend(q: torch.Tensor, q_pos: torch.Tensor, kv: Cache, idx: torch.Tensor, win: Cache, W: int,
               sink: torch.Tensor, inv_freq: Optional[torch.Tensor], rope_dim: int, softmax_scale: float,
               out: torch.Tensor, lse: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None, stream=None):
    """csa_attend: q [B, Tq, H, 512] bf16; idx [B, Tq, topk] int32; out [B, Tq, H, 512]."""
    assert q.dtype == torch.bfloat16 and q.is_contiguous() and out.is_contiguous()
    assert idx.dtype == torch.int32 and idx.is_contiguous()
    B, Tq, H, _ = q.shape
    ck, cw = kv.struct(), win.struct()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load().csa_attend(q.data_ptr(), q_pos.data_ptr(), B, Tq, H, ctypes.byref(ck), idx.data_ptr(),
                           idx.shape[-1], ctypes.byref(cw), W, sink.data_ptr(), _ptr(inv_freq), rope_dim,
                           softmax_scale, out.data_ptr(), _out_code(out), _ptr(lse), _ptr(workspace), ws_bytes,
                           _stream(stream))
    _check("csa_attend", rc)


def csa_attend_noalloc(q: torch.Tensor, q_pos: torch.Tensor, kv: Cache, idx: torch.Tensor, win: Cache, W: int,
                       sink: torch.Tensor, inv_freq: Optional[torch.Tensor], rope_dim: int, softmax_scale: float,
                       out: torch.Tensor, lse: Optional[torch.Tensor] = None, stream=None):
    """csa_attend_noalloc: csa_attend with the library's own scratch instead of a workspace."""
    assert q.dtype == torch.bfloat16 and q.is_contiguous() and out.is_contiguous()
    assert idx.dtype == torch.int32 and idx.is_contiguous()
    B, Tq, H, _ = q.shape
    ck, cw = kv.struct(), win.struct()
    rc = load().csa_attend_noalloc(q.data_ptr(), q_pos.data_ptr(), B, Tq, H, ctypes.byref(ck), idx.data_ptr(),
                                   idx.shape[-1], ctypes.byref(cw), W, sink.data_ptr(), _ptr(inv_freq), rope_dim,
                                   softmax_scale, out.data_ptr(), _out_code(out), _ptr(lse), _stream(stream))
    _check("csa_attend_noalloc", rc)


def hca_attend(q: torch.Tensor, q_pos: torch.Tensor, kv: Cache, win: Cache, W: int, sink: torch.Tensor,
               inv_freq: Optional[torch.Tensor], rope_dim: int, softmax_scale: float, out: torch.Tensor,
               lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """hca_attend: every visible entry of kv plus the window."""
    assert q.dtype == torch.bfloat16 and q.is_contiguous() and out.is_contiguous()
    B, Tq, H, _ = q.shape
    ck, cw = kv.struct(), win.struct()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load().hca_attend(q.data_ptr(), q_pos.data_ptr(), B, Tq, H, ctypes.byref(ck), ctypes.byref(cw), W,
                           sink.data_ptr(), _ptr(inv_freq), rope_dim, softmax_scale, out.data_ptr(),
                           _out_code(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream))
    _check("hca_attend", rc)


def csa_out_proj_workspace_bytes(T: int, G: int, R: int, hidden: int) -> int:
    return int(load().csa_out_proj_workspace_bytes(T, G, R, hidden))


def csa_out_proj(o: torch.Tensor, wa: torch.Tensor, wb: torch.Tensor, y: torch.Tensor,
                 workspace: Optional[torch.Tensor] = None, stream=None):
    """csa_out_proj: o [T, H, D] (fp32 or bf16), wa bf16 [G, R, (H/G) D], wb bf16 [hidden, G R] -> y [T, hidden]."""
    assert o.is_contiguous() and wa.is_contiguous() and wb.is_contiguous() and y.is_contiguous()
    assert wa.dtype == torch.bfloat16 and wb.dtype == torch.bfloat16
    T, H, D = o.shape
    G, R, _ = wa.shape
    hidden = wb.shape[0]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load().csa_out_proj(o.data_ptr(), _out_code(o), T, H, D, G, wa.data_ptr(), R, wb.data_ptr(), hidden,
                             y.data_ptr(), _out_code(y), _ptr(workspace), ws_bytes, _stream(stream))
    _check("csa_out_proj", rc)


def workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    """A 256-byte-aligned byte tensor of at least nbytes (None when nbytes == 0)."""
    if nbytes <= 0:
        return None
    t = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-t.data_ptr()) % 256
    return t[off:off + nbytes]
