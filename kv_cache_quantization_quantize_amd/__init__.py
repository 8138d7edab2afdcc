"""Python binding of libkvq.so, the MI355X (gfx950) fused KV-cache quantizer.

Argument marshalling only: every step of the quantizer runs in the library's
HIP kernels.  PyTorch provides device memory and the current HIP stream.  If
the library has not been built, every call raises -- there is no fallback.

Functions (names as in include/kvq.h):
    quantize(x, lam, signs, group)            -> (codes u8, scales fp16)
    dequantize(codes, scales, lam, signs, group) -> fp16
    vq_encode(x, lam, signs, codebook)        -> indices (int16 storage of uint16)
    vq_decode(idx, codebook, lam, signs)      -> fp16
    append_quantize(x_tok, cache_codes, cache_scales, t, lam, signs, group)
KV tensors are [layers, tokens, heads, head_dim] with the last dimension
contiguous; lam is fp32 [layers, heads, head_dim]; signs int8 [head_dim].
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "KvqError", "lib", "library_path", "quantize", "dequantize", "vq_encode", "vq_decode",
    "append_quantize", "Shape", "View", "STATUS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkvq.so")
_lib = None

STATUS = {0: "KVQ_OK", 1: "KVQ_ERR_NULL", 2: "KVQ_ERR_SHAPE", 3: "KVQ_ERR_ALIGN",
          4: "KVQ_ERR_UNSUPPORTED", 5: "KVQ_ERR_HIP"}


class KvqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS.get(status, status), message))
        self.status = status
        self.message = message


class Shape(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int64), ("tokens", ctypes.c_int64),
                ("heads", ctypes.c_int64), ("head_dim", ctypes.c_int64)]


class View(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_layer", ctypes.c_int64),
                ("stride_token", ctypes.c_int64), ("stride_head", ctypes.c_int64)]


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded libkvq.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libkvq.so is not built (%s); run "
                           "`python -m kv_cache_quantization_quantize_amd.build`" % _LIB_PATH)
    L = ctypes.CDLL(_LIB_PATH)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.kvq_quantize.restype = ctypes.c_int
    L.kvq_quantize.argtypes = [Shape, View, P, P, I32, View, View, P]
    L.kvq_dequantize.restype = ctypes.c_int
    L.kvq_dequantize.argtypes = [Shape, View, View, P, P, I32, View, P]
    L.kvq_quantize_srft.restype = ctypes.c_int
    L.kvq_quantize_srft.argtypes = [Shape, View, P, P, I32, View, View, P]
    L.kvq_dequantize_srft.restype = ctypes.c_int
    L.kvq_dequantize_srft.argtypes = [Shape, View, View, P, P, I32, View, P]
    L.kvq_quantize_int8.restype = ctypes.c_int
    L.kvq_quantize_int8.argtypes = [Shape, View, P, P, I32, View, View, P]
    L.kvq_dequantize_int8.restype = ctypes.c_int
    L.kvq_dequantize_int8.argtypes = [Shape, View, View, P, P, I32, View, P]
    L.kvq_quantize_mxfp4.restype = ctypes.c_int
    L.kvq_quantize_mxfp4.argtypes = [Shape, View, P, P, View, View, P]
    L.kvq_dequantize_mxfp4.restype = ctypes.c_int
    L.kvq_dequantize_mxfp4.argtypes = [Shape, View, View, P, P, View, P]
    L.kvq_vq_encode.restype = ctypes.c_int
    L.kvq_vq_encode.argtypes = [Shape, View, P, P, P, I64, I32, I32, View, P]
    L.kvq_vq_decode.restype = ctypes.c_int
    L.kvq_vq_decode.argtypes = [Shape, View, P, I64, I32, I32, P, P, View, P]
    L.kvq_kmeans_step_workspace.restype = ctypes.c_int
    L.kvq_kmeans_step_workspace.argtypes = [Shape, I32, I32, ctypes.POINTER(ctypes.c_int64)]
    L.kvq_kmeans_step.restype = ctypes.c_int
    L.kvq_kmeans_step.argtypes = [Shape, View, P, P, P, I32, I32, View, P, P, P, I64, P]
    L.kvq_vq_encode_u8.restype = ctypes.c_int
    L.kvq_vq_encode_u8.argtypes = [Shape, View, P, P, P, I64, I32, I32, View, P]
    L.kvq_vq_decode_u8.restype = ctypes.c_int
    L.kvq_vq_decode_u8.argtypes = [Shape, View, P, I64, I32, I32, P, P, View, P]
    L.kvq_attend_decode.restype = ctypes.c_int
    L.kvq_attend_decode.argtypes = [Shape, I32, P, View, View, View, View, P, P, P, I32, P, ctypes.c_float, P, P,
                                    I64, P]
    L.kvq_attend_decode_noalloc.restype = ctypes.c_int
    L.kvq_attend_decode_noalloc.argtypes = [Shape, I32, P, View, View, View, View, P, P, P, I32, P, ctypes.c_float,
                                            P, P]
    L.kvq_attend_decode_workspace.restype = ctypes.c_int
    L.kvq_attend_decode_workspace.argtypes = [Shape, I32, ctypes.POINTER(I64)]
    L.kvq_item_plan.restype = ctypes.c_int
    L.kvq_item_plan.argtypes = [Shape, I32, I32, ctypes.POINTER(I32), ctypes.POINTER(I64), ctypes.POINTER(I32)]
    L.kvq_status_string.restype = ctypes.c_char_p
    L.kvq_status_string.argtypes = [ctypes.c_int]
    L.kvq_last_error.restype = ctypes.c_char_p
    L.kvq_last_error.argtypes = []
    L.kvq_version.restype = I32
    L.kvq_version.argtypes = []
    _lib = L
    return L


def _check(st: int):
    if st != 0:
        raise KvqError(st, lib().kvq_last_error().decode())


# ----------------------------------------------------------------- helpers
def _torch():
    import torch
    return torch


def _view(t) -> View:
    """View of a 4-D tensor [L, T, H, row] whose last dimension is contiguous."""
    if t.dim() != 4:
        raise ValueError("expected a 4-D [layers, tokens, heads, row] tensor, got %s" % (tuple(t.shape),))
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    s = t.stride()
    return View(ctypes.c_void_p(t.data_ptr()), s[0], s[1], s[2])


def _shape(t, D: int) -> Shape:
    return Shape(t.shape[0], t.shape[1], t.shape[2], D)


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device" % name)


def _params(lam, signs, L, H, D):
    torch = _torch()
    _need(lam, torch.float32, "lam")
    _need(signs, torch.int8, "signs")
    if tuple(lam.shape) != (L, H, D) or not lam.is_contiguous():
        raise ValueError("lam must be a contiguous fp32 [layers, heads, head_dim] = %s tensor" % ((L, H, D),))
    if tuple(signs.shape) != (D,) or not signs.is_contiguous():
        raise ValueError("signs must be a contiguous int8 [head_dim] tensor")
    return ctypes.c_void_p(lam.data_ptr()), ctypes.c_void_p(signs.data_ptr())


# ------------------------------------------------------------------ int4
def quantize(x, lam, signs, group: int, codes=None, scales=None, stream=None, _fn="kvq_quantize"):
    """Fused rotate + int4 quantize of x [L, T, H, D] fp16 -> (codes [L, T, H, D/2]
    uint8, scales [L, T, H, D/group] fp16)."""
    torch = _torch()
    _need(x, torch.float16, "x")
    L, T, H, D = x.shape
    if codes is None:
        codes = torch.empty((L, T, H, D // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((L, T, H, max(D // max(group, 1), 1)), dtype=torch.float16, device=x.device)
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.float16, "scales")
    pl, ps = _params(lam, signs, L, H, D)
    _check(getattr(lib(), _fn)(_shape(x, D), _view(x), pl, ps, int(group), _view(codes), _view(scales),
                               _stream(stream)))
    return codes, scales


def dequantize(codes, scales, lam, signs, group: int, out=None, stream=None, _fn="kvq_dequantize"):
    """Mirror of quantize: (codes, scales) -> fp16 [L, T, H, D]."""
    torch = _torch()
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.float16, "scales")
    L, T, H, half = codes.shape
    D = 2 * half
    if out is None:
        out = torch.empty((L, T, H, D), dtype=torch.float16, device=codes.device)
    _need(out, torch.float16, "out")
    pl, ps = _params(lam, signs, L, H, D)
    _check(getattr(lib(), _fn)(_shape(codes, D), _view(codes), _view(scales), pl, ps, int(group), _view(out),
                               _stream(stream)))
    return out


def quantize_srft(x, lam, signs, group: int, codes=None, scales=None, stream=None):
    """quantize() with the SRFT rotation (real-packed unitary DFT) instead of
    the Walsh-Hadamard one."""
    return quantize(x, lam, signs, group, codes, scales, stream, _fn="kvq_quantize_srft")


def dequantize_srft(codes, scales, lam, signs, group: int, out=None, stream=None):
    """Mirror of quantize_srft."""
    return dequantize(codes, scales, lam, signs, group, out, stream, _fn="kvq_dequantize_srft")


def append_quantize(x_tok, cache_codes, cache_scales, t: int, lam, signs, group: int, stream=None):
    """Decode-time append: quantize x_tok [L, 1, H, D] into token slot t of
    preallocated caches [L, Tmax, H, D/2] / [L, Tmax, H, D/group] (a tokens=1
    call on views that start at slot t)."""
    c = cache_codes[:, t:t + 1]
    s = cache_scales[:, t:t + 1]
    quantize(x_tok, lam, signs, group, codes=c, scales=s, stream=stream)
    return c, s


# ------------------------------------------------------------------ int8
def quantize_int8(x, lam, signs, group: int, codes=None, scales=None, stream=None):
    """int8 variant of quantize: x [L, T, H, D] fp16 -> (codes int8 [L, T, H, D],
    scales fp16 [L, T, H, D/group])."""
    torch = _torch()
    _need(x, torch.float16, "x")
    L, T, H, D = x.shape
    if codes is None:
        codes = torch.empty((L, T, H, D), dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty((L, T, H, D // group), dtype=torch.float16, device=x.device)
    _need(codes, torch.int8, "codes")
    _need(scales, torch.float16, "scales")
    pl, ps = _params(lam, signs, L, H, D)
    _check(lib().kvq_quantize_int8(_shape(x, D), _view(x), pl, ps, int(group), _view(codes), _view(scales),
                                   _stream(stream)))
    return codes, scales


def dequantize_int8(codes, scales, lam, signs, group: int, out=None, stream=None):
    """Mirror of quantize_int8: (codes int8, scales) -> fp16 [L, T, H, D]."""
    torch = _torch()
    _need(codes, torch.int8, "codes")
    _need(scales, torch.float16, "scales")
    L, T, H, D = codes.shape
    if out is None:
        out = torch.empty((L, T, H, D), dtype=torch.float16, device=codes.device)
    _need(out, torch.float16, "out")
    pl, ps = _params(lam, signs, L, H, D)
    _check(lib().kvq_dequantize_int8(_shape(codes, D), _view(codes), _view(scales), pl, ps, int(group), _view(out),
                                     _stream(stream)))
    return out


# ----------------------------------------------------------------- MXFP4
def quantize_mxfp4(x, lam, signs, codes=None, scales=None, stream=None):
    """Block-scaled E2M1 variant of quantize: x [L, T, H, D] fp16 -> (codes
    uint8 [L, T, H, D/2] packed E2M1 nibbles, scales uint8 [L, T, H, D/32]
    E8M0 bytes)."""
    torch = _torch()
    _need(x, torch.float16, "x")
    L, T, H, D = x.shape
    if codes is None:
        codes = torch.empty((L, T, H, D // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((L, T, H, D // 32), dtype=torch.uint8, device=x.device)
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.uint8, "scales")
    pl, ps = _params(lam, signs, L, H, D)
    _check(lib().kvq_quantize_mxfp4(_shape(x, D), _view(x), pl, ps, _view(codes), _view(scales), _stream(stream)))
    return codes, scales


def dequantize_mxfp4(codes, scales, lam, signs, out=None, stream=None):
    """Mirror of quantize_mxfp4 -> fp16 [L, T, H, D]."""
    torch = _torch()
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.uint8, "scales")
    L, T, H, half = codes.shape
    D = 2 * half
    if out is None:
        out = torch.empty((L, T, H, D), dtype=torch.float16, device=codes.device)
    _need(out, torch.float16, "out")
    pl, ps = _params(lam, signs, L, H, D)
    _check(lib().kvq_dequantize_mxfp4(_shape(codes, D), _view(codes), _view(scales), pl, ps, _view(out),
                                      _stream(stream)))
    return out


# -------------------------------------------------------------------- VQ
def _vq_encode(x, lam, signs, codebook, sub_dim, idx, codebook_layer_stride, stream, u8):
    torch = _torch()
    _need(x, torch.float16, "x")
    _need(codebook, torch.float16, "codebook")
    L, T, H, D = x.shape
    K = codebook.shape[-2]
    if not codebook.is_contiguous():
        raise ValueError("codebook must be contiguous")
    dt = torch.uint8 if u8 else torch.int16
    if idx is None:
        idx = torch.empty((L, T, H, D // sub_dim), dtype=dt, device=x.device)
    _need(idx, dt, "idx")
    pl, ps = _params(lam, signs, L, H, D)
    fn = lib().kvq_vq_encode_u8 if u8 else lib().kvq_vq_encode
    _check(fn(_shape(x, D), _view(x), pl, ps, ctypes.c_void_p(codebook.data_ptr()), int(codebook_layer_stride),
              int(K), int(sub_dim), _view(idx), _stream(stream)))
    return idx


def _vq_decode(idx, codebook, lam, signs, sub_dim, out, codebook_layer_stride, stream, u8):
    torch = _torch()
    _need(idx, torch.uint8 if u8 else torch.int16, "idx")
    _need(codebook, torch.float16, "codebook")
    L, T, H, nsub = idx.shape
    D = nsub * sub_dim
    K = codebook.shape[-2]
    if out is None:
        out = torch.empty((L, T, H, D), dtype=torch.float16, device=idx.device)
    _need(out, torch.float16, "out")
    pl, ps = _params(lam, signs, L, H, D)
    fn = lib().kvq_vq_decode_u8 if u8 else lib().kvq_vq_decode
    _check(fn(_shape(idx, D), _view(idx), ctypes.c_void_p(codebook.data_ptr()), int(codebook_layer_stride), int(K),
              int(sub_dim), pl, ps, _view(out), _stream(stream)))
    return out


def vq_encode(x, lam, signs, codebook, sub_dim: int = 8, idx=None, codebook_layer_stride: int = 0,
              stream=None):
    """Product-VQ encode of x [L, T, H, D] fp16 against codebook [H, K, sub_dim]
    fp16 (or [L, H, K, sub_dim] with codebook_layer_stride = H*K*sub_dim) ->
    indices [L, T, H, D/sub_dim] stored in an int16 tensor (read as uint16)."""
    return _vq_encode(x, lam, signs, codebook, sub_dim, idx, codebook_layer_stride, stream, False)


def vq_decode(idx, codebook, lam, signs, sub_dim: int = 8, out=None, codebook_layer_stride: int = 0,
              stream=None):
    """Product-VQ decode: indices [L, T, H, D/sub_dim] -> fp16 [L, T, H, D]."""
    return _vq_decode(idx, codebook, lam, signs, sub_dim, out, codebook_layer_stride, stream, False)


def vq_encode_u8(x, lam, signs, codebook, sub_dim: int = 8, idx=None, codebook_layer_stride: int = 0,
                 stream=None):
    """vq_encode with one-byte indices (codebooks of at most 256 centroids) ->
    uint8 [L, T, H, D/sub_dim]."""
    return _vq_encode(x, lam, signs, codebook, sub_dim, idx, codebook_layer_stride, stream, True)


def vq_decode_u8(idx, codebook, lam, signs, sub_dim: int = 8, out=None, codebook_layer_stride: int = 0,
                 stream=None):
    """vq_decode of uint8 indices -> fp16 [L, T, H, D]."""
    return _vq_decode(idx, codebook, lam, signs, sub_dim, out, codebook_layer_stride, stream, True)


# ------------------------------------------------------ codebook training
def kmeans_step_workspace_bytes(L: int, T: int, H: int, D: int, n_centroids: int, sub_dim: int = 8) -> int:
    n = ctypes.c_int64(0)
    _check(lib().kvq_kmeans_step_workspace(Shape(L, T, H, D), int(n_centroids), int(sub_dim), ctypes.byref(n)))
    return int(n.value)


def kmeans_step(x, lam, signs, codebook, sub_dim: int = 8, idx=None, new_codebook=None, counts=None,
                workspace=None, stream=None):
    """One Lloyd iteration for the per-head codebooks [H, K, sub_dim] (fp16)
    on the samples x [L, T, H, D] fp16 -> (idx int16 [L, T, H, D/sub_dim]
    assignments to the input codebook, new codebook fp16 [H, K, sub_dim],
    counts int32 [H, K] (read as uint32))."""
    torch = _torch()
    _need(x, torch.float16, "x")
    _need(codebook, torch.float16, "codebook")
    if not codebook.is_contiguous():
        raise ValueError("codebook must be contiguous")
    L, T, H, D = x.shape
    K = codebook.shape[-2]
    if idx is None:
        idx = torch.empty((L, T, H, D // sub_dim), dtype=torch.int16, device=x.device)
    _need(idx, torch.int16, "idx")
    if new_codebook is None:
        new_codebook = torch.empty_like(codebook)
    _need(new_codebook, torch.float16, "new_codebook")
    if not new_codebook.is_contiguous():
        raise ValueError("new_codebook must be contiguous")
    if counts is None:
        counts = torch.empty((H, K), dtype=torch.int32, device=x.device)
    _need(counts, torch.int32, "counts")
    if tuple(counts.shape) != (H, K) or not counts.is_contiguous():
        raise ValueError("counts must be a contiguous int32 [heads, n_centroids] tensor")
    if tuple(new_codebook.shape) != tuple(codebook.shape):
        raise ValueError("new_codebook must have the codebook's shape")
    need = kmeans_step_workspace_bytes(L, T, H, D, K, sub_dim)
    if workspace is None:
        workspace = torch.empty(max(16, need), dtype=torch.uint8, device=x.device)
    _need(workspace, torch.uint8, "workspace")
    pl, ps = _params(lam, signs, L, H, D)
    _check(lib().kvq_kmeans_step(_shape(x, D), _view(x), pl, ps, ctypes.c_void_p(codebook.data_ptr()), int(K),
                                 int(sub_dim), _view(idx), ctypes.c_void_p(new_codebook.data_ptr()),
                                 ctypes.c_void_p(counts.data_ptr()), ctypes.c_void_p(workspace.data_ptr()),
                                 int(workspace.numel()), _stream(stream)))
    return idx, new_codebook, counts


# -------------------------------------------------------- decode attention
def attend_decode_workspace_bytes(L: int, T: int, H: int, D: int, q_per_kv: int) -> int:
    """Workspace bytes attend_decode needs for this shape on the current device."""
    b = ctypes.c_int64(0)
    _check(lib().kvq_attend_decode_workspace(Shape(L, T, H, D), int(q_per_kv), ctypes.byref(b)))
    return int(b.value)


def attend_decode(q, k_codes, k_scales, v_codes, v_scales, lam_k, lam_v, signs, group: int,
                  softmax_scale=None, lengths=None, out=None, workspace=None, stream=None, noalloc=False):
    """One decode step of attention over int4 caches.  q [L, H*R, D] fp16
    (R query heads per KV head), caches [L, T, H, D/2] u8 and [L, T, H, D/G]
    fp16 as written by quantize, lam_k / lam_v [L, H, D] fp32, lengths [L]
    int32 or None -> fp16 [L, H*R, D].  The workspace (a uint8 tensor) is
    allocated here when not given.  noalloc: call kvq_attend_decode_noalloc,
    which keeps the partial states in the library's static device scratch
    (out must then be given to allocate nothing at all)."""
    torch = _torch()
    for t, dt, name in ((q, torch.float16, "q"), (k_codes, torch.uint8, "k_codes"),
                        (k_scales, torch.float16, "k_scales"), (v_codes, torch.uint8, "v_codes"),
                        (v_scales, torch.float16, "v_scales")):
        _need(t, dt, name)
    L, T, H, half = k_codes.shape
    D = 2 * half
    if q.dim() != 3 or q.shape[0] != L or q.shape[2] != D or q.shape[1] % H or not q.is_contiguous():
        raise ValueError("q must be a contiguous fp16 [layers, heads*q_per_kv, head_dim] tensor")
    R = q.shape[1] // H
    if tuple(v_codes.shape) != (L, T, H, half):
        raise ValueError("v_codes must match k_codes in shape")
    pk, ps = _params(lam_k, signs, L, H, D)
    pv, _ = _params(lam_v, signs, L, H, D)
    if out is None:
        out = torch.empty_like(q)
    _need(out, torch.float16, "out")
    if tuple(out.shape) != tuple(q.shape) or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped like q")
    pl = None
    if lengths is not None:
        _need(lengths, torch.int32, "lengths")
        if tuple(lengths.shape) != (L,) or not lengths.is_contiguous():
            raise ValueError("lengths must be a contiguous int32 [layers] tensor")
        pl = ctypes.c_void_p(lengths.data_ptr())
    scale = (1.0 / D ** 0.5) if softmax_scale is None else float(softmax_scale)
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc takes no workspace")
        _check(lib().kvq_attend_decode_noalloc(Shape(L, T, H, D), int(R), ctypes.c_void_p(q.data_ptr()),
                                               _view(k_codes), _view(k_scales), _view(v_codes), _view(v_scales),
                                               pk, pv, ps, int(group), pl, scale, ctypes.c_void_p(out.data_ptr()),
                                               _stream(stream)))
        return out
    need = attend_decode_workspace_bytes(L, T, H, D, R)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, torch.uint8, "workspace")
    _check(lib().kvq_attend_decode(Shape(L, T, H, D), int(R), ctypes.c_void_p(q.data_ptr()), _view(k_codes),
                                   _view(k_scales), _view(v_codes), _view(v_scales), pk, pv, ps, int(group), pl,
                                   scale, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(workspace.data_ptr()),
                                   int(workspace.numel()), _stream(stream)))
    return out


# ------------------------------------------------------ work decomposition
def item_plan(L: int, T: int, H: int, D: int, inverse: bool = False, fourier: bool = False):
    """(token_major, n_items, items_per_wave) of the quantize (or, with
    inverse, dequantize) kernels of the Walsh-Hadamard formats (or, with
    fourier, SRFT) for a [L, T, H, D] tensor (host arithmetic only)."""
    tm, n, ipw = ctypes.c_int32(0), ctypes.c_int64(0), ctypes.c_int32(0)
    _check(lib().kvq_item_plan(Shape(L, T, H, D), int(bool(inverse)), int(bool(fourier)), ctypes.byref(tm),
                               ctypes.byref(n), ctypes.byref(ipw)))
    return bool(tm.value), int(n.value), int(ipw.value)
