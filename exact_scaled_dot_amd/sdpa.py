"""ctypes binding of libsdpa (include/sdpa.h).

Argument marshalling only: tensor shapes become the C sizes, data pointers and
torch's current HIP stream are passed through, and every step of the
computation runs in the library's HIP kernels.  If libsdpa.so is not built the
first call raises; there is no fallback path.
"""

import ctypes
import os

import torch

# Mirrors of the C enums in include/sdpa.h.
SDPA_OK = 0
SDPA_ERR_INVALID_ARGUMENT = 1
SDPA_ERR_UNSUPPORTED = 2
SDPA_ERR_WORKSPACE = 3
SDPA_ERR_HIP = 4
SDPA_F32 = 0
SDPA_BF16 = 1
SDPA_F16 = 2
MASK_NONE = 0
MASK_CAUSAL = 1
MASK_KEY_PADDING = 2
MAX_SPLITS = 32
NOALLOC_SCRATCH_BYTES = 64 << 20   # SDPA_NOALLOC_SCRATCH_BYTES

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsdpa.so")

EXPORTED = ("sdpa_forward", "sdpa_forward_lse", "sdpa_forward_bias", "sdpa_backward",
            "sdpa_backward_workspace_size", "sdpa_backward_atomic",
            "sdpa_backward_atomic_workspace_size", "sdpa_backward_bias", "sdpa_block_forward",
            "sdpa_block_workspace_size",
            "sdpa_decode", "sdpa_decode_workspace_size", "sdpa_decode_noalloc",
            "sdpa_paged_attention",
            "sdpa_paged_prefill", "sdpa_paged_backward", "sdpa_paged_backward_workspace_size",
            "sdpa_status_string", "sdpa_last_error")

_lib = None


class SdpaError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__("libsdpa: %s (%d): %s" % (status_string(status), status, detail))


def load_library():
    """Load libsdpa.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libsdpa.so is not built (%s); run `python -m exact_scaled_dot_amd.build`"
                           % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.sdpa_forward.restype = i32
    lib.sdpa_forward.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_float, i32, vp,
                                 vp, i32, vp]
    lib.sdpa_forward_lse.restype = i32
    lib.sdpa_forward_lse.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_float, i32,
                                     vp, vp, vp, i32, vp]
    lib.sdpa_forward_bias.restype = i32
    lib.sdpa_forward_bias.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_float, i32,
                                      vp, vp, i64, i64, vp, vp, i32, vp]
    lib.sdpa_backward_workspace_size.restype = ctypes.c_size_t
    lib.sdpa_backward_workspace_size.argtypes = [i64, i64, i64]
    lib.sdpa_backward.restype = i32
    lib.sdpa_backward.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                  ctypes.c_float, i32, vp, vp, vp, vp, vp, ctypes.c_size_t, i32, vp]
    lib.sdpa_backward_atomic.restype = i32
    lib.sdpa_backward_atomic.argtypes = lib.sdpa_backward.argtypes
    lib.sdpa_backward_bias.restype = i32
    lib.sdpa_backward_bias.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                       ctypes.c_float, i32, vp, vp, i64, i64, vp, vp, vp, vp, vp,
                                       ctypes.c_size_t, i32, vp]
    lib.sdpa_backward_atomic_workspace_size.restype = ctypes.c_size_t
    lib.sdpa_backward_atomic_workspace_size.argtypes = [i64, i64, i64, i64]
    lib.sdpa_block_workspace_size.restype = ctypes.c_size_t
    lib.sdpa_block_workspace_size.argtypes = [i64, i64, i64]
    lib.sdpa_block_forward.restype = i32
    lib.sdpa_block_forward.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float, i32,
                                       vp, vp, vp, ctypes.c_size_t, i32, vp]
    lib.sdpa_decode.restype = i32
    lib.sdpa_decode.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float, vp, i32, vp,
                                ctypes.c_size_t, vp, i32, vp]
    lib.sdpa_decode_noalloc.restype = i32
    lib.sdpa_decode_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float, vp,
                                        i32, vp, i32, vp]
    lib.sdpa_decode_workspace_size.restype = ctypes.c_size_t
    lib.sdpa_decode_workspace_size.argtypes = [i64, i64, i64, i32]
    lib.sdpa_paged_attention.restype = i32
    lib.sdpa_paged_attention.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, vp, i64, i64,
                                         vp, vp, vp, i64, ctypes.c_float, i32, i32, vp,
                                         ctypes.c_size_t, vp, i32, vp]
    lib.sdpa_paged_prefill.restype = i32
    lib.sdpa_paged_prefill.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, vp, i64, i64, vp,
                                       vp, i64, i64, ctypes.c_float, i32, vp, vp, i32, vp]
    lib.sdpa_paged_backward_workspace_size.restype = ctypes.c_size_t
    lib.sdpa_paged_backward_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, i32]
    lib.sdpa_paged_backward.restype = i32
    lib.sdpa_paged_backward.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, vp,
                                        i64, i64, vp, vp, i64, ctypes.c_float, i32, vp, vp, vp, vp,
                                        ctypes.c_size_t, i32, vp]
    lib.sdpa_status_string.restype = ctypes.c_char_p
    lib.sdpa_status_string.argtypes = [i32]
    lib.sdpa_last_error.restype = ctypes.c_char_p
    lib.sdpa_last_error.argtypes = []
    _lib = lib
    return lib


def status_string(status):
    return load_library().sdpa_status_string(status).decode()


def last_error():
    return load_library().sdpa_last_error().decode()


def _check(status):
    if status != SDPA_OK:
        raise SdpaError(status, last_error())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return SDPA_BF16
    if t.dtype == torch.float16:
        return SDPA_F16
    if t.dtype == torch.float32:
        return SDPA_F32
    raise TypeError("libsdpa supports bfloat16, float16 and float32 tensors, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_tensor(name, t, ndim):
    if not isinstance(t, torch.Tensor) or t.dim() != ndim:
        raise ValueError("%s must be a %d-D torch tensor" % (name, ndim))
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _check_qkv(q, k, v, key_lens):
    """Shape / dtype checks shared by the dense entry points; returns the sizes."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, 4)
    if key_lens is not None:
        _check_tensor("key_lens", key_lens, 1)
        if key_lens.dtype != torch.int32:
            raise TypeError("key_lens must be int32")
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Sk, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, Sk, D] matching q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    return B, Hq, Hkv, Sq, Sk, D


def sdpa_forward(q, k, v, scale, mask_kind=MASK_NONE, key_lens=None, out=None, stream=None):
    """O = softmax(Q K^T * scale + mask) V.  q [B,Hq,Sq,D], k/v [B,Hkv,Sk,D]."""
    B, Hq, Hkv, Sq, Sk, D = _check_qkv(q, k, v, key_lens)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor("out", out, 4)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q in shape and dtype")
    lib = load_library()
    _check(lib.sdpa_forward(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, Sq, Sk, D, float(scale),
                            int(mask_kind), _ptr(key_lens), _ptr(out), _dtype_code(q),
                            _stream(stream)))
    return out


def sdpa_forward_lse(q, k, v, scale, mask_kind=MASK_NONE, key_lens=None, out=None, lse=None,
                     stream=None):
    """sdpa_forward that also returns each row's log-sum-exp: (out, lse [B,Hq,Sq] fp32)."""
    B, Hq, Hkv, Sq, Sk, D = _check_qkv(q, k, v, key_lens)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor("out", out, 4)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q in shape and dtype")
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    else:
        _check_tensor("lse", lse, 3)
        if tuple(lse.shape) != (B, Hq, Sq) or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [B, Hq, Sq]")
    lib = load_library()
    _check(lib.sdpa_forward_lse(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, Sq, Sk, D, float(scale),
                                int(mask_kind), _ptr(key_lens), _ptr(out), _ptr(lse),
                                _dtype_code(q), _stream(stream)))
    return out, lse


def _bias_strides(bias, q, B, Hq, Sq, Sk):
    """Validate a [B or 1, Hq or 1, Sq, Sk] bias; its batch and head strides (0 if broadcast)."""
    if not isinstance(bias, torch.Tensor) or bias.dim() != 4 or not bias.is_cuda:
        raise ValueError("bias must be a 4-D device tensor")
    if bias.dtype != q.dtype:
        raise TypeError("bias must have q's dtype")
    if (bias.shape[0] not in (1, B) or bias.shape[1] not in (1, Hq)
            or tuple(bias.shape[2:]) != (Sq, Sk)):
        raise ValueError("bias must be [B or 1, Hq or 1, Sq, Sk]")
    if bias.stride(3) != 1 or bias.stride(2) != Sk:
        raise ValueError("bias rows must be contiguous (stride Sk between rows)")
    return (bias.stride(0) if bias.shape[0] > 1 else 0, bias.stride(1) if bias.shape[1] > 1 else 0)


def sdpa_forward_bias(q, k, v, bias, scale, mask_kind=MASK_NONE, key_lens=None, out=None,
                      lse=None, stream=None):
    """O = softmax(Q K^T * scale + bias + mask) V.

    bias is [B or 1, Hq or 1, Sq, Sk] in q's dtype, contiguous in its last two
    axes (a size-1 leading axis broadcasts).  lse: None, or True to allocate
    and return it, or a float32 [B, Hq, Sq] tensor.  Returns out, or
    (out, lse) when lse is requested.
    """
    B, Hq, Hkv, Sq, Sk, D = _check_qkv(q, k, v, key_lens)
    sb, sh = _bias_strides(bias, q, B, Hq, Sq, Sk)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor("out", out, 4)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q in shape and dtype")
    want_lse = lse is not None
    if lse is True:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_tensor("lse", lse, 3)
        if tuple(lse.shape) != (B, Hq, Sq) or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [B, Hq, Sq]")
    lib = load_library()
    _check(lib.sdpa_forward_bias(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, Sq, Sk, D, float(scale),
                                 int(mask_kind), _ptr(key_lens), _ptr(bias), sb, sh, _ptr(out),
                                 _ptr(lse), _dtype_code(q), _stream(stream)))
    return (out, lse) if want_lse else out


def sdpa_backward_workspace_size(B, Hq, Sq):
    return int(load_library().sdpa_backward_workspace_size(B, Hq, Sq))


def sdpa_backward_atomic_workspace_size(B, Hq, Sq, D):
    return int(load_library().sdpa_backward_atomic_workspace_size(B, Hq, Sq, D))


def sdpa_backward_bias(q, k, v, out, dout, lse, bias, scale, mask_kind=MASK_NONE, key_lens=None,
                       dbias=None, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """(dq, dk, dv, dbias) of O = softmax(Q K^T * scale + bias + mask) V given dout.

    out and lse are sdpa_forward_bias's with the same bias.  dbias: None (not
    computed), True (allocated), or a [B, Hq, Sq, Sk] tensor in q's dtype; it
    is dS per (batch, query head) and is returned as the fourth value (None
    when not computed).
    """
    B, Hq, Hkv, Sq, Sk, D = _check_qkv(q, k, v, key_lens)
    sb, sh = _bias_strides(bias, q, B, Hq, Sq, Sk)
    for name, t in (("out", out), ("dout", dout)):
        _check_tensor(name, t, 4)
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("%s must match q in shape and dtype" % name)
    _check_tensor("lse", lse, 3)
    if tuple(lse.shape) != (B, Hq, Sq) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, Hq, Sq]")
    if dbias is True:
        dbias = torch.empty((B, Hq, Sq, Sk), dtype=q.dtype, device=q.device)
    elif dbias is not None:
        _check_tensor("dbias", dbias, 4)
        if tuple(dbias.shape) != (B, Hq, Sq, Sk) or dbias.dtype != q.dtype:
            raise ValueError("dbias must be [B, Hq, Sq, Sk] in q's dtype")
    outs = []
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t is None:
            t = torch.empty_like(like)
        else:
            _check_tensor(name, t, 4)
            if t.shape != like.shape or t.dtype != like.dtype:
                raise ValueError("%s must match its input in shape and dtype" % name)
        outs.append(t)
    dq, dk, dv = outs
    need = sdpa_backward_workspace_size(B, Hq, Sq)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    lib = load_library()
    _check(lib.sdpa_backward_bias(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                                  B, Hq, Hkv, Sq, Sk, D, float(scale), int(mask_kind),
                                  _ptr(key_lens), _ptr(bias), sb, sh, _ptr(dq), _ptr(dk), _ptr(dv),
                                  _ptr(dbias), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _dtype_code(q),
                                  _stream(stream)))
    return dq, dk, dv, dbias


def sdpa_backward(q, k, v, out, dout, lse, scale, mask_kind=MASK_NONE, key_lens=None,
                  dq=None, dk=None, dv=None, workspace=None, stream=None, atomic=False):
    """(dq, dk, dv) of O = softmax(Q K^T * scale + mask) V given dout = dL/dO.

    out and lse are the forward's (sdpa_forward_lse); dq is [B,Hq,Sq,D], dk and
    dv [B,Hkv,Sk,D], all in the input dtype.  atomic=True calls
    sdpa_backward_atomic (dQ summed with fp32 atomics) instead of the ordered
    sdpa_backward.
    """
    B, Hq, Hkv, Sq, Sk, D = _check_qkv(q, k, v, key_lens)
    for name, t in (("out", out), ("dout", dout)):
        _check_tensor(name, t, 4)
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("%s must match q in shape and dtype" % name)
    _check_tensor("lse", lse, 3)
    if tuple(lse.shape) != (B, Hq, Sq) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, Hq, Sq]")
    outs = []
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t is None:
            t = torch.empty_like(like)
        else:
            _check_tensor(name, t, 4)
            if t.shape != like.shape or t.dtype != like.dtype:
                raise ValueError("%s must match its input in shape and dtype" % name)
        outs.append(t)
    dq, dk, dv = outs
    need = (sdpa_backward_atomic_workspace_size(B, Hq, Sq, D) if atomic
            else sdpa_backward_workspace_size(B, Hq, Sq))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    lib = load_library()
    fn = lib.sdpa_backward_atomic if atomic else lib.sdpa_backward
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                             B, Hq, Hkv, Sq, Sk, D, float(scale), int(mask_kind), _ptr(key_lens),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _dtype_code(q),
                             _stream(stream)))
    return dq, dk, dv


def sdpa_block_workspace_size(B, S, model):
    return int(load_library().sdpa_block_workspace_size(B, S, model))


def sdpa_block_forward(x, wq, wk, wv, wo, heads, scale=None, mask_kind=MASK_NONE, key_lens=None,
                       y=None, workspace=None, stream=None):
    """The multi-head attention block: heads^-1(sdpa(heads(x.wq), heads(x.wk), heads(x.wv))).wo.

    x [B, S, model]; weights [model, model]; scale defaults to 1/sqrt(model/heads).
    """
    _check_tensor("x", x, 3)
    for name, w in (("wq", wq), ("wk", wk), ("wv", wv), ("wo", wo)):
        _check_tensor(name, w, 2)
        if tuple(w.shape) != (x.shape[2], x.shape[2]) or w.dtype != x.dtype:
            raise ValueError("%s must be [model, model] in x's dtype" % name)
    if key_lens is not None:
        _check_tensor("key_lens", key_lens, 1)
        if key_lens.dtype != torch.int32:
            raise TypeError("key_lens must be int32")
    B, S, M = x.shape
    if scale is None:
        scale = 1.0 / (M // heads) ** 0.5
    if y is None:
        y = torch.empty_like(x)
    else:
        _check_tensor("y", y, 3)
        if y.shape != x.shape or y.dtype != x.dtype:
            raise ValueError("y must match x in shape and dtype")
    need = sdpa_block_workspace_size(B, S, M)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    lib = load_library()
    _check(lib.sdpa_block_forward(_ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo), B, S, M, heads,
                                  float(scale), int(mask_kind), _ptr(key_lens), _ptr(y),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _dtype_code(x), _stream(stream)))
    return y


def sdpa_decode_workspace_size(B, Hq, D, num_splits):
    return int(load_library().sdpa_decode_workspace_size(B, Hq, D, num_splits))


def sdpa_decode(q, k, v, scale, key_lens=None, num_splits=MAX_SPLITS, workspace=None, out=None,
                stream=None):
    """Single-query decode: q [B,Hq,1,D], k/v [B,Hkv,Sk,D], split-KV + merge."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, 4)
    B, Hq, Sq, D = q.shape
    if Sq != 1:
        raise ValueError("decode takes one query per (batch, head): q must be [B, Hq, 1, D]")
    Hkv, Sk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Sk, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, Sk, D] matching q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    if key_lens is not None:
        _check_tensor("key_lens", key_lens, 1)
        if key_lens.dtype != torch.int32:
            raise TypeError("key_lens must be int32")
    lib = load_library()
    need = int(lib.sdpa_decode_workspace_size(B, Hq, D, int(num_splits)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    _check(lib.sdpa_decode(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, Sk, D, float(scale),
                           _ptr(key_lens), int(num_splits), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _ptr(out),
                           _dtype_code(q), _stream(stream)))
    return out


def sdpa_decode_noalloc(q, k, v, scale, out, key_lens=None, num_splits=MAX_SPLITS, stream=None):
    """sdpa_decode with its partials in the library's static device scratch:
    the call allocates no device memory (out is the caller's)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _check_tensor(name, t, 4)
    B, Hq, Sq, D = q.shape
    if Sq != 1:
        raise ValueError("decode takes one query per (batch, head): q must be [B, Hq, 1, D]")
    Hkv, Sk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Sk, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, Sk, D] matching q")
    if k.dtype != q.dtype or v.dtype != q.dtype or out.dtype != q.dtype:
        raise TypeError("q, k, v and out must share one dtype")
    if out.shape != q.shape:
        raise ValueError("out must be [B, Hq, 1, D]")
    if key_lens is not None:
        _check_tensor("key_lens", key_lens, 1)
        if key_lens.dtype != torch.int32:
            raise TypeError("key_lens must be int32")
    _check(load_library().sdpa_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, Sk, D,
                                              float(scale), _ptr(key_lens), int(num_splits),
                                              _ptr(out), _dtype_code(q), _stream(stream)))
    return out


def decode_workspace_views(workspace, B, Hq, D, num_splits):
    """(o_part [B,Hq,n,D], lse [B,Hq,n]) fp32 views of a decode workspace.

    Each partial row is D floats rounded up to a multiple of 4; the view
    drops the padding."""
    Dp = (D + 3) // 4 * 4
    n_o = B * Hq * num_splits * Dp
    off = (n_o * 4 + 255) // 256 * 256
    f = workspace.view(torch.uint8)
    o_part = f[: n_o * 4].view(torch.float32).view(B, Hq, num_splits, Dp)[..., :D]
    lse = f[off: off + B * Hq * num_splits * 4].view(torch.float32).view(B, Hq, num_splits)
    return o_part, lse


def sdpa_paged_attention(q, k_cache, v_cache, block_tables, seq_lens, query_seq, query_pos, scale,
                         causal, max_seq_len, num_splits=MAX_SPLITS, workspace=None, out=None,
                         stream=None):
    """Packed queries over a K/V page cache.

    q [queries, Hq, D]; k_cache [pages, page_size, Hkv, D]; v_cache [pages,
    page_size, Hkv, Dv]; block_tables int32 [num_seqs, max_pages_per_seq];
    seq_lens int32 [num_seqs]; query_seq, query_pos int32 [queries];
    max_seq_len (host int) bounds seq_lens.  Returns out [queries, Hq, Dv].
    """
    _check_tensor("q", q, 3)
    _check_tensor("k_cache", k_cache, 4)
    _check_tensor("v_cache", v_cache, 4)
    _check_tensor("block_tables", block_tables, 2)
    for name, t in (("seq_lens", seq_lens), ("query_seq", query_seq), ("query_pos", query_pos)):
        _check_tensor(name, t, 1)
    for name, t in (("block_tables", block_tables), ("seq_lens", seq_lens),
                    ("query_seq", query_seq), ("query_pos", query_pos)):
        if t.dtype != torch.int32:
            raise TypeError("%s must be int32" % name)
    nq, Hq, D = q.shape
    pages, page_size, Hkv, Dk = k_cache.shape
    Dv = v_cache.shape[3]
    if Dk != D or tuple(v_cache.shape[:3]) != (pages, page_size, Hkv):
        raise ValueError("k_cache must be [pages, page_size, Hkv, D] matching q and v_cache "
                         "[pages, page_size, Hkv, Dv]")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share one dtype")
    num_seqs, max_pages = block_tables.shape
    if seq_lens.shape[0] != num_seqs or query_seq.shape[0] != nq or query_pos.shape[0] != nq:
        raise ValueError("seq_lens must have num_seqs entries, query_seq and query_pos one per query")
    lib = load_library()
    need = int(lib.sdpa_decode_workspace_size(nq, Hq, Dv, int(num_splits)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((nq, Hq, Dv), dtype=q.dtype, device=q.device)
    _check(lib.sdpa_paged_attention(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), nq, Hq, Hkv, D, Dv, pages, page_size,
        _ptr(block_tables),
        num_seqs, max_pages, _ptr(seq_lens), _ptr(query_seq), _ptr(query_pos), int(max_seq_len),
        float(scale), int(bool(causal)), int(num_splits), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _dtype_code(q), _stream(stream)))
    return out


def sdpa_paged_prefill(q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q, scale, causal,
                       max_q, max_seq_len, out=None, stream=None, lse=False):
    """Packed prefill chunks over a K/V page cache.

    q [total_q, Hq, D]; k_cache [pages, page_size, Hkv, D]; v_cache [pages,
    page_size, Hkv, Dv]; block_tables int32 [num_seqs, max_pages_per_seq];
    seq_lens int32 [num_seqs] (the chunk included); cu_seqlens_q int32
    [num_seqs + 1]; max_q, max_seq_len host bounds.  Row i of sequence s's
    chunk sits at position seq_lens[s] - n_s + i.  Returns out [total_q, Hq, Dv],
    or (out, lse fp32 [total_q, Hq]) with lse=True (or an lse tensor to fill).
    """
    _check_tensor("q", q, 3)
    _check_tensor("k_cache", k_cache, 4)
    _check_tensor("v_cache", v_cache, 4)
    _check_tensor("block_tables", block_tables, 2)
    _check_tensor("seq_lens", seq_lens, 1)
    _check_tensor("cu_seqlens_q", cu_seqlens_q, 1)
    for name, t in (("block_tables", block_tables), ("seq_lens", seq_lens),
                    ("cu_seqlens_q", cu_seqlens_q)):
        if t.dtype != torch.int32:
            raise TypeError("%s must be int32" % name)
    nq, Hq, D = q.shape
    pages, page_size, Hkv, Dk = k_cache.shape
    Dv = v_cache.shape[3]
    if Dk != D or tuple(v_cache.shape[:3]) != (pages, page_size, Hkv):
        raise ValueError("k_cache must be [pages, page_size, Hkv, D] matching q and v_cache "
                         "[pages, page_size, Hkv, Dv]")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share one dtype")
    num_seqs, max_pages = block_tables.shape
    if seq_lens.shape[0] != num_seqs or cu_seqlens_q.shape[0] != num_seqs + 1:
        raise ValueError("seq_lens needs num_seqs entries and cu_seqlens_q num_seqs + 1")
    if out is None:
        out = torch.empty((nq, Hq, Dv), dtype=q.dtype, device=q.device)
    lse_t = None
    if isinstance(lse, torch.Tensor):
        _check_tensor("lse", lse, 2)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (nq, Hq):
            raise ValueError("lse must be float32 [total_q, Hq]")
        lse_t = lse
    elif lse:
        lse_t = torch.empty((nq, Hq), dtype=torch.float32, device=q.device)
    lib = load_library()
    _check(lib.sdpa_paged_prefill(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), nq, Hq, Hkv, D, Dv, pages, page_size,
        _ptr(block_tables),
        num_seqs, max_pages, _ptr(seq_lens), _ptr(cu_seqlens_q), int(max_q), int(max_seq_len),
        float(scale), int(bool(causal)), _ptr(out), _ptr(lse_t), _dtype_code(q), _stream(stream)))
    return out if lse_t is None else (out, lse_t)


def sdpa_paged_backward_workspace_size(num_seqs, Hq, Hkv, max_seq_len, D, Dv=None,
                                       dtype=SDPA_BF16):
    Dv = D if Dv is None else Dv
    return int(load_library().sdpa_paged_backward_workspace_size(num_seqs, Hq, Hkv, max_seq_len, D,
                                                                 Dv, dtype))


def sdpa_paged_backward(q, k_cache, v_cache, out, dout, lse, block_tables, seq_lens, cu_seqlens_q,
                        scale, causal, max_seq_len, dq=None, dk_cache=None, dv_cache=None,
                        workspace=None, stream=None):
    """Backward of sdpa_paged_prefill: (dq [total_q, Hq, D], dk_cache [pages,
    page_size, Hkv, D], dv_cache [pages, page_size, Hkv, Dv]) for dL/dout =
    dout [total_q, Hq, Dv], from the forward's out and lse (fp32 [total_q,
    Hq])."""
    for name, t, nd in (("q", q, 3), ("k_cache", k_cache, 4), ("v_cache", v_cache, 4),
                        ("out", out, 3), ("dout", dout, 3), ("lse", lse, 2),
                        ("block_tables", block_tables, 2), ("seq_lens", seq_lens, 1),
                        ("cu_seqlens_q", cu_seqlens_q, 1)):
        _check_tensor(name, t, nd)
    for name, t in (("block_tables", block_tables), ("seq_lens", seq_lens),
                    ("cu_seqlens_q", cu_seqlens_q)):
        if t.dtype != torch.int32:
            raise TypeError("%s must be int32" % name)
    nq, Hq, D = q.shape
    pages, page_size, Hkv, Dk = k_cache.shape
    Dv = v_cache.shape[3]
    if Dk != D or v_cache.shape[:3] != k_cache.shape[:3]:
        raise ValueError("k_cache must be [pages, page_size, Hkv, D] matching q and v_cache "
                         "[pages, page_size, Hkv, Dv]")
    if tuple(out.shape) != (nq, Hq, Dv) or tuple(dout.shape) != (nq, Hq, Dv):
        raise ValueError("out and dout must be [total_q, Hq, Dv]")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (nq, Hq):
        raise ValueError("lse must be float32 [total_q, Hq]")
    for t in (k_cache, v_cache, out, dout):
        if t.dtype != q.dtype:
            raise TypeError("q, the caches, out and dout must share one dtype")
    num_seqs, max_pages = block_tables.shape
    if seq_lens.shape[0] != num_seqs or cu_seqlens_q.shape[0] != num_seqs + 1:
        raise ValueError("seq_lens needs num_seqs entries and cu_seqlens_q num_seqs + 1")
    lib = load_library()
    need = int(lib.sdpa_paged_backward_workspace_size(num_seqs, Hq, Hkv, int(max_seq_len), D, Dv,
                                                      _dtype_code(q)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk_cache = torch.empty_like(k_cache) if dk_cache is None else dk_cache
    dv_cache = torch.empty_like(v_cache) if dv_cache is None else dv_cache
    _check(lib.sdpa_paged_backward(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(dout), _ptr(lse), nq, Hq, Hkv, D,
        Dv, pages, page_size, _ptr(block_tables), num_seqs, max_pages, _ptr(seq_lens),
        _ptr(cu_seqlens_q), int(max_seq_len), float(scale), int(bool(causal)), _ptr(dq),
        _ptr(dk_cache), _ptr(dv_cache), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _dtype_code(q), _stream(stream)))
    return dq, dk_cache, dv_cache
