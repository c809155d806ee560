"""ctypes binding of libattn.so (declared in include/attn.h).

Argument marshalling only: every step of the attention forward runs in the
HIP kernels behind the C ABI.  torch is used for device memory and streams.
There is no fallback: if libattn.so is missing or fails to load, importing
this module raises.
"""

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EHIP = 0, -1, -2, -3
EXP_MODES = {"hw": 0, "poly": 1, "mix": 2}

# entry points declared in include/attn.h
EXPORTS = ("attn_default_opts", "attn_fwd", "attn_fwd_ex", "attn_fwd_mxfp4", "attn_fwd_mxfp4_ex",
           "attn_quantize_mxfp4_rows", "attn_quantize_mxfp4_cols_t", "attn_fwd_mxfp8",
           "attn_fwd_mxfp8_ex", "attn_quantize_mxfp8_rows", "attn_quantize_mxfp8_cols_t",
           "attn_bwd", "attn_bwd_ex", "attn_bwd_noalloc", "attn_strerror", "attn_last_hip_error")


class AttnOpts(ctypes.Structure):
    _fields_ = [("tau", ctypes.c_float), ("exp_mode", ctypes.c_int),
                ("poly_frac", ctypes.c_float), ("stats", ctypes.c_void_p),
                ("window", ctypes.c_int), ("alibi_slopes", ctypes.c_void_p),
                ("softcap", ctypes.c_float), ("doc_offsets", ctypes.c_void_p),
                ("n_docs", ctypes.c_int)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run "
                          "`python -m exact_attention_forward_tiled_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, LL = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_longlong
    OP = ctypes.POINTER(AttnOpts)
    sig = {
        "attn_default_opts": (None, [OP]),
        "attn_fwd": (I, [P, P, P, P, P, I, I, I, I, I, I, F]),
        "attn_fwd_ex": (I, [P, P, P, P, P, I, I, I, I, I, I, F, OP, P]),
        "attn_fwd_mxfp4": (I, [P] * 8 + [I] * 6 + [F]),
        "attn_fwd_mxfp4_ex": (I, [P] * 8 + [I] * 6 + [F, OP, P]),
        "attn_quantize_mxfp4_rows": (I, [P, P, P, LL, I, P]),
        "attn_quantize_mxfp4_cols_t": (I, [P, P, P, I, I, I, P]),
        "attn_fwd_mxfp8": (I, [P] * 8 + [I] * 6 + [F]),
        "attn_fwd_mxfp8_ex": (I, [P] * 8 + [I] * 6 + [F, OP, P]),
        "attn_quantize_mxfp8_rows": (I, [P, P, P, LL, I, P]),
        "attn_quantize_mxfp8_cols_t": (I, [P, P, P, I, I, I, P]),
        "attn_bwd": (I, [P] * 10 + [I] * 6 + [F, P]),
        "attn_bwd_ex": (I, [P] * 10 + [I] * 6 + [F, OP, P]),
        "attn_bwd_noalloc": (I, [P] * 9 + [I] * 6 + [F, OP, P]),
        "attn_strerror": (ctypes.c_char_p, [I]),
        "attn_last_hip_error": (I, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class AttnError(RuntimeError):
    pass


def check(status):
    """Map a libattn status code to an exception."""
    if status == ATTN_OK:
        return
    msg = lib.attn_strerror(status).decode()
    if status == ATTN_EINVAL:
        raise ValueError(f"libattn: {msg}")
    if status == ATTN_EUNSUPPORTED:
        raise NotImplementedError(f"libattn: {msg}")
    if status == ATTN_EHIP:
        raise AttnError(f"libattn: {msg} (hipError_t {lib.attn_last_hip_error()})")
    raise AttnError(f"libattn: status {status}")


def make_opts(tau=8.0, exp_mode="hw", stats_ptr=None, poly_frac=None, window=0, alibi_ptr=None,
              softcap=0.0, doc_ptr=None, n_docs=0):
    o = AttnOpts()
    lib.attn_default_opts(ctypes.byref(o))
    o.tau = float(tau)
    o.exp_mode = EXP_MODES[exp_mode] if isinstance(exp_mode, str) else int(exp_mode)
    if poly_frac is not None:
        o.poly_frac = float(poly_frac)
    o.stats = stats_ptr
    o.window = int(window)
    o.alibi_slopes = alibi_ptr
    o.softcap = float(softcap)
    o.doc_offsets = doc_ptr
    o.n_docs = int(n_docs)
    return o


# ---- raw C-ABI calls (pointers are ints, streams are hipStream_t handles or None) ----

def attn_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale):
    return lib.attn_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale)


def attn_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, opts=None, stream=None):
    return lib.attn_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale,
                           ctypes.byref(opts) if opts is not None else None, stream)


def attn_fwd_mxfp4_ex(q4, qs, k4, ks, vt4, vts, o, lse, B, Hq, Hkv, N, d, causal, scale,
                      opts=None, stream=None):
    return lib.attn_fwd_mxfp4_ex(q4, qs, k4, ks, vt4, vts, o, lse, B, Hq, Hkv, N, d, causal,
                                 scale, ctypes.byref(opts) if opts is not None else None, stream)


def attn_fwd_mxfp4(q4, qs, k4, ks, vt4, vts, o, lse, B, Hq, Hkv, N, d, causal, scale):
    return lib.attn_fwd_mxfp4(q4, qs, k4, ks, vt4, vts, o, lse, B, Hq, Hkv, N, d, causal, scale)


def attn_fwd_mxfp8_ex(q8, qs, k8, ks, vt8, vts, o, lse, B, Hq, Hkv, N, d, causal, scale,
                      opts=None, stream=None):
    return lib.attn_fwd_mxfp8_ex(q8, qs, k8, ks, vt8, vts, o, lse, B, Hq, Hkv, N, d, causal,
                                 scale, ctypes.byref(opts) if opts is not None else None, stream)


def attn_fwd_mxfp8(q8, qs, k8, ks, vt8, vts, o, lse, B, Hq, Hkv, N, d, causal, scale):
    return lib.attn_fwd_mxfp8(q8, qs, k8, ks, vt8, vts, o, lse, B, Hq, Hkv, N, d, causal, scale)


def attn_quantize_mxfp8_rows(x, codes, scales, rows, cols, stream=None):
    return lib.attn_quantize_mxfp8_rows(x, codes, scales, rows, cols, stream)


def attn_quantize_mxfp8_cols_t(x, codes, scales, batch, rows, cols, stream=None):
    return lib.attn_quantize_mxfp8_cols_t(x, codes, scales, batch, rows, cols, stream)


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, Hq, Hkv, N, d, causal, scale,
             stream=None):
    return lib.attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, Hq, Hkv, N, d, causal,
                        scale, stream)


def attn_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, delta, B, Hq, Hkv, N, d, causal, scale,
                opts=None, stream=None):
    return lib.attn_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, delta, B, Hq, Hkv, N, d, causal,
                           scale, ctypes.byref(opts) if opts is not None else None, stream)


def attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale,
                     opts=None, stream=None):
    return lib.attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, causal,
                                scale, ctypes.byref(opts) if opts is not None else None, stream)


def attn_quantize_mxfp4_rows(x, codes, scales, rows, cols, stream=None):
    return lib.attn_quantize_mxfp4_rows(x, codes, scales, rows, cols, stream)


def attn_quantize_mxfp4_cols_t(x, codes, scales, batch, rows, cols, stream=None):
    return lib.attn_quantize_mxfp4_cols_t(x, codes, scales, batch, rows, cols, stream)


# ---- torch-level wrappers: shape checks, output allocation, current stream ----

def _torch():
    import torch
    return torch


def _stream(torch, device):
    return torch.cuda.current_stream(device).cuda_stream


STATS_COUNTERS = 4


def require(t, name, shape, dtype, device):
    """Raise ValueError unless t is a contiguous tensor of this exact shape and dtype on this
    device.  The C ABI sees only pointers, so a wrong buffer would mean out-of-bounds device
    accesses: every caller tensor is checked here, before any launch."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(t):
    """The kernels read and write device memory only."""
    if not t.is_cuda:
        raise ValueError("the operands must be CUDA tensors")


def _outputs(torch, out, shapes, names, device):
    """Caller-given output tensors (checked) or new fp32 ones."""
    if out is None:
        return tuple(torch.empty(sh, dtype=torch.float32, device=device) for sh in shapes)
    out = tuple(out)
    if len(out) != len(shapes):
        raise ValueError(f"out must hold {len(shapes)} tensors ({', '.join(names)})")
    for t, sh, nm in zip(out, shapes, names):
        require(t, nm, sh, torch.float32, device)
    return out


def _stats_ptr(torch, stats):
    """Device pointer of the optional statistics buffer (int64 [>= STATS_COUNTERS], CUDA)."""
    if stats is None:
        return None
    if stats.dtype != torch.int64 or not stats.is_cuda or not stats.is_contiguous() \
            or stats.numel() < STATS_COUNTERS:
        raise ValueError(f"stats must be a contiguous int64 CUDA tensor of {STATS_COUNTERS} counters")
    return stats.data_ptr()


def fwd(q, k, v, causal=False, scale=None, tau=8.0, exp_mode="hw", stats=None, out=None,
        poly_frac=None, window=0, alibi=None, softcap=0.0, docs=None):
    """bf16 attention forward on the GPU: returns (O fp32 [B,Hq,N,d], LSE fp32 [B,Hq,N]).
    exp_mode "hw", "poly" or "mix" (poly_frac of the exponentials on the cubic); window W:
    key j visible from query i only when i - W < j (and j < i + W without the causal mask);
    alibi: float32 CUDA tensor of Hq slopes a_h (score -= a_h |i - j|); softcap C > 0: score ->
    C tanh(score / C); docs: int32 CUDA tensor of document offsets 0 < ... < N (packed
    documents, keys visible only within the query's document)."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d] tensors")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    require(q, "q", (B, Hq, N, d), torch.bfloat16, q.device)
    require(k, "k", (B, Hkv, N, d), torch.bfloat16, q.device)
    require(v, "v", (B, Hkv, N, d), torch.bfloat16, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o, lse = _outputs(torch, out, ((B, Hq, N, d), (B, Hq, N)), ("o", "lse"), q.device)
    _on_gpu(q)
    alibi_ptr = None
    if alibi is not None:
        if (alibi.dtype != torch.float32 or not alibi.is_cuda or not alibi.is_contiguous()
                or alibi.numel() != Hq):
            raise ValueError("alibi must be a contiguous float32 CUDA tensor of Hq slopes")
        alibi_ptr = alibi.data_ptr()
    doc_ptr, n_docs = None, 0
    if docs is not None:
        if docs.dtype != torch.int32 or not docs.is_cuda or not docs.is_contiguous() \
                or docs.numel() < 2:
            raise ValueError("docs must be a contiguous int32 CUDA tensor of document offsets")
        doc_ptr, n_docs = docs.data_ptr(), docs.numel() - 1
    opts = make_opts(tau, exp_mode, _stats_ptr(torch, stats), poly_frac, window, alibi_ptr,
                     softcap, doc_ptr, n_docs)
    check(attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      B, Hq, Hkv, N, d, int(bool(causal)), float(scale), opts,
                      _stream(torch, q.device)))
    return o, lse


def quantize_mxfp4_rows(x):
    """fp32 [..., cols] -> (codes uint8 [..., cols/2], scales uint8 [..., cols/32])."""
    torch = _torch()
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous fp32 CUDA tensor")
    cols = x.shape[-1]
    rows = x.numel() // cols
    codes = torch.empty(x.shape[:-1] + (cols // 2,), dtype=torch.uint8, device=x.device)
    scales = torch.empty(x.shape[:-1] + (cols // 32,), dtype=torch.uint8, device=x.device)
    check(attn_quantize_mxfp4_rows(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), rows, cols,
                                   _stream(torch, x.device)))
    return codes, scales


def quantize_mxfp4_cols_t(x):
    """fp32 [..., rows, cols] -> transposed (codes [..., cols, rows/2], scales [..., cols, rows/32])."""
    torch = _torch()
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous fp32 CUDA tensor")
    rows, cols = x.shape[-2], x.shape[-1]
    batch = x.numel() // (rows * cols)
    lead = x.shape[:-2]
    codes = torch.empty(lead + (cols, rows // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty(lead + (cols, rows // 32), dtype=torch.uint8, device=x.device)
    check(attn_quantize_mxfp4_cols_t(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), batch,
                                     rows, cols, _stream(torch, x.device)))
    return codes, scales


def fwd_mxfp4(q4, qs, k4, ks, vt4, vts, causal=False, scale=None, tau=8.0, stats=None, out=None,
              window=0, docs=None):
    """MXFP4 Direct-P forward: returns (O fp32 [B,Hq,N,d], LSE fp32 [B,Hq,N]).  window, docs:
    sliding window and document offsets (int32 CUDA tensor), as for fwd."""
    torch = _torch()
    if q4.dim() != 4 or k4.dim() != 4:
        raise ValueError("MXFP4 codes must be [B, H, N, d/2] tensors")
    B, Hq, N, half_d = q4.shape
    d = 2 * half_d
    Hkv = k4.shape[1]
    u8, dev = torch.uint8, q4.device
    require(q4, "q4", (B, Hq, N, d // 2), u8, dev)
    require(qs, "qs", (B, Hq, N, d // 32), u8, dev)
    require(k4, "k4", (B, Hkv, N, d // 2), u8, dev)
    require(ks, "ks", (B, Hkv, N, d // 32), u8, dev)
    require(vt4, "vt4", (B, Hkv, d, N // 2), u8, dev)
    require(vts, "vts", (B, Hkv, d, N // 32), u8, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o, lse = _outputs(torch, out, ((B, Hq, N, d), (B, Hq, N)), ("o", "lse"), dev)
    _on_gpu(q4)
    doc_ptr, n_docs = None, 0
    if docs is not None:
        if docs.dtype != torch.int32 or not docs.is_cuda or not docs.is_contiguous() \
                or docs.numel() < 2:
            raise ValueError("docs must be a contiguous int32 CUDA tensor of document offsets")
        doc_ptr, n_docs = docs.data_ptr(), docs.numel() - 1
    opts = make_opts(tau, "hw", _stats_ptr(torch, stats), window=window, doc_ptr=doc_ptr,
                     n_docs=n_docs)
    check(attn_fwd_mxfp4_ex(q4.data_ptr(), qs.data_ptr(), k4.data_ptr(), ks.data_ptr(),
                            vt4.data_ptr(), vts.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            B, Hq, Hkv, N, d, int(bool(causal)), float(scale), opts,
                            _stream(torch, q4.device)))
    return o, lse


def quantize_mxfp8_rows(x):
    """fp32 [..., cols] -> (E4M3 codes uint8 [..., cols], E8M0 scales uint8 [..., cols/32])."""
    torch = _torch()
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous fp32 CUDA tensor")
    cols = x.shape[-1]
    rows = x.numel() // cols
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scales = torch.empty(x.shape[:-1] + (cols // 32,), dtype=torch.uint8, device=x.device)
    check(attn_quantize_mxfp8_rows(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), rows, cols,
                                   _stream(torch, x.device)))
    return codes, scales


def quantize_mxfp8_cols_t(x):
    """fp32 [..., rows, cols] -> transposed (codes [..., cols, rows], scales [..., cols, rows/32])."""
    torch = _torch()
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous fp32 CUDA tensor")
    rows, cols = x.shape[-2], x.shape[-1]
    batch = x.numel() // (rows * cols)
    lead = x.shape[:-2]
    codes = torch.empty(lead + (cols, rows), dtype=torch.uint8, device=x.device)
    scales = torch.empty(lead + (cols, rows // 32), dtype=torch.uint8, device=x.device)
    check(attn_quantize_mxfp8_cols_t(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), batch,
                                     rows, cols, _stream(torch, x.device)))
    return codes, scales


def fwd_mxfp8(q8, qs, k8, ks, vt8, vts, causal=False, scale=None, tau=8.0, stats=None, out=None,
              window=0, docs=None):
    """MXFP8 forward: returns (O fp32 [B,Hq,N,d], LSE fp32 [B,Hq,N]).  window, docs: sliding
    window and document offsets (int32 CUDA tensor), as for fwd."""
    torch = _torch()
    if q8.dim() != 4 or k8.dim() != 4:
        raise ValueError("MXFP8 codes must be [B, H, N, d] tensors")
    B, Hq, N, d = q8.shape
    Hkv = k8.shape[1]
    u8, dev = torch.uint8, q8.device
    require(q8, "q8", (B, Hq, N, d), u8, dev)
    require(qs, "qs", (B, Hq, N, d // 32), u8, dev)
    require(k8, "k8", (B, Hkv, N, d), u8, dev)
    require(ks, "ks", (B, Hkv, N, d // 32), u8, dev)
    require(vt8, "vt8", (B, Hkv, d, N), u8, dev)
    require(vts, "vts", (B, Hkv, d, N // 32), u8, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o, lse = _outputs(torch, out, ((B, Hq, N, d), (B, Hq, N)), ("o", "lse"), dev)
    _on_gpu(q8)
    doc_ptr, n_docs = None, 0
    if docs is not None:
        if docs.dtype != torch.int32 or not docs.is_cuda or not docs.is_contiguous() \
                or docs.numel() < 2:
            raise ValueError("docs must be a contiguous int32 CUDA tensor of document offsets")
        doc_ptr, n_docs = docs.data_ptr(), docs.numel() - 1
    opts = make_opts(tau, "hw", _stats_ptr(torch, stats), window=window, doc_ptr=doc_ptr,
                     n_docs=n_docs)
    check(attn_fwd_mxfp8_ex(q8.data_ptr(), qs.data_ptr(), k8.data_ptr(), ks.data_ptr(),
                            vt8.data_ptr(), vts.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            B, Hq, Hkv, N, d, int(bool(causal)), float(scale), opts,
                            _stream(torch, q8.device)))
    return o, lse


def bwd(q, k, v, o, lse, dout, causal=False, scale=None, out=None, delta=None, window=0,
        docs=None, alibi=None, softcap=0.0):
    """bf16 attention backward: returns (dQ fp32 [B,Hq,N,d], dK, dV fp32 [B,Hkv,N,d]).
    o, lse: the forward's outputs for the same q, k, v (fp32); dout: bf16 like q.
    delta: optional fp32 CUDA workspace of B*Hq*N floats.  window, docs, alibi, softcap:
    the forward's sliding window, document offsets, ALiBi slopes and soft-capping (as for
    fwd)."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d] tensors")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    bf, f32, dev = torch.bfloat16, torch.float32, q.device
    require(q, "q", (B, Hq, N, d), bf, dev)
    require(k, "k", (B, Hkv, N, d), bf, dev)
    require(v, "v", (B, Hkv, N, d), bf, dev)
    require(dout, "dout", (B, Hq, N, d), bf, dev)
    require(o, "o", (B, Hq, N, d), f32, dev)
    require(lse, "lse", (B, Hq, N), f32, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = _outputs(torch, out, ((B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d)),
                          ("dq", "dk", "dv"), dev)
    if delta is None:
        delta = torch.empty((B, Hq, N), dtype=f32, device=dev)
    elif (delta.dtype != f32 or delta.device != dev or not delta.is_contiguous()
          or delta.numel() < B * Hq * N):
        raise ValueError("delta must be a contiguous fp32 tensor of at least B*Hq*N floats "
                         "on the inputs' device")
    _on_gpu(q)
    doc_ptr, n_docs = None, 0
    if docs is not None:
        if docs.dtype != torch.int32 or not docs.is_cuda or not docs.is_contiguous() \
                or docs.numel() < 2:
            raise ValueError("docs must be a contiguous int32 CUDA tensor of document offsets")
        doc_ptr, n_docs = docs.data_ptr(), docs.numel() - 1
    alibi_ptr = None
    if alibi is not None:
        if (alibi.dtype != torch.float32 or not alibi.is_cuda or not alibi.is_contiguous()
                or alibi.numel() != Hq):
            raise ValueError("alibi must be a contiguous float32 CUDA tensor of Hq slopes")
        alibi_ptr = alibi.data_ptr()
    opts = make_opts(window=window, doc_ptr=doc_ptr, n_docs=n_docs, alibi_ptr=alibi_ptr,
                     softcap=softcap)
    check(attn_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                      delta.data_ptr(), B, Hq, Hkv, N, d, int(bool(causal)), float(scale), opts,
                      _stream(torch, q.device)))
    return dq, dk, dv
