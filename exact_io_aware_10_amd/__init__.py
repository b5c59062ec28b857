"""Python binding of libfa_mi355x.so, the gfx950 exact-attention library (include/fa.h).

Argument marshalling only: every step of the computation runs in the library's HIP
kernels. PyTorch supplies device memory (outputs are allocated with torch.empty) and the
current HIP stream. There is no fallback: if the library is missing the calls raise.

    o, lse = fa_fwd(q, k, v, causal=False, softmax_scale=None)
    dq, dk, dv = fa_bwd(q, k, v, o, lse, dout, causal=False, softmax_scale=None)
    o, lse = fa_fwd_varlen(q, k, v, cu_seqlens, max_seqlen, causal=False, softmax_scale=None)
    o, lse = fa_fwd_splitkv(q, k, v, causal=False, softmax_scale=None, num_splits=0)
    o, lse = fa_fwd_fp8(q, k, v, q_descale, k_descale, v_descale, causal=False,
                        softmax_scale=None)
    fa_merge(o_acc, lse_acc, o_part, lse_part, out=None)

q, k, v, o, dout: [B, N, H, d] (packed: [T, H, d]) contiguous bf16 or fp16 CUDA tensors;
lse: fp32 [B, H, N] (packed: [H, T]); d in {64, 128}; softmax_scale defaults to 1/sqrt(d).
fa_fwd_fp8 takes e4m3 tensors (torch.float8_e4m3fn, or uint8 holding the codes) with one
float descale per tensor and returns a bf16 output.
"""
import contextlib
import ctypes
import math
import os

__all__ = ["fa_fwd", "fa_bwd", "fa_bwd_prep", "fa_bwd_dkdv", "fa_bwd_dq", "fa_fwd_varlen",
           "fa_bwd_varlen", "fa_fwd_splitkv", "fa_fwd_splitkv_workspace_size", "fa_fwd_fp8",
           "fa_merge", "fa_fwd_splitkv_noalloc", "fa_noalloc_scratch_bytes",
           "fa_bwd_workspace_size", "fa_status_string", "FAError", "library_path",
           "load_library"]

_HERE = os.path.dirname(os.path.abspath(__file__))
# FA_LIBRARY selects another build of the same library (the debug variants of build.py)
library_path = os.environ.get("FA_LIBRARY") or os.path.join(_HERE, "libfa_mi355x.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3
FA_F16, FA_BF16 = 0, 1

_lib = None


class FAError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {fa_status_string(code)} (status {code})")
        self.code = code


def load_library():
    """Load the built library (ctypes). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise ImportError(
            f"{library_path} is missing; build it with `python -m exact_io_aware_10_amd.build`")
    lib = ctypes.CDLL(library_path)
    vp, i, f, s = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_bwd_workspace_size.argtypes = [i, i, i, i]
    lib.fa_bwd_workspace_size.restype = s
    for name in ("fa_bwd", "fa_bwd_prep", "fa_bwd_dkdv", "fa_bwd_dq"):
        getattr(lib, name).argtypes = [vp] * 10 + [i, i, i, i, i, f, i, vp]
        getattr(lib, name).restype = i
    lib.fa_fwd_varlen.argtypes = [vp] * 6 + [i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_varlen.restype = i
    lib.fa_bwd_varlen.argtypes = [vp] * 11 + [i, i, i, i, i, i, f, i, vp]
    lib.fa_bwd_varlen.restype = i
    lib.fa_fwd_splitkv_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.fa_fwd_splitkv_workspace_size.restype = s
    lib.fa_fwd_splitkv.argtypes = [vp] * 6 + [i, i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd_splitkv.restype = i
    lib.fa_noalloc_scratch_bytes.argtypes = []
    lib.fa_noalloc_scratch_bytes.restype = s
    lib.fa_fwd_splitkv_noalloc.argtypes = [vp] * 5 + [i, i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd_splitkv_noalloc.restype = i
    lib.fa_fwd_fp8.argtypes = [vp] * 5 + [i, i, i, i, f, f, f, f, i, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_merge.argtypes = [vp] * 5 + [i, i, i, i, i, vp]
    lib.fa_merge.restype = i
    _lib = lib
    return lib


def fa_status_string(code: int) -> str:
    return load_library().fa_status_string(int(code)).decode()


def fa_bwd_workspace_size(B: int, N: int, H: int, d: int) -> int:
    return int(load_library().fa_bwd_workspace_size(B, N, H, d))


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float16:
        return FA_F16
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float16")


def _check_tensor(name, t, shape, dtype, device):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device):
    return ctypes.c_void_p(_torch().cuda.current_stream(device).cuda_stream)


def _on(device):
    """Context in which the library's kernels go to `device` (the library launches on the
    current HIP device): a no-op when that is already the current one."""
    torch = _torch()
    if device.index is None or device.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(device)


def _scale(softmax_scale, d):
    return 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)


def fa_fwd(q, k, v, causal=False, softmax_scale=None, out=None, lse=None):
    """Forward attention. Returns (o [B,N,H,d], lse fp32 [B,H,N])."""
    torch = _torch()
    lib = load_library()
    if q.dim() != 4:
        raise ValueError("q must be [B, N, H, d]")
    B, N, H, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, q.shape, q.dtype, q.device)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensor("out", o, q.shape, q.dtype, q.device)
    _check_tensor("lse", lse, (B, H, N), torch.float32, q.device)
    with _on(q.device):
        rc = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        B, N, H, d, _dtype_code(q), _scale(softmax_scale, d), int(bool(causal)),
                        _stream(q.device))
    if rc != FA_OK:
        raise FAError("fa_fwd", rc)
    return o, lse


def fa_fwd_fp8(q, k, v, q_descale=1.0, k_descale=1.0, v_descale=1.0, causal=False,
               softmax_scale=None, out=None, lse=None):
    """FP8 forward: q, k, v hold e4m3 codes ([B, N, H, d], torch.float8_e4m3fn or uint8),
    each tensor's value being its descale times the codes' values. Returns (o bf16
    [B,N,H,d], lse fp32 [B,H,N])."""
    torch = _torch()
    lib = load_library()
    if q.dim() != 4:
        raise ValueError("q must be [B, N, H, d]")
    if q.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise TypeError(f"unsupported dtype {q.dtype}; expected float8_e4m3fn or uint8")
    B, N, H, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, q.shape, q.dtype, q.device)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensor("out", o, q.shape, torch.bfloat16, q.device)
    _check_tensor("lse", lse, (B, H, N), torch.float32, q.device)
    with _on(q.device):
        rc = lib.fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            B, N, H, d, float(q_descale), float(k_descale), float(v_descale),
                            _scale(softmax_scale, d), int(bool(causal)), _stream(q.device))
    if rc != FA_OK:
        raise FAError("fa_fwd_fp8", rc)
    return o, lse


def fa_merge(o_acc, lse_acc, o_part, lse_part, out=None):
    """Merge (o_part, lse_part) into the running (o_acc fp32 [B,N,H,d], lse_acc fp32
    [B,H,N]) in place; o_part is bf16/fp16. If out is given (same dtype as o_part) it also
    receives the merged output rounded to that dtype. Returns out (or None)."""
    torch = _torch()
    lib = load_library()
    if o_part.dim() != 4:
        raise ValueError("o_part must be [B, N, H, d]")
    B, N, H, d = o_part.shape
    _check_tensor("o_part", o_part, o_part.shape, o_part.dtype, o_part.device)
    _check_tensor("o_acc", o_acc, o_part.shape, torch.float32, o_part.device)
    _check_tensor("lse_acc", lse_acc, (B, H, N), torch.float32, o_part.device)
    _check_tensor("lse_part", lse_part, (B, H, N), torch.float32, o_part.device)
    if out is not None:
        _check_tensor("out", out, o_part.shape, o_part.dtype, o_part.device)
    with _on(o_part.device):
        rc = lib.fa_merge(o_acc.data_ptr(), lse_acc.data_ptr(), o_part.data_ptr(),
                          lse_part.data_ptr(), None if out is None else out.data_ptr(), B, N, H, d,
                          _dtype_code(o_part), _stream(o_part.device))
    if rc != FA_OK:
        raise FAError("fa_merge", rc)
    return out


def _bwd_call(fn, q, k, v, o, lse, dout, causal, softmax_scale, workspace, grads):
    torch = _torch()
    lib = load_library()
    B, N, H, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_tensor(name, t, q.shape, q.dtype, q.device)
    _check_tensor("lse", lse, (B, H, N), torch.float32, q.device)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q))
    for name, t in zip(("dq", "dk", "dv"), grads):
        _check_tensor(name, t, q.shape, q.dtype, q.device)
    nbytes = fa_bwd_workspace_size(B, N, H, d)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    dq, dk, dv = grads
    with _on(q.device):
        rc = getattr(lib, fn)(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                              dv.data_ptr(), workspace.data_ptr(), B, N, H, d, _dtype_code(q),
                              _scale(softmax_scale, d), int(bool(causal)), _stream(q.device))
    if rc != FA_OK:
        raise FAError(fn, rc)
    return grads


def fa_bwd(q, k, v, o, lse, dout, causal=False, softmax_scale=None, workspace=None,
           grads=None):
    """Backward attention from the forward's o and lse. Returns (dq, dk, dv).
    grads: optional preallocated (dq, dk, dv)."""
    return _bwd_call("fa_bwd", q, k, v, o, lse, dout, causal, softmax_scale, workspace, grads)


def fa_bwd_prep(q, k, v, o, lse, dout, causal=False, softmax_scale=None, workspace=None,
                grads=None):
    """Stage 1 of fa_bwd: row terms into `workspace` (pass the same workspace to the next
    stages)."""
    return _bwd_call("fa_bwd_prep", q, k, v, o, lse, dout, causal, softmax_scale, workspace,
                     grads)


def fa_bwd_dkdv(q, k, v, o, lse, dout, causal=False, softmax_scale=None, workspace=None,
                grads=None):
    """Stage 2 of fa_bwd: dk and dv (into grads[1], grads[2])."""
    return _bwd_call("fa_bwd_dkdv", q, k, v, o, lse, dout, causal, softmax_scale, workspace,
                     grads)


def fa_bwd_dq(q, k, v, o, lse, dout, causal=False, softmax_scale=None, workspace=None,
              grads=None):
    """Stage 3 of fa_bwd: dq (into grads[0])."""
    return _bwd_call("fa_bwd_dq", q, k, v, o, lse, dout, causal, softmax_scale, workspace,
                     grads)


def fa_fwd_varlen(q, k, v, cu_seqlens, max_seqlen, causal=False, softmax_scale=None):
    """Packed-sequence forward. q, k, v: [T, H, d]; cu_seqlens: int32 CUDA [nseq + 1].
    Returns (o [T,H,d], lse fp32 [H,T])."""
    torch = _torch()
    lib = load_library()
    if q.dim() != 3:
        raise ValueError("q must be [T, H, d]")
    T, H, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, q.shape, q.dtype, q.device)
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a 1-D int32 GPU tensor")
    o = torch.empty_like(q)
    lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    with _on(q.device):
        rc = lib.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                               lse.data_ptr(), cu_seqlens.data_ptr(), cu_seqlens.numel() - 1, T,
                               int(max_seqlen), H, d, _dtype_code(q), _scale(softmax_scale, d),
                               int(bool(causal)), _stream(q.device))
    if rc != FA_OK:
        raise FAError("fa_fwd_varlen", rc)
    return o, lse


def fa_bwd_varlen(q, k, v, o, lse, dout, cu_seqlens, max_seqlen, causal=False,
                  softmax_scale=None, workspace=None):
    """Packed-sequence backward from fa_fwd_varlen's o and lse. Returns (dq, dk, dv);
    rows of tokens outside every sequence are left as allocated (torch.zeros)."""
    torch = _torch()
    lib = load_library()
    T, H, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_tensor(name, t, q.shape, q.dtype, q.device)
    _check_tensor("lse", lse, (H, T), torch.float32, q.device)
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a 1-D int32 GPU tensor")
    dq, dk, dv = torch.zeros_like(q), torch.zeros_like(q), torch.zeros_like(q)
    nbytes = fa_bwd_workspace_size(1, T, H, d)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    with _on(q.device):
        rc = lib.fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                               lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                               dv.data_ptr(), workspace.data_ptr(), cu_seqlens.data_ptr(),
                               cu_seqlens.numel() - 1, T, int(max_seqlen), H, d, _dtype_code(q),
                               _scale(softmax_scale, d), int(bool(causal)), _stream(q.device))
    if rc != FA_OK:
        raise FAError("fa_bwd_varlen", rc)
    return dq, dk, dv


def fa_fwd_splitkv_workspace_size(B: int, Nq: int, Nk: int, H: int, d: int,
                                  num_splits: int = 0) -> int:
    return int(load_library().fa_fwd_splitkv_workspace_size(B, Nq, Nk, H, d, num_splits))


def fa_fwd_splitkv(q, k, v, causal=False, softmax_scale=None, num_splits=0, workspace=None):
    """Split-KV forward for decode shapes. q: [B, Nq, H, d]; k, v: [B, Nk, H, d] (same
    dtype, contiguous). Query row i stands at position Nk - Nq + i (causal: it sees keys up
    to that position). Returns (o [B,Nq,H,d], lse fp32 [B,H,Nq])."""
    torch = _torch()
    lib = load_library()
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, Nq, H, d] and k, v [B, Nk, H, d]")
    B, Nq, H, d = q.shape
    Nk = k.shape[1]
    _check_tensor("q", q, q.shape, q.dtype, q.device)
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, (B, Nk, H, d), q.dtype, q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    nbytes = fa_fwd_splitkv_workspace_size(B, Nq, Nk, H, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    with _on(q.device):
        rc = lib.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), workspace.data_ptr(), B, Nq, Nk, H, d,
                                _dtype_code(q), _scale(softmax_scale, d), int(bool(causal)),
                                int(num_splits), _stream(q.device))
    if rc != FA_OK:
        raise FAError("fa_fwd_splitkv", rc)
    return o, lse


def fa_noalloc_scratch_bytes() -> int:
    return int(load_library().fa_noalloc_scratch_bytes())


def fa_fwd_splitkv_noalloc(q, k, v, causal=False, softmax_scale=None, num_splits=0, out=None,
                           lse=None):
    """fa_fwd_splitkv with its workspace in the library's scratch array (the library
    allocates nothing; see include/fa.h). Outputs are allocated here unless passed in.
    Returns (o [B,Nq,H,d], lse fp32 [B,H,Nq])."""
    torch = _torch()
    lib = load_library()
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, Nq, H, d] and k, v [B, Nk, H, d]")
    B, Nq, H, d = q.shape
    Nk = k.shape[1]
    _check_tensor("q", q, q.shape, q.dtype, q.device)
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, (B, Nk, H, d), q.dtype, q.device)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensor("out", o, q.shape, q.dtype, q.device)
    _check_tensor("lse", lse, (B, H, Nq), torch.float32, q.device)
    with _on(q.device):
        rc = lib.fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                        lse.data_ptr(), B, Nq, Nk, H, d, _dtype_code(q),
                                        _scale(softmax_scale, d), int(bool(causal)),
                                        int(num_splits), _stream(q.device))
    if rc != FA_OK:
        raise FAError("fa_fwd_splitkv_noalloc", rc)
    return o, lse
