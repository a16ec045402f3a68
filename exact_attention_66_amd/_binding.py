"""ctypes binding of libattn.so: the C ABI declared in include/attn.h.

Argument marshalling only: tensors become device pointers and sizes, the
stream becomes a hipStream_t handle, and nonzero status codes become
``AttnError``.  Every step of the computation runs in the HIP kernels; there
is no fallback of any kind when the library is missing or a call fails.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

import torch

# The in-tree build; ATTN_LIBRARY names another build of the same library
# (the host-sanitizer build of the argument checks uses it).
LIB_PATH = os.environ.get("ATTN_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

# attn_status / attn_dtype values of include/attn.h
ATTN_OK = 0
ATTN_DTYPE_BF16 = 0
ATTN_DTYPE_FP16 = 1
STATUS_NAMES = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL_PTR", 2: "ATTN_ERR_BAD_SHAPE", 3: "ATTN_ERR_UNSUPPORTED_HEAD_DIM",
    4: "ATTN_ERR_BAD_DTYPE", 5: "ATTN_ERR_MISALIGNED", 6: "ATTN_ERR_UNSUPPORTED_SEQLEN",
    7: "ATTN_ERR_BAD_SCALE", 8: "ATTN_ERR_WORKSPACE_TOO_SMALL", 9: "ATTN_ERR_ALIASING", 10: "ATTN_ERR_HIP",
    11: "ATTN_ERR_BAD_LAYOUT", 12: "ATTN_ERR_BAD_DROPOUT", 13: "ATTN_ERR_SCRATCH_TOO_SMALL",
}
# ATTN_KV_SCRATCH_BYTES of include/attn.h: the static buffer of attn_fwd_kvcache_noalloc
ATTN_KV_SCRATCH_BYTES = 32 << 20
EXPORTED = ["attn_fwd", "attn_fwd_strided", "attn_bwd_workspace_bytes", "attn_bwd", "attn_fwd_kvcache",
            "attn_fwd_kvcache_noalloc",
            "attn_fwd_kvcache_strided", "attn_fwd_kvcache_workspace_bytes", "attn_fwd_kvcache_splits",
            "attn_bwd_strided", "attn_bwd_strided_workspace_bytes", "attn_fwd_alibi", "attn_bwd_alibi",
            "attn_fwd_kvcache_alibi", "attn_fwd_kvcache_gqa", "attn_fwd_kvcache_gqa_workspace_bytes",
            "attn_dropout_threshold", "attn_fwd_dropout", "attn_bwd_dropout", "attn_dropout_draws",
            "attn_fwd_dropout_strided", "attn_bwd_dropout_strided",
            "attn_profile_start",
            "attn_profile_stop", "attn_status_string", "attn_last_hip_error"]
# attn_kernel_kind values
KERNEL_KINDS = ["fwd", "bwd_prep", "bwd_dkdv", "bwd_dq", "kv_split", "kv_merge"]

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {STATUS_NAMES.get(status, status)}: {attn_status_string(status)}"
        if status == 10:
            msg += f" (hipError_t {attn_last_hip_error()})"
        super().__init__(msg)


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libattn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} not found: build it with `python -m exact_attention_66_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    vp, i64, f32, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, i32, i32, vp]
    lib.attn_fwd.restype = i32
    lib.attn_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.attn_bwd_workspace_bytes.restype = sz
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, i32, i32, vp, sz, vp]
    lib.attn_bwd.restype = i32
    lib.attn_fwd_kvcache.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, i32, i32, i32, vp, sz, vp]
    lib.attn_fwd_kvcache.restype = i32
    lib.attn_fwd_kvcache_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, i32, i32, i32, vp]
    lib.attn_fwd_kvcache_noalloc.restype = i32
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.attn_fwd_strided.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64p, f32, i32, i32, vp]
    lib.attn_fwd_strided.restype = i32
    lib.attn_fwd_kvcache_strided.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64p, f32, i32, i32, i32,
                                             vp, sz, vp]
    lib.attn_fwd_kvcache_strided.restype = i32
    lib.attn_bwd_strided.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64p, f32, i32, i32, vp,
                                     sz, vp]
    lib.attn_bwd_strided.restype = i32
    lib.attn_fwd_alibi.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, f32, i32, i32, vp]
    lib.attn_fwd_alibi.restype = i32
    lib.attn_bwd_alibi.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, f32, i32, i32, vp,
                                   sz, vp]
    lib.attn_bwd_alibi.restype = i32
    lib.attn_fwd_kvcache_alibi.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, f32, i32, i32, i32, vp,
                                           sz, vp]
    lib.attn_fwd_kvcache_alibi.restype = i32
    lib.attn_fwd_kvcache_gqa.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp, f32, i32, i32, i32,
                                         vp, sz, vp]
    lib.attn_fwd_kvcache_gqa.restype = i32
    lib.attn_fwd_kvcache_gqa_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, i32]
    lib.attn_fwd_kvcache_gqa_workspace_bytes.restype = sz
    lib.attn_bwd_strided_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.attn_bwd_strided_workspace_bytes.restype = sz
    lib.attn_fwd_kvcache_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32]
    lib.attn_fwd_kvcache_workspace_bytes.restype = sz
    lib.attn_fwd_kvcache_splits.argtypes = [i64, i64, i64, i64, i64, i32]
    lib.attn_fwd_kvcache_splits.restype = i32
    u64, u32 = ctypes.c_uint64, ctypes.c_uint32
    lib.attn_dropout_threshold.argtypes = [f32]
    lib.attn_dropout_threshold.restype = i32
    lib.attn_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, i32, i32, f32, u64, u32, vp]
    lib.attn_fwd_dropout.restype = i32
    lib.attn_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, i32, i32, f32, u64,
                                     u32, vp, sz, vp]
    lib.attn_bwd_dropout.restype = i32
    lib.attn_dropout_draws.argtypes = [vp, i64, i64, i64, u64, u32, vp]
    lib.attn_fwd_dropout_strided.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64p, f32, i32, i32, f32, u64,
                                             u32, vp]
    lib.attn_fwd_dropout_strided.restype = i32
    lib.attn_bwd_dropout_strided.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64p, f32, i32,
                                             i32, f32, u64, u32, vp, sz, vp]
    lib.attn_bwd_dropout_strided.restype = i32
    lib.attn_dropout_draws.restype = i32
    lib.attn_profile_start.argtypes = []
    lib.attn_profile_start.restype = i32
    lib.attn_profile_stop.argtypes = [ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)]
    lib.attn_profile_stop.restype = i32
    lib.attn_status_string.argtypes = [i32]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_last_hip_error.argtypes = []
    lib.attn_last_hip_error.restype = i32
    _lib = lib
    return lib


def attn_status_string(status: int) -> str:
    return load().attn_status_string(int(status)).decode()


def attn_last_hip_error() -> int:
    return int(load().attn_last_hip_error())


def attn_profile_start() -> None:
    st = load().attn_profile_start()
    if st != ATTN_OK:
        raise AttnError(st, "attn_profile_start")


def attn_profile_stop() -> dict:
    """Close the profiling window: {kernel: (launches, total_ms)} per kernel kind."""
    n = len(KERNEL_KINDS)
    counts = (ctypes.c_int64 * n)()
    total = (ctypes.c_double * n)()
    st = load().attn_profile_stop(counts, total)
    if st != ATTN_OK:
        raise AttnError(st, "attn_profile_stop")
    return {k: (int(counts[i]), float(total[i])) for i, k in enumerate(KERNEL_KINDS)}


def attn_bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(load().attn_bwd_workspace_bytes(B, H, N, d))


def attn_bwd_strided_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(load().attn_bwd_strided_workspace_bytes(B, H, N, d))


def attn_fwd_kvcache_workspace_bytes(B: int, H: int, Nq: int, Nk: int, d: int, num_splits: int = 0) -> int:
    return int(load().attn_fwd_kvcache_workspace_bytes(B, H, Nq, Nk, d, int(num_splits)))


def attn_fwd_kvcache_splits(B: int, H: int, Nq: int, Nk: int, d: int, num_splits: int = 0) -> int:
    return int(load().attn_fwd_kvcache_splits(B, H, Nq, Nk, d, int(num_splits)))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_DTYPE_BF16
    if t.dtype == torch.float16:
        return ATTN_DTYPE_FP16
    return -1  # rejected by the library as ATTN_ERR_BAD_DTYPE


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if t.numel() and not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr() or None


def _strided_ptr(t: torch.Tensor) -> Optional[int]:
    """Device pointer of a tensor whose last dimension is contiguous (any other strides)."""
    if t.dim() and t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError("the last (head-dimension) axis must be contiguous")
    return t.data_ptr() or None


def _strides12(*ts) -> "ctypes.Array":
    """(batch, head, token) element strides of [B, H, N, d] tensors, as int64[3 * len(ts)]."""
    vals = []
    for t in ts:
        vals += [int(t.stride(0)), int(t.stride(1)), int(t.stride(2))]
    return (ctypes.c_int64 * len(vals))(*vals)


def _all_contiguous(*ts) -> bool:
    return all(t.is_contiguous() for t in ts)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream or None
    return int(stream) or None


def _shape4(q: torch.Tensor):
    if q.dim() != 4:
        raise ValueError(f"expected a [B, H, N, d] tensor, got shape {tuple(q.shape)}")
    return tuple(int(x) for x in q.shape)


def attn_fwd(q, k, v, o, lse, scale: float, causal: bool, stream=None) -> None:
    """Enqueue the forward pass: writes o [B,H,N,d] and lse [B,H,N] fp32."""
    B, H, N, d = _shape4(q)
    for t in (k, v, o):
        if tuple(t.shape) != (B, H, N, d) or t.dtype != q.dtype:
            raise ValueError("q, k, v and o must share shape and dtype")
    if tuple(lse.shape) != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be a float32 [B, H, N] tensor")
    if _all_contiguous(q, k, v, o):
        st = load().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                             int(bool(causal)), _dtype_code(q), _stream(stream))
    else:   # [B, H, N, d] views of other layouts (e.g. [B, N, H, d] transposed): strides passed through
        st = load().attn_fwd_strided(_strided_ptr(q), _strided_ptr(k), _strided_ptr(v), _strided_ptr(o),
                                     _ptr(lse), B, H, N, d, _strides12(q, k, v, o), float(scale),
                                     int(bool(causal)), _dtype_code(q), _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd")


def attn_bwd(q, k, v, o, dO, lse, dq, dk, dv, scale: float, causal: bool, workspace, stream=None) -> None:
    """Enqueue the backward pass: writes dq, dk, dv; overwrites workspace (a uint8 tensor)."""
    B, H, N, d = _shape4(q)
    for t in (k, v, o, dO, dq, dk, dv):
        if tuple(t.shape) != (B, H, N, d) or t.dtype != q.dtype:
            raise ValueError("q, k, v, o, dO, dq, dk and dv must share shape and dtype")
    if tuple(lse.shape) != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be a float32 [B, H, N] tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    if _all_contiguous(q, k, v, o, dO, dq, dk, dv):
        st = load().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                             B, H, N, d, float(scale), int(bool(causal)), _dtype_code(q), _ptr(workspace),
                             ws_bytes, _stream(stream))
    else:   # other layouts: strides passed through (workspace: attn_bwd_strided_workspace_bytes)
        ts = (q, k, v, o, dO, dq, dk, dv)
        st = load().attn_bwd_strided(*(_strided_ptr(t) for t in ts[:5]), _ptr(lse),
                                     *(_strided_ptr(t) for t in ts[5:]), B, H, N, d, _strides12(*ts),
                                     float(scale), int(bool(causal)), _dtype_code(q), _ptr(workspace), ws_bytes,
                                     _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd")


def attn_fwd_kvcache(q, k, v, o, lse, scale: float, causal: bool, workspace, num_splits: int = 0,
                     stream=None) -> None:
    """Enqueue the KV-cache forward: q, o [B,H,Nq,d], k, v [B,H,Nk,d], lse [B,H,Nq] fp32."""
    B, H, Nq, d = _shape4(q)
    Nk = int(k.shape[2]) if k.dim() == 4 else -1
    if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape) != (B, H, Nk, d) or tuple(o.shape) != (B, H, Nq, d):
        raise ValueError("q, o must be [B,H,Nq,d] and k, v [B,H,Nk,d]")
    if any(t.dtype != q.dtype for t in (k, v, o)):
        raise ValueError("q, k, v and o must share the dtype")
    if tuple(lse.shape) != (B, H, Nq) or lse.dtype != torch.float32:
        raise ValueError("lse must be a float32 [B, H, Nq] tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    if _all_contiguous(q, k, v, o):
        st = load().attn_fwd_kvcache(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d, float(scale),
                                     int(bool(causal)), _dtype_code(q), int(num_splits), _ptr(workspace), ws_bytes,
                                     _stream(stream))
    else:
        st = load().attn_fwd_kvcache_strided(_strided_ptr(q), _strided_ptr(k), _strided_ptr(v), _strided_ptr(o),
                                             _ptr(lse), B, H, Nq, Nk, d, _strides12(q, k, v, o), float(scale),
                                             int(bool(causal)), _dtype_code(q), int(num_splits), _ptr(workspace),
                                             ws_bytes, _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_kvcache")


def attn_fwd_kvcache_noalloc(q, k, v, o, lse, scale: float, causal: bool, num_splits: int = 0, stream=None) -> None:
    """Enqueue the KV-cache forward with the split partials in the library's static buffer (no workspace, no
    allocation): contiguous q, o [B,H,Nq,d], k, v [B,H,Nk,d], lse [B,H,Nq] fp32, all caller-allocated."""
    B, H, Nq, d = _shape4(q)
    Nk = int(k.shape[2]) if k.dim() == 4 else -1
    if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape) != (B, H, Nk, d) or tuple(o.shape) != (B, H, Nq, d):
        raise ValueError("q, o must be [B,H,Nq,d] and k, v [B,H,Nk,d]")
    if any(t.dtype != q.dtype for t in (k, v, o)):
        raise ValueError("q, k, v and o must share the dtype")
    if tuple(lse.shape) != (B, H, Nq) or lse.dtype != torch.float32:
        raise ValueError("lse must be a float32 [B, H, Nq] tensor")
    st = load().attn_fwd_kvcache_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d,
                                         float(scale), int(bool(causal)), _dtype_code(q), int(num_splits),
                                         _stream(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_kvcache_noalloc")


# ------------------------------------------------------------------ conveniences
# Each convenience call allocates its outputs and temporaries (workspace,
# slopes) on the stream its kernels are enqueued on: torch's caching
# allocator ties a block to the stream it was allocated on, so a temporary
# freed when the call returns is only handed out again to work ordered after
# the kernels on that stream.  (Allocated on the current stream while the
# kernels ran on another, it could be reused and overwritten by work on the
# current stream while those kernels still read it.)
def _on_stream(stream, device):
    """Context in which allocations and the kernel launch share the kernels' stream."""
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream), device=device)
    return torch.cuda.stream(stream)


def default_scale(d: int) -> float:
    """fp32(1/sqrt(d)), the default softmax scale."""
    return float(torch.tensor(d, dtype=torch.float32).rsqrt().item())


def forward(q, k, v, scale: Optional[float] = None, causal: bool = False, stream=None):
    """Allocate (o, lse) with torch on q's device and run attn_fwd."""
    with _on_stream(stream, q.device):
        B, H, N, d = _shape4(q)
        scale = default_scale(d) if scale is None else scale
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        attn_fwd(q, k, v, o, lse, scale, causal, stream)
        return o, lse


def backward(q, k, v, o, lse, dO, scale: Optional[float] = None, causal: bool = False, workspace=None,
             stream=None):
    """Allocate (dq, dk, dv) and, if not given, the workspace; run attn_bwd."""
    with _on_stream(stream, q.device):
        B, H, N, d = _shape4(q)
        scale = default_scale(d) if scale is None else scale
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        if workspace is None:
            nbytes = (attn_bwd_workspace_bytes(B, H, N, d) if _all_contiguous(q, k, v, o, dO, dq, dk, dv)
                      else attn_bwd_strided_workspace_bytes(B, H, N, d))
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        attn_bwd(q, k, v, o, dO, lse, dq, dk, dv, scale, causal, workspace, stream)
        return dq, dk, dv


def forward_kvcache(q, k, v, scale: Optional[float] = None, causal: bool = False, num_splits: int = 0,
                    workspace=None, stream=None):
    """Allocate (o, lse) and, if not given, the workspace; run attn_fwd_kvcache."""
    with _on_stream(stream, q.device):
        B, H, Nq, d = _shape4(q)
        Nk = int(k.shape[2])
        scale = default_scale(d) if scale is None else scale
        if workspace is None:
            workspace = torch.empty(attn_fwd_kvcache_workspace_bytes(B, H, Nq, Nk, d, num_splits), dtype=torch.uint8,
                                    device=q.device)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
        attn_fwd_kvcache(q, k, v, o, lse, scale, causal, workspace, num_splits, stream)
        return o, lse


def _check_same(q, others, names: str):
    """The convenience calls: every tensor of ``others`` has q's [B, H, N, d] shape and dtype."""
    shape = _shape4(q)
    for t in others:
        if tuple(t.shape) != shape or t.dtype != q.dtype:
            raise ValueError(f"{names} must share shape and dtype")
    return shape


def _check_lse(lse, B: int, H: int, N: int):
    if tuple(lse.shape) != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be a float32 [B, H, N] tensor")


def _check_kv(q, k, v):
    """KV-cache calls: q [B, H, Nq, d]; k, v [B, Hkv, Nk, d] with q's dtype; returns Hkv, Nk."""
    B, H, Nq, d = _shape4(q)
    if k.dim() != 4:
        raise ValueError("k must be a [B, Hkv, Nk, d] tensor")
    Hkv, Nk = int(k.shape[1]), int(k.shape[2])
    if tuple(k.shape) != (B, Hkv, Nk, d) or tuple(v.shape) != (B, Hkv, Nk, d):
        raise ValueError("k and v must be [B, Hkv, Nk, d] with the batch and head size of q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share the dtype")
    return Hkv, Nk


def _slopes(alibi_slopes, H: int, device):
    """The [H] fp32 slopes as a contiguous device tensor."""
    t = torch.as_tensor(alibi_slopes, dtype=torch.float32, device=device).contiguous()
    if tuple(t.shape) != (H,):
        raise ValueError(f"alibi_slopes must have shape [H] = [{H}]")
    return t


def forward_alibi(q, k, v, alibi_slopes, scale: Optional[float] = None, causal: bool = False, stream=None):
    """attn_fwd_alibi on contiguous [B, H, N, d] tensors: (o, lse)."""
    with _on_stream(stream, q.device):
        B, H, N, d = _check_same(q, (k, v), "q, k and v")
        scale = default_scale(d) if scale is None else scale
        sl = _slopes(alibi_slopes, H, q.device)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        st = load().attn_fwd_alibi(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, _ptr(sl), float(scale),
                                   int(bool(causal)), _dtype_code(q), _stream(stream))
        if st != ATTN_OK:
            raise AttnError(st, "attn_fwd_alibi")
        return o, lse


def backward_alibi(q, k, v, o, lse, dO, alibi_slopes, scale: Optional[float] = None, causal: bool = False,
                   stream=None):
    """attn_bwd_alibi on contiguous tensors: (dq, dk, dv)."""
    with _on_stream(stream, q.device):
        B, H, N, d = _check_same(q, (k, v, o, dO), "q, k, v, o and dO")
        _check_lse(lse, B, H, N)
        scale = default_scale(d) if scale is None else scale
        sl = _slopes(alibi_slopes, H, q.device)
        ws = torch.empty(attn_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        st = load().attn_bwd_alibi(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                   B, H, N, d, _ptr(sl), float(scale), int(bool(causal)), _dtype_code(q), _ptr(ws),
                                   ws.numel(), _stream(stream))
        if st != ATTN_OK:
            raise AttnError(st, "attn_bwd_alibi")
        return dq, dk, dv


def dropout_threshold(dropout_p: float) -> int:
    """attn_dropout_threshold: the 8-bit drop threshold t (effective probability t / 256); ValueError if invalid."""
    t = load().attn_dropout_threshold(float(dropout_p))
    if t < 0:
        raise ValueError("dropout_p must be 0 or lie in [1/512, 511/512) (steps of 1/256)")
    return t


def forward_dropout(q, k, v, dropout_p: float, seed: int, offset: int = 0, scale: Optional[float] = None,
                    causal: bool = False, stream=None):
    """attn_fwd_dropout on [B, H, N, d] tensors (other layouts, e.g. transposed [B, N, H, d] views, through
    attn_fwd_dropout_strided; o takes q's layout): (o, lse)."""
    with _on_stream(stream, q.device):
        B, H, N, d = _check_same(q, (k, v), "q, k and v")
        scale = default_scale(d) if scale is None else scale
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        if _all_contiguous(q, k, v, o):
            st = load().attn_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                                         int(bool(causal)), _dtype_code(q), float(dropout_p), int(seed), int(offset),
                                         _stream(stream))
        else:
            st = load().attn_fwd_dropout_strided(_strided_ptr(q), _strided_ptr(k), _strided_ptr(v), _strided_ptr(o),
                                                 _ptr(lse), B, H, N, d, _strides12(q, k, v, o), float(scale),
                                                 int(bool(causal)), _dtype_code(q), float(dropout_p), int(seed),
                                                 int(offset), _stream(stream))
        if st != ATTN_OK:
            raise AttnError(st, "attn_fwd_dropout")
        return o, lse


def backward_dropout(q, k, v, o, lse, dO, dropout_p: float, seed: int, offset: int = 0,
                     scale: Optional[float] = None, causal: bool = False, stream=None):
    """attn_bwd_dropout (same dropout arguments as the forward; other layouts through
    attn_bwd_dropout_strided, gradients in the layouts of q, k, v): (dq, dk, dv)."""
    with _on_stream(stream, q.device):
        B, H, N, d = _check_same(q, (k, v, o, dO), "q, k, v, o and dO")
        _check_lse(lse, B, H, N)
        scale = default_scale(d) if scale is None else scale
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ts = (q, k, v, o, dO, dq, dk, dv)
        if _all_contiguous(*ts):
            ws = torch.empty(attn_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)
            st = load().attn_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse), _ptr(dq), _ptr(dk),
                                         _ptr(dv), B, H, N, d, float(scale), int(bool(causal)), _dtype_code(q),
                                         float(dropout_p), int(seed), int(offset), _ptr(ws), ws.numel(),
                                         _stream(stream))
        else:
            ws = torch.empty(attn_bwd_strided_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)
            st = load().attn_bwd_dropout_strided(*(_strided_ptr(t) for t in ts[:5]), _ptr(lse),
                                                 *(_strided_ptr(t) for t in ts[5:]), B, H, N, d, _strides12(*ts),
                                                 float(scale), int(bool(causal)), _dtype_code(q), float(dropout_p),
                                                 int(seed), int(offset), _ptr(ws), ws.numel(), _stream(stream))
        if st != ATTN_OK:
            raise AttnError(st, "attn_bwd_dropout")
        return dq, dk, dv


def dropout_draws(BH: int, Nq: int, Nk: int, seed: int, offset: int = 0, device="cuda", stream=None):
    """attn_dropout_draws: the [BH, Nq, Nk] uint8 draws (dropped where draw < dropout_threshold(p))."""
    with _on_stream(stream, device):
        out = torch.empty((BH, Nq, Nk), dtype=torch.uint8, device=device)
        st = load().attn_dropout_draws(_ptr(out), int(BH), int(Nq), int(Nk), int(seed), int(offset), _stream(stream))
        if st != ATTN_OK:
            raise AttnError(st, "attn_dropout_draws")
        return out


def forward_kvcache_alibi(q, k, v, alibi_slopes, scale: Optional[float] = None, causal: bool = False,
                          num_splits: int = 0, stream=None):
    """attn_fwd_kvcache_alibi on contiguous tensors: (o, lse)."""
    with _on_stream(stream, q.device):
        B, H, Nq, d = _shape4(q)
        Hkv, Nk = _check_kv(q, k, v)
        if Hkv != H:
            raise ValueError("k and v must have q's head count (grouped heads: forward_kvcache_gqa)")
        scale = default_scale(d) if scale is None else scale
        sl = _slopes(alibi_slopes, H, q.device)
        ws = torch.empty(attn_fwd_kvcache_workspace_bytes(B, H, Nq, Nk, d, num_splits), dtype=torch.uint8,
                         device=q.device)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
        st = load().attn_fwd_kvcache_alibi(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d, _ptr(sl),
                                           float(scale), int(bool(causal)), _dtype_code(q), int(num_splits), _ptr(ws),
                                           ws.numel(), _stream(stream))
        if st != ATTN_OK:
            raise AttnError(st, "attn_fwd_kvcache_alibi")
        return o, lse


def attn_fwd_kvcache_gqa_workspace_bytes(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int,
                                         num_splits: int = 0) -> int:
    return int(load().attn_fwd_kvcache_gqa_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, int(num_splits)))


def forward_kvcache_gqa(q, k, v, scale: Optional[float] = None, causal: bool = False, num_splits: int = 0,
                        alibi_slopes=None, workspace=None, stream=None):
    """attn_fwd_kvcache_gqa on contiguous q [B,Hq,Nq,d] and k, v [B,Hkv,Nk,d]: (o, lse)."""
    with _on_stream(stream, q.device):
        B, Hq, Nq, d = _shape4(q)
        Hkv, Nk = _check_kv(q, k, v)
        scale = default_scale(d) if scale is None else scale
        sl = None if alibi_slopes is None else _slopes(alibi_slopes, Hq, q.device)
        if workspace is None:
            workspace = torch.empty(attn_fwd_kvcache_gqa_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, num_splits),
                                    dtype=torch.uint8, device=q.device)
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
        st = load().attn_fwd_kvcache_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                                         None if sl is None else _ptr(sl), float(scale), int(bool(causal)),
                                         _dtype_code(q), int(num_splits), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(stream))
        if st != ATTN_OK:
            raise AttnError(st, "attn_fwd_kvcache_gqa")
        return o, lse
