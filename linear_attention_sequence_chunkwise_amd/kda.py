"""Thin ctypes binding of libkda.so (include/kda.h).  Argument marshalling only: every step
of the computation runs in the HIP kernels.  PyTorch supplies device memory and the stream.

There is no fallback: if libkda.so is missing or no GPU is present the calls raise.
"""
from __future__ import annotations

import ctypes
import functools
import itertools
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_OK = 0
KDA_F32 = 0
KDA_BF16 = 1
G_MIN = -5.0

# exported symbols, in the order include/kda.h declares them
SYMBOLS = ("kda_gate", "kda_prefill_workspace_size", "kda_prefill_fwd",
           "kda_prefill_fwd_noalloc", "kda_prefill_fwd_checkpointed", "kda_decode_step",
           "kda_decode_verify", "kda_decode_commit", "kda_output_gate", "kda_short_conv",
           "kda_status_str")
MAX_DRAFT = 16
NOALLOC_SCRATCH_BYTES = 64 << 20   # KDA_NOALLOC_SCRATCH_BYTES
KDA_ERR_SCRATCH = -7

_lib = None


class KDAError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed: {status_str(code)} ({code})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m linear_attention_sequence_chunkwise_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    lib.kda_status_str.argtypes = [i32]
    lib.kda_status_str.restype = ctypes.c_char_p
    lib.kda_gate.argtypes = [vp, vp, vp, vp, i64, i32, i32, vp, i32, i32, f32, vp]
    lib.kda_gate.restype = i32
    lib.kda_prefill_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32]
    lib.kda_prefill_workspace_size.restype = ctypes.c_size_t
    lib.kda_prefill_fwd.argtypes = [i32, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, i32, i64, i32,
                                    i32, i32, vp, vp, ctypes.c_size_t, vp]
    lib.kda_prefill_fwd.restype = i32
    lib.kda_prefill_fwd_noalloc.argtypes = [i32, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, i32,
                                            i64, i32, i32, i32, vp, vp]
    lib.kda_prefill_fwd_noalloc.restype = i32
    lib.kda_prefill_fwd_checkpointed.argtypes = [i32, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, i32,
                                                 i64, i32, i32, i32, vp, vp, vp, i32, vp,
                                                 ctypes.c_size_t, vp]
    lib.kda_prefill_fwd_checkpointed.restype = i32
    lib.kda_decode_step.argtypes = [i32, vp, vp, vp, vp, vp, vp, f32, vp, i32, i32, i32, i32, vp,
                                    vp]
    lib.kda_decode_step.restype = i32
    lib.kda_decode_verify.argtypes = [i32, vp, vp, vp, vp, vp, vp, f32, vp, i32, i32, i32, i32,
                                      i32, vp, vp]
    lib.kda_decode_verify.restype = i32
    lib.kda_decode_commit.argtypes = [i32, vp, vp, vp, vp, vp, f32, vp, i32, i32, i32, i32, i32,
                                      vp, vp]
    lib.kda_decode_commit.restype = i32
    lib.kda_output_gate.argtypes = [i32, vp, vp, vp, f32, i64, i32, vp, vp]
    lib.kda_output_gate.restype = i32
    lib.kda_short_conv.argtypes = [i32, vp, vp, i32, vp, vp, vp, i32, i64, i32, i32, vp, vp]
    lib.kda_short_conv.restype = i32
    _lib = lib
    return lib


def status_str(code: int) -> str:
    return load_library().kda_status_str(int(code)).decode()


kda_status_str = status_str


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported element type {t.dtype} (bf16 or fp32)")


def _check(fn: str, code: int):
    if code != KDA_OK:
        raise KDAError(fn, code)


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous and on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors on different devices ({dev} and {t.device})")


def _on_tensor_device(fn):
    """Run a binding call with its tensors' GPU current: the library launches on the current
    HIP device and sizes the prefill workspace for it."""
    @functools.wraps(fn)
    def run(*args, **kwargs):
        for a in itertools.chain(args, kwargs.values()):
            if isinstance(a, torch.Tensor) and a.is_cuda:
                with torch.cuda.device(a.device):
                    return fn(*args, **kwargs)
        return fn(*args, **kwargs)
    return run


def _expect(name: str, t: Optional[torch.Tensor], shape, dtype: torch.dtype):
    """The kernels take plain pointers and trust these shapes: check them before any call."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")


@_on_tensor_device
def kda_gate(z: torch.Tensor, A: torch.Tensor, g: Optional[torch.Tensor] = None,
             gcum: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None,
             n_seqs: int = 1, chunk: int = 64, g_min: float = G_MIN, want_g: bool = True,
             want_gcum: bool = True, stream=None):
    """g = g_min*Sigmoid(e^A z) and its chunk-local inclusive cumsum; z [T,H,dk], A [H,dk]."""
    lib = load_library()
    T, H, dk = z.shape
    if g is None and want_g:
        g = torch.empty_like(z)
    if gcum is None and want_gcum:
        gcum = torch.empty_like(z)
    if cu_seqlens is not None:
        n_seqs = cu_seqlens.numel() - 1
    f32 = torch.float32
    _expect("z", z, (T, H, dk), f32)
    _expect("A", A, (H, dk), f32)
    _expect("g", g, (T, H, dk), f32)
    _expect("gcum", gcum, (T, H, dk), f32)
    _expect("cu_seqlens", cu_seqlens, (n_seqs + 1,), torch.int32)
    _dev(z, A, g, gcum, cu_seqlens)
    _check("kda_gate", lib.kda_gate(_ptr(z), _ptr(A), _ptr(g), _ptr(gcum), T, H, dk,
                                    _ptr(cu_seqlens), n_seqs, chunk, g_min, _stream(stream)))
    return g, gcum


def kda_prefill_workspace_size(total_tokens: int, n_seqs: int, H: int, dk: int, dv: int,
                               dtype: torch.dtype = torch.bfloat16) -> int:
    """Workspace bytes kda_prefill_fwd needs on the current device (the fused form, taken by
    bf16 calls with a (sequence, head) chain per compute unit, needs only a small table)."""
    code = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    return int(load_library().kda_prefill_workspace_size(total_tokens, n_seqs, H, dk, dv, code))


@_on_tensor_device
def kda_prefill_fwd(q, k, v, beta, z, A, g_min: float = G_MIN, initial_state=None,
                    final_state=None, cu_seqlens=None, n_seqs: Optional[int] = None, o=None,
                    workspace=None, stream=None, checkpoints=None, checkpoint_offsets=None,
                    checkpoint_interval: int = 0):
    """Chunkwise prefill over packed tokens.  q,k,z [total,H,dk]; v [total,H,dv];
    beta [total,H]; A [H,dk]; states [N,H,dk,dv] fp32; cu_seqlens [N+1] int32 or None (then
    n_seqs equal-length sequences, default 1).  Returns o [total,H,dv].
    With `checkpoints` ([n_ckpt,H,dk,dv] fp32) the call goes to kda_prefill_fwd_checkpointed:
    the state after every `checkpoint_interval` tokens of each sequence is written there
    (`checkpoint_offsets` [N+1] int32 is required with cu_seqlens)."""
    lib = load_library()
    total, H, dk = q.shape
    dv = v.shape[2]
    dt = _dtype_code(q)
    if cu_seqlens is not None:
        N = cu_seqlens.numel() - 1
        T_or_total = total
    else:
        N = 1 if n_seqs is None else int(n_seqs)
        if total % N:
            raise ValueError("total tokens not divisible by n_seqs")
        T_or_total = total // N
    if o is None:
        o = torch.empty((total, H, dv), dtype=q.dtype, device=q.device)
    need = kda_prefill_workspace_size(total, N, H, dk, dv, q.dtype)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    et, f32 = q.dtype, torch.float32
    _expect("k", k, (total, H, dk), et)
    _expect("v", v, (total, H, dv), et)
    _expect("beta", beta, (total, H), et)
    _expect("z", z, (total, H, dk), f32)
    _expect("A", A, (H, dk), f32)
    _expect("initial_state", initial_state, (N, H, dk, dv), f32)
    _expect("final_state", final_state, (N, H, dk, dv), f32)
    _expect("cu_seqlens", cu_seqlens, (N + 1,), torch.int32)
    _expect("o", o, (total, H, dv), et)
    if checkpoints is not None:
        if checkpoints.dim() != 4 or tuple(checkpoints.shape[1:]) != (H, dk, dv) or checkpoints.dtype != f32:
            raise ValueError(f"checkpoints: expected fp32 [n_ckpt, {H}, {dk}, {dv}]")
        if cu_seqlens is None and checkpoint_interval > 0 and \
                checkpoints.shape[0] < N * (T_or_total // checkpoint_interval):
            raise ValueError("checkpoints: fewer rows than the sequences' checkpoints")
        _expect("checkpoint_offsets", checkpoint_offsets, (N + 1,), torch.int32)
    _dev(q, k, v, beta, z, A, initial_state, final_state, cu_seqlens, o, workspace, checkpoints,
         checkpoint_offsets)
    if checkpoints is not None:
        _check("kda_prefill_fwd_checkpointed", lib.kda_prefill_fwd_checkpointed(
            dt, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(z), _ptr(A), g_min,
            _ptr(initial_state), _ptr(final_state), _ptr(cu_seqlens), N, T_or_total, H, dk, dv,
            _ptr(o), _ptr(checkpoints), _ptr(checkpoint_offsets), int(checkpoint_interval),
            _ptr(workspace), wbytes, _stream(stream)))
        return o
    _check("kda_prefill_fwd", lib.kda_prefill_fwd(
        dt, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(z), _ptr(A), g_min, _ptr(initial_state),
        _ptr(final_state), _ptr(cu_seqlens), N, T_or_total, H, dk, dv, _ptr(o), _ptr(workspace),
        wbytes, _stream(stream)))
    return o


@_on_tensor_device
def kda_prefill_fwd_noalloc(q, k, v, beta, z, A, g_min: float = G_MIN, initial_state=None,
                            final_state=None, cu_seqlens=None, n_seqs: Optional[int] = None,
                            o=None, stream=None):
    """kda_prefill_fwd with its workspace in the library's static per-device scratch array
    (at most NOALLOC_SCRATCH_BYTES; larger problems raise KDAError with KDA_ERR_SCRATCH).
    Allocates nothing when `o` is given.  Calls that overlap on one device race."""
    lib = load_library()
    total, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens is not None:
        N = cu_seqlens.numel() - 1
        T_or_total = total
    else:
        N = 1 if n_seqs is None else int(n_seqs)
        if total % N:
            raise ValueError("total tokens not divisible by n_seqs")
        T_or_total = total // N
    if o is None:
        o = torch.empty((total, H, dv), dtype=q.dtype, device=q.device)
    et, f32 = q.dtype, torch.float32
    _expect("k", k, (total, H, dk), et)
    _expect("v", v, (total, H, dv), et)
    _expect("beta", beta, (total, H), et)
    _expect("z", z, (total, H, dk), f32)
    _expect("A", A, (H, dk), f32)
    _expect("initial_state", initial_state, (N, H, dk, dv), f32)
    _expect("final_state", final_state, (N, H, dk, dv), f32)
    _expect("cu_seqlens", cu_seqlens, (N + 1,), torch.int32)
    _expect("o", o, (total, H, dv), et)
    _dev(q, k, v, beta, z, A, initial_state, final_state, cu_seqlens, o)
    _check("kda_prefill_fwd_noalloc", lib.kda_prefill_fwd_noalloc(
        _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(z), _ptr(A), g_min,
        _ptr(initial_state), _ptr(final_state), _ptr(cu_seqlens), N, T_or_total, H, dk, dv,
        _ptr(o), _stream(stream)))
    return o


@_on_tensor_device
def kda_decode_step(q, k, v, beta, z, A, state, g_min: float = G_MIN, o=None, stream=None):
    """One decode step; q,k,z [N,H,dk]; v [N,H,dv]; beta [N,H]; state [N,H,dk,dv] fp32 is
    updated in place.  Returns o [N,H,dv]."""
    lib = load_library()
    N, H, dk = q.shape
    dv = v.shape[2]
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    et, f32 = q.dtype, torch.float32
    _expect("k", k, (N, H, dk), et)
    _expect("v", v, (N, H, dv), et)
    _expect("beta", beta, (N, H), et)
    _expect("z", z, (N, H, dk), f32)
    _expect("A", A, (H, dk), f32)
    _expect("state", state, (N, H, dk, dv), f32)
    _expect("o", o, (N, H, dv), et)
    _dev(q, k, v, beta, z, A, state, o)
    _check("kda_decode_step", lib.kda_decode_step(
        _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(z), _ptr(A), g_min,
        _ptr(state), N, H, dk, dv, _ptr(o), _stream(stream)))
    return o


@_on_tensor_device
def kda_decode_verify(q, k, v, beta, z, A, state, g_min: float = G_MIN, o=None, stream=None):
    """Outputs of K draft tokens per sequence from the committed state (read only);
    q,k,z [N,K,H,dk]; v [N,K,H,dv]; beta [N,K,H]; state [N,H,dk,dv] fp32.
    Returns o [N,K,H,dv]."""
    lib = load_library()
    N, K, H, dk = q.shape
    dv = v.shape[3]
    if o is None:
        o = torch.empty((N, K, H, dv), dtype=q.dtype, device=q.device)
    et, f32 = q.dtype, torch.float32
    _expect("k", k, (N, K, H, dk), et)
    _expect("v", v, (N, K, H, dv), et)
    _expect("beta", beta, (N, K, H), et)
    _expect("z", z, (N, K, H, dk), f32)
    _expect("A", A, (H, dk), f32)
    _expect("state", state, (N, H, dk, dv), f32)
    _expect("o", o, (N, K, H, dv), et)
    _dev(q, k, v, beta, z, A, state, o)
    _check("kda_decode_verify", lib.kda_decode_verify(
        _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(z), _ptr(A), g_min,
        _ptr(state), N, K, H, dk, dv, _ptr(o), _stream(stream)))
    return o


@_on_tensor_device
def kda_decode_commit(k, v, beta, z, A, state, accepted, g_min: float = G_MIN, stream=None):
    """Advance state [N,H,dk,dv] in place by the first accepted[n] (device int32 [N]) of the
    K draft tokens k,z [N,K,H,dk]; v [N,K,H,dv]; beta [N,K,H]."""
    lib = load_library()
    N, K, H, dk = k.shape
    dv = v.shape[3]
    et, f32 = k.dtype, torch.float32
    _expect("v", v, (N, K, H, dv), et)
    _expect("beta", beta, (N, K, H), et)
    _expect("z", z, (N, K, H, dk), f32)
    _expect("A", A, (H, dk), f32)
    _expect("state", state, (N, H, dk, dv), f32)
    _expect("accepted", accepted, (N,), torch.int32)
    _dev(k, v, beta, z, A, state, accepted)
    _check("kda_decode_commit", lib.kda_decode_commit(
        _dtype_code(k), _ptr(k), _ptr(v), _ptr(beta), _ptr(z), _ptr(A), g_min, _ptr(state), N, K,
        H, dk, dv, _ptr(accepted), _stream(stream)))
    return state


@_on_tensor_device
def kda_output_gate(o, gate, weight, eps: float = 1e-6, y=None, stream=None):
    """y = Sigmoid(gate) * o / sqrt(mean(o^2) + eps) * weight over the last axis (dv);
    o, gate [..., dv] of one dtype; weight [dv] fp32.  Returns y (new, or the given tensor)."""
    lib = load_library()
    dv = o.shape[-1]
    rows = o.numel() // dv if dv else 0
    if y is None:
        y = torch.empty_like(o)
    _expect("gate", gate, tuple(o.shape), o.dtype)
    _expect("weight", weight, (dv,), torch.float32)
    _expect("y", y, tuple(o.shape), o.dtype)
    _dev(o, gate, weight, y)
    _check("kda_output_gate", lib.kda_output_gate(
        _dtype_code(o), _ptr(o), _ptr(gate), _ptr(weight), float(eps), rows, dv, _ptr(y),
        _stream(stream)))
    return y


@_on_tensor_device
def kda_short_conv(x, weight, cache_in=None, cache_out=None, cu_seqlens=None,
                   n_seqs: Optional[int] = None, l2_group: int = 0, y=None, stream=None):
    """y = Swish(ShortConv(x)) (then L2Norm over groups of l2_group channels); x [total, C];
    weight [C, width] fp32; caches [N, C, width-1] fp32.  Returns y [total, C]."""
    lib = load_library()
    total, C = x.shape
    width = weight.shape[1]
    if cu_seqlens is not None:
        N = cu_seqlens.numel() - 1
        T_or_total = total
    else:
        N = 1 if n_seqs is None else int(n_seqs)
        if total % N:
            raise ValueError("total tokens not divisible by n_seqs")
        T_or_total = total // N
    if y is None:
        y = torch.empty_like(x)
    f32 = torch.float32
    _expect("weight", weight, (C, width), f32)
    if width > 1:
        _expect("cache_in", cache_in, (N, C, width - 1), f32)
        _expect("cache_out", cache_out, (N, C, width - 1), f32)
    _expect("cu_seqlens", cu_seqlens, (N + 1,), torch.int32)
    _expect("y", y, (total, C), x.dtype)
    _dev(x, weight, cache_in, cache_out, cu_seqlens, y)
    _check("kda_short_conv", lib.kda_short_conv(
        _dtype_code(x), _ptr(x), _ptr(weight), width, _ptr(cache_in), _ptr(cache_out),
        _ptr(cu_seqlens), N, T_or_total, C, int(l2_group), _ptr(y), _stream(stream)))
    return y
