"""CPU fp64 oracle for the KDA forward pass -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this
package.  The product path (the HIP library and its Python binding) never imports, links or
calls it, and the oracle shares no code with that path.

The arithmetic lives in ``kda_oracle.c`` (plain C99, fp64, OpenMP over (sequence, head)
pairs); this module only builds it with gcc and marshals numpy arrays through ctypes.
Definitions follow "Kimi K3: Architecture, Training, and Million-Token Agentic RL"
§3.1-§3.3 (recurrence, edit/read order, lower-bounded gate); see the C file's header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")

G_MIN = -5.0  # lower bound of the log-decay, "Kimi K3: Architecture..." §3.3


def build(out: str = LIB_PATH, mutant: int = 0, quiet: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP).  ``mutant`` > 0 plants one
    known mistake (tests only).  Returns the path of the shared object."""
    cmd = ["gcc", "-std=c99", "-O2", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
           f"-DKDA_ORACLE_MUTANT={int(mutant)}", _SRC, "-o", out, "-lm"]
    subprocess.run(cmd, check=True, capture_output=quiet)
    return out


_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_ip = ctypes.POINTER(ctypes.c_int32)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a: Optional[np.ndarray], typ):
    if a is None:
        return ctypes.cast(None, typ)
    return a.ctypes.data_as(typ)


class Oracle:
    """ctypes front end of one compiled oracle (the real one or a planted mutant)."""

    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            raise FileNotFoundError(f"oracle library {path} is not built; run oracle.build()")
        self.path = path
        lib = ctypes.CDLL(path)
        lib.kda_oracle_mutant.restype = ctypes.c_int
        lib.kda_oracle_gate.argtypes = [_fp, _fp, ctypes.c_double, ctypes.c_int64, ctypes.c_int,
                                        ctypes.c_int, _dp]
        lib.kda_oracle_gate.restype = None
        lib.kda_oracle_chunk_cumsum.argtypes = [_dp, _ip, ctypes.c_int, ctypes.c_int64,
                                                ctypes.c_int, ctypes.c_int, ctypes.c_int, _dp]
        lib.kda_oracle_chunk_cumsum.restype = ctypes.c_int
        lib.kda_oracle_prefill.argtypes = [_fp, _fp, _fp, _fp, _fp, _fp, _dp, ctypes.c_double,
                                           _fp, _ip, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, _ip, ctypes.c_int, _dp,
                                           _dp, ctypes.c_int]
        lib.kda_oracle_prefill.restype = ctypes.c_int
        lib.kda_oracle_output_gate.argtypes = [_fp, _fp, _fp, ctypes.c_double, ctypes.c_int64,
                                               ctypes.c_int, _dp]
        lib.kda_oracle_output_gate.restype = None
        lib.kda_oracle_short_conv.argtypes = [_fp, _fp, ctypes.c_int, _fp, _dp, _ip, ctypes.c_int,
                                              ctypes.c_int64, ctypes.c_int, ctypes.c_int, _dp]
        lib.kda_oracle_short_conv.restype = ctypes.c_int
        lib.kda_oracle_decode_step.argtypes = [_fp, _fp, _fp, _fp, _fp, _fp, ctypes.c_double,
                                               _dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, _ip, ctypes.c_int, _dp,
                                               ctypes.c_int]
        lib.kda_oracle_decode_step.restype = ctypes.c_int
        self.lib = lib
        self.mutant = lib.kda_oracle_mutant()

    # -- gate ---------------------------------------------------------------------------
    def gate(self, z, A, g_min: float = G_MIN) -> np.ndarray:
        """g = g_min * Sigmoid(exp(A) * z) for z [T, H, dk] and A [H, dk]; fp64 result."""
        z = _f32(z)
        A = _f32(A)
        T, H, dk = z.shape
        assert A.shape == (H, dk)
        g = np.empty(z.shape, dtype=np.float64)
        self.lib.kda_oracle_gate(_ptr(z, _fp), _ptr(A, _fp), g_min, T, H, dk, _ptr(g, _dp))
        return g

    def chunk_cumsum(self, g, cu_seqlens=None, chunk: int = 64) -> np.ndarray:
        """Chunk-local inclusive cumsum of g [total, H, dk] (chunks restart per sequence)."""
        g = np.ascontiguousarray(g, dtype=np.float64)
        total, H, dk = g.shape
        out = np.empty_like(g)
        if cu_seqlens is None:
            cu = None
            N, T = 1, total
        else:
            cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
            N, T = len(cu) - 1, 0
        rc = self.lib.kda_oracle_chunk_cumsum(_ptr(g, _dp), _ptr(cu, _ip), N, T, H, dk, chunk,
                                              _ptr(out, _dp))
        if rc != 0:
            raise ValueError(f"kda_oracle_chunk_cumsum failed: {rc}")
        return out

    # -- prefill ------------------------------------------------------------------------
    def prefill(self, q, k, v, beta, z=None, A=None, g=None, g_min: float = G_MIN,
                S0=None, cu_seqlens=None, pairs: Optional[Sequence[Sequence[int]]] = None,
                n_threads: int = 0, want_state: bool = True):
        """Token recurrence over packed sequences.

        q, k, z: [total, H, dk]; v: [total, H, dv]; beta: [total, H]; A: [H, dk];
        g: optional fp64 log-decay [total, H, dk] replacing the gate; S0: [N, H, dk, dv];
        cu_seqlens: [N+1] or None (then one sequence of length total).

        Without ``pairs`` returns (o [total, H, dv], S [N, H, dk, dv]) in fp64.  With
        ``pairs`` ((n, h) list) returns (list of o [L_n, dv], S [n_pairs, dk, dv]).
        """
        q, k, v, beta = _f32(q), _f32(k), _f32(v), _f32(beta)
        total, H, dk = q.shape
        dv = v.shape[2]
        if cu_seqlens is None:
            cu = np.array([0, total], dtype=np.int32)
        else:
            cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        N = len(cu) - 1
        zf = _f32(z) if z is not None else None
        Af = _f32(A) if A is not None else None
        gd = np.ascontiguousarray(g, dtype=np.float64) if g is not None else None
        s0 = _f32(S0) if S0 is not None else None
        if pairs is None:
            pa = None
            plist = [(n, h) for n in range(N) for h in range(H)]
        else:
            plist = [(int(n), int(h)) for n, h in pairs]
            pa = np.ascontiguousarray(np.array(plist, dtype=np.int32).reshape(-1, 2))
        lens = [int(cu[n + 1] - cu[n]) for n, _ in plist]
        o_packed = np.empty((max(sum(lens), 1), dv), dtype=np.float64)
        S_out = np.empty((len(plist), dk, dv), dtype=np.float64) if want_state else None
        rc = self.lib.kda_oracle_prefill(
            _ptr(q, _fp), _ptr(k, _fp), _ptr(v, _fp), _ptr(beta, _fp), _ptr(zf, _fp),
            _ptr(Af, _fp), _ptr(gd, _dp), g_min, _ptr(s0, _fp), _ptr(cu, _ip), N, 0, H, dk, dv,
            _ptr(pa, _ip), len(plist), _ptr(o_packed, _dp), _ptr(S_out, _dp), int(n_threads))
        if rc != 0:
            raise ValueError(f"kda_oracle_prefill failed: {rc}")
        offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        if pairs is None:
            o = np.empty((total, H, dv), dtype=np.float64)
            for p, (n, h) in enumerate(plist):
                o[cu[n]:cu[n + 1], h, :] = o_packed[offs[p]:offs[p + 1]]
            S = S_out.reshape(N, H, dk, dv) if want_state else None
            return o, S
        outs = [o_packed[offs[p]:offs[p + 1]].copy() for p in range(len(plist))]
        return outs, S_out

    # -- decode -------------------------------------------------------------------------
    def decode_step(self, q, k, v, beta, z, A, S: np.ndarray, pairs=None, g_min: float = G_MIN,
                    n_threads: int = 0) -> np.ndarray:
        """Advance fp64 states S ([N,H,dk,dv] for all pairs, else [n_pairs,dk,dv]) by one
        token in place; returns o ([N,H,dv] or [n_pairs,dv]) in fp64."""
        q, k, v, beta, z, A = _f32(q), _f32(k), _f32(v), _f32(beta), _f32(z), _f32(A)
        N, H, dk = q.shape
        dv = v.shape[2]
        assert S.dtype == np.float64 and S.flags.c_contiguous
        if pairs is None:
            pa = None
            np_ = N * H
            o = np.empty((N, H, dv), dtype=np.float64)
        else:
            pa = np.ascontiguousarray(np.array(pairs, dtype=np.int32).reshape(-1, 2))
            np_ = pa.shape[0]
            o = np.empty((np_, dv), dtype=np.float64)
        assert S.size == np_ * dk * dv
        rc = self.lib.kda_oracle_decode_step(
            _ptr(q, _fp), _ptr(k, _fp), _ptr(v, _fp), _ptr(beta, _fp), _ptr(z, _fp),
            _ptr(A, _fp), g_min, _ptr(S, _dp), N, H, dk, dv, _ptr(pa, _ip), np_,
            _ptr(o, _dp), int(n_threads))
        if rc != 0:
            raise ValueError(f"kda_oracle_decode_step failed: {rc}")
        return o

    def output_gate(self, o, gate, w, eps: float = 1e-6):
        """y = Sigmoid(gate) * o / sqrt(mean(o^2) + eps) * w per row of the last axis (fp64)."""
        o, gate, w = _f32(o), _f32(gate), _f32(w)
        dv = o.shape[-1]
        rows = o.size // dv
        assert gate.shape == o.shape and w.shape == (dv,)
        y = np.empty(o.shape, dtype=np.float64)
        self.lib.kda_oracle_output_gate(_ptr(o, _fp), _ptr(gate, _fp), _ptr(w, _fp), float(eps),
                                        rows, dv, _ptr(y, _dp))
        return y

    def short_conv(self, x, w, cache_in=None, cu_seqlens=None, l2_group: int = 0):
        """Causal depthwise conv (width w.shape[1]) + Swish (+ L2Norm over groups) per
        sequence; x [total, C]; returns (y [total, C], cache_out [N, C, W-1]) in fp64."""
        x, w = _f32(x), _f32(w)
        total, C = x.shape
        Wk = w.shape[1]
        cu = np.array([0, total], np.int32) if cu_seqlens is None else \
            np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        N = len(cu) - 1
        ci = None if cache_in is None else _f32(cache_in)
        y = np.empty((total, C), np.float64)
        co = np.zeros((N, C, max(Wk - 1, 0)), np.float64)
        rc = self.lib.kda_oracle_short_conv(_ptr(x, _fp), _ptr(w, _fp), Wk, _ptr(ci, _fp),
                                            _ptr(co, _dp), _ptr(cu, _ip), N, 0, C, int(l2_group),
                                            _ptr(y, _dp))
        if rc != 0:
            raise ValueError(f"kda_oracle_short_conv failed: {rc}")
        return y, co


_default: Optional[Oracle] = None


def load() -> Oracle:
    """The real oracle (built on first use when gcc is available)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build()
        _default = Oracle(LIB_PATH)
    return _default
