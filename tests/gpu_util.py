"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI binding and
the CPU oracle on identical inputs, and measure the disagreement the way the acceptance
criteria state it:
  * outputs: max over every element of |o_gpu - o_oracle|            (bound 2e-2)
  * states:  per (sequence, head) ||S_gpu - S_ref||_F / max(||S_ref||_F, 1e-6), max over
             pairs                                                   (bound 1e-2)
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from linear_attention_sequence_chunkwise_amd import kda

OUT_TOL = 2e-2
STATE_TOL = 1e-2


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(t):
    return None if t is None else t.cuda()


def gpu_prefill(inp, use_cu=None, with_state=True, final_into_initial=False):
    """Run kda_prefill_fwd on a workloads.PrefillInputs; returns (o fp64 numpy, S fp64 numpy)."""
    if use_cu is None:
        use_cu = not inp.equal_length
    q, k, v, beta = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.beta)
    z, A = dev(inp.z), dev(inp.A)
    s0 = dev(inp.S0)
    N, H, dk, dv = inp.N, inp.H, inp.dk, inp.dv
    sN = None
    if with_state:
        sN = s0 if (final_into_initial and s0 is not None) else torch.empty(
            (N, H, dk, dv), dtype=torch.float32, device="cuda")
    cu = dev(inp.cu_seqlens) if use_cu else None
    o = kda.kda_prefill_fwd(q, k, v, beta, z, A, initial_state=s0, final_state=sN,
                            cu_seqlens=cu, n_seqs=None if use_cu else N)
    torch.cuda.synchronize()
    o_np = o.float().cpu().numpy().astype(np.float64)
    S_np = None if sN is None else sN.cpu().numpy().astype(np.float64)
    return o_np, S_np


def oracle_prefill(inp, pairs=None, threads=0):
    orc = oracle.load()
    f = lambda t: t.float().numpy()
    return orc.prefill(f(inp.q), f(inp.k), f(inp.v), f(inp.beta), z=inp.z.numpy(),
                       A=inp.A.numpy(), S0=None if inp.S0 is None else inp.S0.numpy(),
                       cu_seqlens=inp.cu_seqlens.numpy(), pairs=pairs, n_threads=threads)


def state_rel_err(S, Sref):
    S = np.asarray(S, np.float64).reshape(-1, Sref.shape[-2] * Sref.shape[-1])
    R = np.asarray(Sref, np.float64).reshape(S.shape)
    num = np.linalg.norm(S - R, axis=1)
    den = np.maximum(np.linalg.norm(R, axis=1), 1e-6)
    return float(np.max(num / den)) if len(num) else 0.0


def max_abs(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0
