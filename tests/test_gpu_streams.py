"""Calls on several streams at once.  The library keeps no state between calls: everything a
call uses lives in the caller's tensors and workspace, and it works on the stream it is given.
So three prefills (two on the split kernels, one on the fused kernel) and a decode launched
together on four streams (default priority), each with its own workspace, must give exactly
the results of the same calls run one after another.
"""
from __future__ import annotations

import pytest
import torch

from linear_attention_sequence_chunkwise_amd import kda, workloads
from tests.gpu_util import dev, note

pytestmark = pytest.mark.gpu


def _prefill_bufs(inp, use_cu):
    q, k, v, b, z, A, s0 = (dev(t) for t in (inp.q, inp.k, inp.v, inp.beta, inp.z, inp.A, inp.S0))
    cu = dev(inp.cu_seqlens) if use_cu else None
    o = torch.empty((inp.total, inp.H, inp.dv), dtype=q.dtype, device="cuda")
    sN = torch.empty((inp.N, inp.H, inp.dk, inp.dv), dtype=torch.float32, device="cuda")
    ws = torch.empty(kda.kda_prefill_workspace_size(inp.total, inp.N, inp.H, inp.dk, inp.dv, q.dtype),
                     dtype=torch.uint8, device="cuda")

    def call(stream):
        kda.kda_prefill_fwd(q, k, v, b, z, A, initial_state=s0, final_state=sN, cu_seqlens=cu,
                            n_seqs=None if use_cu else inp.N, o=o, workspace=ws, stream=stream)
    return call, (o, sN)


def _decode_bufs(d):
    q, k, v, b, z = (t.cuda() for t in (d.q, d.k, d.v, d.beta, d.z))
    A, s_init = d.A.cuda(), d.S0.cuda()
    state = s_init.clone()
    o = torch.empty((d.steps, d.N, d.H, d.dv), dtype=q.dtype, device="cuda")

    def call(stream):
        for t in range(d.steps):
            kda.kda_decode_step(q[t], k[t], v[t], b[t], z[t], A, state, o=o[t], stream=stream)
    return call, (o, state), lambda: state.copy_(s_init)


def test_concurrent_streams_match_sequential():
    a = workloads.prefill_inputs([300, 0, 77, 129], H=8, dk=128, dv=128, dtype="bf16", seed=71,
                                 s0_std=0.02, name="streams_a")
    b = workloads.prefill_inputs([256, 256], H=4, dk=64, dv=64, dtype="fp32", seed=72,
                                 s0_std=0.02, name="streams_b")
    d = workloads.decode_inputs(N=64, H=8, dk=128, dv=128, steps=2, dtype="bf16", seed=73,
                                name="streams_decode")
    # 256 chains: the fused kernel (on 256 CUs), beside the split calls above
    f = workloads.prefill_inputs([300, 0, 77, 129], H=64, dk=128, dv=128, dtype="bf16", seed=74,
                                 s0_std=0.02, name="streams_fused")
    run_a, out_a = _prefill_bufs(a, use_cu=True)
    run_b, out_b = _prefill_bufs(b, use_cu=False)
    run_d, out_d, reset_d = _decode_bufs(d)
    run_f, out_f = _prefill_bufs(f, use_cu=True)
    outs = out_a + out_b + out_d + out_f

    main = torch.cuda.current_stream()
    for run in (run_a, run_b, run_d, run_f):
        run(main)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    for t in outs:
        t.zero_()
    reset_d()
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(4)]
    for s, run in zip(streams, (run_a, run_b, run_d, run_f)):
        s.wait_stream(main)
        run(s)
    torch.cuda.synchronize()
    same = [torch.equal(t, r) for t, r in zip(outs, ref)]
    note(f"[streams] prefill varlen bf16 d128, prefill batch fp32 d64, decode 2 steps, fused "
         f"prefill: identical = {same}")
    assert all(same)
