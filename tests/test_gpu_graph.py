"""HIP-graph capture: the library allocates nothing and issues no memset, so a prefill call
(varlen, with initial and final state) followed by decode steps can be captured once and
replayed.  Every replay, with eager work and synchronisations in between, must reproduce
the eager results bit for bit.
"""
from __future__ import annotations

import pytest
import torch

from linear_attention_sequence_chunkwise_amd import kda, workloads
from tests.gpu_util import note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("H", [4, 64])
def test_prefill_and_decode_graph_replays_match_eager(H):
    """H = 4: 16 chains, the split kernels; H = 64: 256 chains, the fused kernel (on 256 CUs)."""
    inp = workloads.prefill_inputs([150, 0, 97, 64], H=H, dk=128, dv=128, dtype="bf16", seed=61,
                                   s0_std=0.02, name=f"graph_varlen_h{H}")
    dec = workloads.decode_inputs(N=4, H=H, dk=128, dv=128, steps=3, dtype="bf16", seed=62,
                                  name="graph_decode")
    c = lambda t: t.cuda()
    q, k, v, b, z, A, s0 = map(c, (inp.q, inp.k, inp.v, inp.beta, inp.z, inp.A, inp.S0))
    cu = c(inp.cu_seqlens)
    dq, dk_, dv_, db, dz = map(c, (dec.q, dec.k, dec.v, dec.beta, dec.z))
    dA = c(dec.A)
    ws = torch.empty(kda.kda_prefill_workspace_size(inp.total, inp.N, inp.H, inp.dk, inp.dv, q.dtype),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty((inp.total, inp.H, inp.dv), dtype=q.dtype, device="cuda")
    sN = torch.empty((inp.N, inp.H, inp.dk, inp.dv), dtype=torch.float32, device="cuda")
    od = torch.empty((dec.steps, dec.N, dec.H, dec.dv), dtype=q.dtype, device="cuda")

    def step():
        kda.kda_prefill_fwd(q, k, v, b, z, A, initial_state=s0, final_state=sN, cu_seqlens=cu,
                            o=o, workspace=ws)
        # the prefill's final state feeds the decode steps (updated in place)
        for t in range(dec.steps):
            kda.kda_decode_step(dq[t], dk_[t], dv_[t], db[t], dz[t], dA, sN, o=od[t])

    step()
    torch.cuda.synchronize()
    ref = (o.clone(), sN.clone(), od.clone())

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        o.zero_(); sN.zero_(); od.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(o, ref[0]) and torch.equal(sN, ref[1]) and torch.equal(od, ref[2])
        note(f"    replay {rep}: identical to eager = {same}")
        assert same
        # unrelated eager work between replays
        x = torch.randn(1 << 20, device="cuda")
        (x * 2).sum().item()


def test_serving_calls_graph_replays_match_eager():
    """The serving-side calls in one captured graph: the input prologue with its caches, a
    speculative verify and commit (the state advanced in place), and the output epilogue.
    The state is reset before every run; each replay must equal the eager run bit for bit."""
    N, K, H, d, C = 5, 4, 4, 128, 4 * 128
    gen = torch.Generator().manual_seed(63)
    lens = [7, 0, 3, 12, 1]
    cu = torch.tensor([0, 7, 7, 10, 22, 23], dtype=torch.int32).cuda()
    x = torch.randn(sum(lens), C, generator=gen).to(torch.bfloat16).cuda()
    w = (torch.randn(C, 4, generator=gen) * 0.5).cuda()
    cache = torch.randn(N, C, 3, generator=gen).to(torch.bfloat16).float().cuda()
    dec = workloads.decode_inputs(N=N, H=H, dk=d, dv=d, steps=K, dtype="bf16", seed=64,
                                  name="graph_spec")
    nk = lambda t: t.transpose(0, 1).contiguous().cuda()
    q, k, v, b, z = (nk(t) for t in (dec.q, dec.k, dec.v, dec.beta, dec.z))
    A, s_init = dec.A.cuda(), dec.S0.cuda()
    acc = torch.tensor([4, 0, 2, 9, 1], dtype=torch.int32).cuda()
    gate = torch.randn(N, K, H, d, generator=gen).to(torch.bfloat16).cuda()
    wn = (1.0 + 0.1 * torch.randn(d, generator=gen)).cuda()
    state = s_init.clone()
    yc = torch.empty_like(x)
    co = torch.empty_like(cache)
    ov = torch.empty((N, K, H, d), dtype=torch.bfloat16, device="cuda")
    yo = torch.empty_like(ov)

    def step():
        kda.kda_short_conv(x, w, cache_in=cache, cache_out=co, cu_seqlens=cu, l2_group=128, y=yc)
        kda.kda_decode_verify(q, k, v, b, z, A, state, o=ov)
        kda.kda_decode_commit(k, v, b, z, A, state, acc)
        kda.kda_output_gate(ov, gate, wn, y=yo)

    outs = (yc, co, ov, state, yo)
    step()
    torch.cuda.synchronize()
    ref = tuple(t.clone() for t in outs)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (yc, co, ov, yo):
            t.zero_()
        state.copy_(s_init)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = all(torch.equal(a, r) for a, r in zip(outs, ref))
        note(f"    replay {rep}: identical to eager = {same}")
        assert same
        x2 = torch.randn(1 << 20, device="cuda")
        (x2 * 2).sum().item()
