"""GPU parity at the named workloads' full sizes, in the launch configuration bench.py times.

The GPU computes the whole workload; the oracle recomputes sampled (sequence, head) pairs one
by one (pairs are independent, so each sampled pair's outputs and final state are exact
references).  Same tolerances as the small parity tests.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_chunkwise_amd import kda, workloads
from tests.gpu_util import OUT_TOL, STATE_TOL, max_abs, note, state_rel_err

pytestmark = pytest.mark.gpu


def _run_full(inp, want_state):
    c = lambda t: None if t is None else t.cuda()
    sN = torch.empty((inp.N, inp.H, inp.dk, inp.dv), dtype=torch.float32, device="cuda") \
        if want_state else None
    cu = None if inp.equal_length else c(inp.cu_seqlens)
    o = kda.kda_prefill_fwd(c(inp.q), c(inp.k), c(inp.v), c(inp.beta), c(inp.z), c(inp.A),
                            initial_state=c(inp.S0), final_state=sN, cu_seqlens=cu,
                            n_seqs=None if cu is not None else inp.N)
    torch.cuda.synchronize()
    return o, sN


def _check_pairs(inp, o, sN, pairs):
    orc = oracle.load()
    worst_o = worst_s = 0.0
    for n, h in pairs:
        p = inp.pair_slice(n, h)
        o_ref, S_ref = orc.prefill(p["q"], p["k"], p["v"], p["beta"], z=p["z"], A=p["A"],
                                   S0=p["S0"])
        s, e = int(inp.cu_seqlens[n]), int(inp.cu_seqlens[n + 1])
        og = o[s:e, h].float().cpu().numpy()
        eo = max_abs(og, o_ref[:, 0])
        es = 0.0 if sN is None else state_rel_err(sN[n, h].cpu().numpy()[None],
                                                   S_ref.reshape(1, inp.dk, inp.dv))
        note(f"    pair (seq {n}, head {h}) L={e - s}: max|do| = {eo:.3e}  rel dS = {es:.3e}")
        worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
    assert worst_o <= OUT_TOL and worst_s <= STATE_TOL
    return worst_o, worst_s


def test_prefill_b1_h16_t4096_all_heads():
    inp = workloads.make(workloads.PREFILL_B1)
    note(f"[full] {inp.name}")
    o, sN = _run_full(inp, want_state=True)
    _check_pairs(inp, o, sN, [(0, h) for h in range(inp.H)])


def test_prefill_b4_h32_t32768_sampled():
    inp = workloads.make(workloads.PREFILL_B4)
    note(f"[full] {inp.name}")
    o, sN = _run_full(inp, want_state=True)
    assert torch.isfinite(o.float()).all() and torch.isfinite(sN).all()
    _check_pairs(inp, o, sN, [(0, 0), (1, 17), (2, 5), (3, 31)])


def test_prefill_varlen64_h32_sampled():
    inp = workloads.make(workloads.PREFILL_VARLEN)
    note(f"[full] {inp.name} total={inp.total} min/max len={min(inp.lengths)}/{max(inp.lengths)}")
    o, sN = _run_full(inp, want_state=True)
    assert torch.isfinite(o.float()).all() and torch.isfinite(sN).all()
    L = np.array(inp.lengths)
    pairs = [(int(L.argmax()), 0), (int(L.argmin()), 31), (int(np.argsort(L)[32]), 13),
             (63, 7)]
    _check_pairs(inp, o, sN, pairs)


def test_decode_n512_h32_256_steps_sampled():
    d = workloads.make(workloads.DECODE)
    note(f"[full] {d.name}")
    pairs = [(0, 0), (511, 31), (100, 7), (257, 20), (33, 31), (400, 2)]
    pa = np.array(pairs, dtype=np.int32)
    S_ref = np.ascontiguousarray(np.stack([d.S0[n, h].numpy() for n, h in pairs]).astype(np.float64))
    state = d.S0.cuda()
    A = d.A.cuda()
    orc = oracle.load()
    worst = 0.0
    f = lambda t: t.float().numpy()
    for t in range(d.steps):
        o = kda.kda_decode_step(d.q[t].cuda(), d.k[t].cuda(), d.v[t].cuda(), d.beta[t].cuda(),
                                d.z[t].cuda(), A, state)
        o_ref = orc.decode_step(f(d.q[t]), f(d.k[t]), f(d.v[t]), f(d.beta[t]), d.z[t].numpy(),
                                d.A.numpy(), S_ref, pairs=pa)
        og = o.float().cpu().numpy()
        worst = max(worst, max_abs(np.stack([og[n, h] for n, h in pairs]), o_ref))
    torch.cuda.synchronize()
    Sg = np.stack([state[n, h].cpu().numpy() for n, h in pairs])
    es = state_rel_err(Sg, S_ref)
    note(f"    256 steps: max|do| = {worst:.3e}  rel dS = {es:.3e}")
    assert worst <= OUT_TOL and es <= STATE_TOL


def test_spec_decode_n512_h32_k4_sampled():
    """One speculative round at the timed size (512 sequences x 32 heads, d = 128, bf16, K = 4):
    verify's per-position outputs and commit's states for accepted counts 0..4 (and one
    value above K, which clamps to K), on sampled (sequence, head) pairs."""
    K = 4
    d = workloads.decode_inputs(N=512, H=32, dk=128, dv=128, steps=K, dtype="bf16", seed=5,
                                name="spec_decode_n512_h32_d128_bf16")
    note(f"[full] {d.name} K={K}")
    nk = lambda x: x.transpose(0, 1).contiguous().cuda()  # [K, N, ...] -> [N, K, ...]
    q, k, v, beta, z = (nk(t) for t in (d.q, d.k, d.v, d.beta, d.z))
    A = d.A.cuda()
    state = d.S0.cuda()
    rng = np.random.default_rng(6)
    acc = rng.integers(0, K + 1, d.N).astype(np.int32)
    pairs = [(0, 0), (511, 31), (100, 7), (257, 20), (33, 31), (400, 2)]
    for (n, _), a in zip(pairs, [0, 4, 7, 1, 2, 3]):
        acc[n] = a
    o = kda.kda_decode_verify(q, k, v, beta, z, A, state)
    torch.cuda.synchronize()
    og = np.stack([o[n, :, h].float().cpu().numpy() for n, h in pairs])  # [P, K, dv]
    untouched = all(torch.equal(state[n, h], d.S0[n, h].cuda()) for n, h in pairs)
    kda.kda_decode_commit(k, v, beta, z, A, state, torch.from_numpy(acc).cuda())
    torch.cuda.synchronize()

    pa = np.array(pairs, dtype=np.int32)
    S_ref = np.ascontiguousarray(np.stack([d.S0[n, h].numpy() for n, h in pairs]).astype(np.float64))
    orc = oracle.load()
    f = lambda t: t.float().numpy()
    o_ref, snaps = [], [S_ref.copy()]
    for t in range(K):
        o_ref.append(orc.decode_step(f(d.q[t]), f(d.k[t]), f(d.v[t]), f(d.beta[t]), d.z[t].numpy(),
                                     d.A.numpy(), S_ref, pairs=pa))
        snaps.append(S_ref.copy())
    e_o = max_abs(og, np.stack(o_ref, 1))
    S_want = np.stack([snaps[min(int(acc[n]), K)][i] for i, (n, _) in enumerate(pairs)])
    Sg = np.stack([state[n, h].cpu().numpy() for n, h in pairs])
    e_s = state_rel_err(Sg, S_want)
    note(f"    verify max|do| = {e_o:.3e}   commit rel dS = {e_s:.3e}")
    assert untouched
    assert e_o <= OUT_TOL and e_o <= 2e-3
    assert e_s <= STATE_TOL and e_s <= 1e-4
