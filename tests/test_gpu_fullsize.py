"""GPU parity at the named workloads' full sizes, in the launch configuration bench.py times.

The GPU computes the whole workload and the oracle recomputes every (sequence, head) pair:
all outputs and all final states are compared, with the tolerances of the small parity tests.
The standalone kernels at the end are checked on sampled outputs at their timed sizes.
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


def _check_all_pairs(inp, o, sN):
    """Every (sequence, head) pair against the oracle, one sequence (all heads) per oracle call
    so host memory stays bounded; returns the worst output and state errors."""
    orc = oracle.load()
    f = lambda t: t.float().numpy()
    o_cpu = o.cpu()
    S_cpu = None if sN is None else sN.cpu().numpy()
    cu = inp.cu_seqlens.numpy()
    worst_o = worst_s = 0.0
    for n in range(inp.N):
        s, e = int(cu[n]), int(cu[n + 1])
        S0 = None if inp.S0 is None else inp.S0[n:n + 1].numpy()
        if e == s:
            if S_cpu is not None:
                want = np.zeros_like(S_cpu[n]) if S0 is None else S0[0]
                assert np.array_equal(S_cpu[n], want)
            continue
        o_ref, S_ref = orc.prefill(f(inp.q[s:e]), f(inp.k[s:e]), f(inp.v[s:e]),
                                   f(inp.beta[s:e]), z=inp.z[s:e].numpy(), A=inp.A.numpy(),
                                   S0=S0)
        eo = max_abs(o_cpu[s:e].float().numpy(), o_ref)
        es = 0.0 if S_cpu is None else state_rel_err(S_cpu[n], S_ref[0])
        worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
    note(f"    all {inp.N * inp.H} pairs: max|do| = {worst_o:.3e}  max rel dS = {worst_s:.3e}")
    assert worst_o <= OUT_TOL and worst_s <= STATE_TOL
    return worst_o, worst_s


def test_prefill_b1_h16_t4096_all_pairs():
    inp = workloads.make(workloads.PREFILL_B1)
    note(f"[full] {inp.name}")
    o, sN = _run_full(inp, want_state=True)
    _check_all_pairs(inp, o, sN)


def test_prefill_b4_h32_t32768_all_pairs():
    inp = workloads.make(workloads.PREFILL_B4)
    note(f"[full] {inp.name}")
    o, sN = _run_full(inp, want_state=True)
    assert torch.isfinite(o.float()).all() and torch.isfinite(sN).all()
    _check_all_pairs(inp, o, sN)


def test_prefill_b4_h32_t32768_slow_decay_all_pairs():
    """The batched workload's shape (4 x 32768 tokens, 32 heads: 128 chains of 512 chunks, the
    four-wave state pass) with slow-decay gates z ~ N(-4, 1) and an initial state, so the
    state persists across chunks and its bf16 rounding inside the state products accumulates
    over the longest chains of any workload."""
    inp = workloads.prefill_inputs([32768] * 4, H=32, dk=128, dv=128, dtype="bf16", seed=22,
                                   z_mean=-4.0, s0_std=0.02,
                                   name="prefill_b4_h32_t32768_d128_bf16_z-4_s0")
    note(f"[full] {inp.name}")
    o, sN = _run_full(inp, want_state=True)
    assert torch.isfinite(o.float()).all() and torch.isfinite(sN).all()
    _check_all_pairs(inp, o, sN)


def test_prefill_fused_long_chains_slow_decay_all_pairs():
    """The fused kernel (8 sequences x 32 heads = 256 chains, one per compute unit) over chains
    of 63 chunks with slow-decay gates z ~ N(-4, 1) and an initial state of unit scale, so the
    state carried in the consumers' accumulators persists, and is rounded to bf16 for the
    chunk products, over every chunk of every chain."""
    inp = workloads.prefill_inputs([4000] * 8, H=32, dk=128, dv=128, dtype="bf16", seed=23,
                                   z_mean=-4.0, s0_std=1.0,
                                   name="prefill_b8_h32_t4000_d128_bf16_z-4_s0")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if inp.N * inp.H < cus:
        pytest.skip(f"{inp.N * inp.H} chains do not reach the fused form on {cus} CUs")
    note(f"[full] {inp.name}")
    o, sN = _run_full(inp, want_state=True)
    assert torch.isfinite(o.float()).all() and torch.isfinite(sN).all()
    _check_all_pairs(inp, o, sN)


def test_prefill_varlen64_h32_all_pairs():
    inp = workloads.make(workloads.PREFILL_VARLEN)
    note(f"[full] {inp.name} total={inp.total} min/max len={min(inp.lengths)}/{max(inp.lengths)}")
    o, sN = _run_full(inp, want_state=True)
    assert torch.isfinite(o.float()).all() and torch.isfinite(sN).all()
    _check_all_pairs(inp, o, sN)


def test_decode_n512_h32_256_steps_all_pairs():
    """256 consecutive decode steps over all 512 x 32 (sequence, head) pairs: every output of
    every step and every final state against the oracle's fp64 steps."""
    d = workloads.make(workloads.DECODE)
    note(f"[full] {d.name}")
    S_ref = d.S0.numpy().astype(np.float64)
    state = d.S0.cuda()
    A = d.A.cuda()
    orc = oracle.load()
    worst = 0.0
    f = lambda t: t.float().numpy()
    for t in range(d.steps):
        o = kda.kda_decode_step(d.q[t].cuda(), d.k[t].cuda(), d.v[t].cuda(), d.beta[t].cuda(),
                                d.z[t].cuda(), A, state)
        o_ref = orc.decode_step(f(d.q[t]), f(d.k[t]), f(d.v[t]), f(d.beta[t]), d.z[t].numpy(),
                                d.A.numpy(), S_ref)
        worst = max(worst, max_abs(o.float().cpu().numpy(), o_ref))
    torch.cuda.synchronize()
    es = state_rel_err(state.cpu().numpy(), S_ref)
    note(f"    256 steps, {d.N * d.H} pairs: max|do| = {worst:.3e}  rel dS = {es:.3e}")
    assert worst <= OUT_TOL and es <= STATE_TOL
    assert worst <= 2e-3 and es <= 1e-4  # fp32 state; only q, k, v, o are bf16-rounded


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


# --- standalone kernels at the sizes bench.py times (inputs drawn on the host, seeded) ------

def _gate_tol(chunk):
    return chunk * float(np.spacing(np.float32(5.0 * chunk))) / 2 + chunk * 1e-5


def test_gate_b4_t32768_h32_sampled():
    """kda_gate with the chunk-local cumulative sum over 4 x 32768 tokens x 32 heads x 128
    channels (fp32), checked on whole sampled chunks: first and last of a sequence, across a
    sequence boundary, and inside."""
    N, T, H, dk = 4, 32768, 32, 128
    gen = torch.Generator().manual_seed(11)
    z = torch.randn(N * T, H, dk, generator=gen)
    A = torch.randn(H, dk, generator=gen) * 0.5
    note(f"[full] gate b4 t32768 h32 d128 f32")
    g, gc = kda.kda_gate(z.cuda(), A.cuda(), n_seqs=N)
    torch.cuda.synchronize()
    orc = oracle.load()
    worst_g = worst_c = 0.0
    for s in (0, T - 64, T, 2 * T + 640, N * T - 64):
        zs = z[s:s + 64].numpy()
        g_ref = orc.gate(zs, A.numpy())
        c_ref = orc.chunk_cumsum(g_ref, np.array([0, 64], dtype=np.int32), chunk=64)
        worst_g = max(worst_g, max_abs(g[s:s + 64].cpu().numpy(), g_ref))
        worst_c = max(worst_c, max_abs(gc[s:s + 64].cpu().numpy(), c_ref))
    note(f"    max|dg| = {worst_g:.2e}  max|dGamma| = {worst_c:.2e}")
    assert worst_g <= 1e-5 and worst_c <= _gate_tol(64)


def test_output_gate_rows4194304_sampled():
    """kda_output_gate over 4 x 32768 x 32 rows of d_v = 128 (bf16), sampled rows."""
    rows, dv = 4 * 32768 * 32, 128
    gen = torch.Generator().manual_seed(6)
    o = (torch.randn(rows, dv, generator=gen) * 0.05).to(torch.bfloat16)
    gate = torch.randn(rows, dv, generator=gen).to(torch.bfloat16)
    w = 1.0 + 0.1 * torch.randn(dv, generator=gen)
    note(f"[full] output gate rows={rows} dv={dv} bf16")
    y = kda.kda_output_gate(o.cuda(), gate.cuda(), w.cuda(), eps=1e-6)
    torch.cuda.synchronize()
    idx = np.concatenate([np.arange(1024), np.arange(rows - 1024, rows),
                          np.random.default_rng(8).integers(0, rows, 4096)])
    it = torch.from_numpy(idx)
    ref = oracle.load().output_gate(o[it].float().numpy(), gate[it].float().numpy(), w.numpy(), eps=1e-6)
    got = y[it.cuda()].float().cpu().numpy()
    d = np.abs(got - ref)
    note(f"    {len(idx)} rows: max|dy| = {d.max():.3e}")
    assert d.max() <= OUT_TOL
    assert np.all(d <= 2.0 ** -8 * np.abs(ref) + 1e-6)


def test_short_conv_b4_t32768_c4096_sampled():
    """kda_short_conv (width 4, per-head L2Norm over 128 channels, caches in and out) over
    4 x 32768 tokens x 4096 channels (bf16).  Checked: each sequence's first 16 tokens (their
    windows reach into the cache), 16-token runs inside, and every cache out exactly."""
    N, T, C, width = 4, 32768, 32 * 128, 4
    gen = torch.Generator().manual_seed(7)
    x = torch.randn(N * T, C, generator=gen).to(torch.bfloat16)
    w = torch.randn(C, width, generator=gen) * 0.5
    cache = torch.randn(N, C, width - 1, generator=gen).to(torch.bfloat16).float()
    note(f"[full] short conv b4 t32768 c4096 w4 bf16")
    co = torch.full((N, C, width - 1), float("nan"), device="cuda")
    y = kda.kda_short_conv(x.cuda(), w.cuda(), cache_in=cache.cuda(), cache_out=co, n_seqs=N,
                           l2_group=128)
    torch.cuda.synchronize()
    orc = oracle.load()
    worst = 0.0
    for n in range(N):
        s = n * T
        # the first 16 tokens, with this sequence's cache
        ref, _ = orc.short_conv(x[s:s + 16].float().numpy(), w.numpy(), cache[n:n + 1].numpy(),
                                cu_seqlens=np.array([0, 16], np.int32), l2_group=128)
        runs = [(s, ref)]
        # 16 tokens inside: the window of token t needs t-3 .. t, so the run starts 3 early
        t = s + 1000 + 7919 * n
        ref, _ = orc.short_conv(x[t - 3:t + 16].float().numpy(), w.numpy(), None,
                                cu_seqlens=np.array([0, 19], np.int32), l2_group=128)
        runs.append((t, ref[3:]))
        for t0, r in runs:
            got = y[t0:t0 + 16].float().cpu().numpy()
            d = np.abs(got - r)
            worst = max(worst, float(d.max()))
            assert np.all(d <= 2.0 ** -8 * np.abs(r) + 1e-5)
        # cache out: the sequence's last width - 1 inputs, channel-major
        want = x[s + T - (width - 1):s + T].float().numpy().T
        assert np.array_equal(co[n].cpu().numpy(), want)
    note(f"    max|dy| = {worst:.3e}")
    assert worst <= OUT_TOL
