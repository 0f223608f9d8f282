"""GPU parity of prefix-cache checkpoints written by kda_prefill_fwd_checkpointed.

[K3 note] §9 and [K3 hood] "Serving two incompatible cache types": KDA keeps one recurrent
state per sequence, so checkpoints are taken only at sparse (512-token hash) boundaries; a
prefix hit restores the state at the boundary and resumes prefill from it.

Checked against the oracle: checkpoint j of a sequence must equal the final state of the same
prefill truncated after (j + 1) * interval tokens (the oracle runs the token recurrence on the
truncated sequences).  And resuming the HIP prefill from a checkpoint must reproduce the
remaining tokens' outputs of the uninterrupted run bit for bit (same chunk boundaries, same
kernels).  Tolerances as in test_gpu_parity: 1e-2 relative on states, guard 5e-3.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_chunkwise_amd import kda, workloads
from tests.gpu_util import STATE_TOL, dev, note, state_rel_err

pytestmark = pytest.mark.gpu
GUARD_STATE = 5e-3


def _truncated_reference(inp, interval):
    """Oracle states after every `interval` tokens of each sequence, in checkpoint order."""
    orc = oracle.load()
    cu = inp.cu_seqlens.numpy()
    f = lambda t: t.float().numpy()
    refs = []
    for n in range(inp.N):
        L = int(cu[n + 1] - cu[n])
        for j in range(L // interval):
            Lt = (j + 1) * interval
            sl = slice(int(cu[n]), int(cu[n]) + Lt)
            s0 = None if inp.S0 is None else inp.S0[n:n + 1].numpy()
            _, S = orc.prefill(f(inp.q[sl]), f(inp.k[sl]), f(inp.v[sl]), f(inp.beta[sl]),
                               z=inp.z[sl].numpy(), A=inp.A.numpy(), S0=s0,
                               cu_seqlens=np.array([0, Lt], dtype=np.int32))
            refs.append(S[0])
    return refs


def _run(inp, interval, use_cu):
    cu = inp.cu_seqlens.numpy()
    counts = [int(cu[n + 1] - cu[n]) // interval for n in range(inp.N)]
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    ck = torch.full((max(1, int(offs[-1])), inp.H, inp.dk, inp.dv), float("nan"), device="cuda")
    sN = torch.empty((inp.N, inp.H, inp.dk, inp.dv), device="cuda")
    o = kda.kda_prefill_fwd(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.beta), dev(inp.z),
                            dev(inp.A), initial_state=dev(inp.S0), final_state=sN,
                            cu_seqlens=dev(inp.cu_seqlens) if use_cu else None,
                            n_seqs=None if use_cu else inp.N, checkpoints=ck,
                            checkpoint_offsets=torch.from_numpy(offs).cuda() if use_cu else None,
                            checkpoint_interval=interval)
    torch.cuda.synchronize()
    return o, sN, ck, counts, offs


def _check(inp, interval, use_cu):
    note(f"[checkpoints] {inp.name} lens={inp.lengths[:8]}{'...' if inp.N > 8 else ''} "
         f"interval={interval} use_cu={use_cu}")
    o, sN, ck, counts, offs = _run(inp, interval, use_cu)
    refs = _truncated_reference(inp, interval)
    assert len(refs) == int(offs[-1])
    ck_np = ck.cpu().numpy().astype(np.float64)
    worst = 0.0
    for i, S_ref in enumerate(refs):
        e = state_rel_err(ck_np[i:i + 1], S_ref[None])
        worst = max(worst, e)
    note(f"    {len(refs)} checkpoints, max rel dS = {worst:.3e}")
    assert worst <= STATE_TOL and worst <= GUARD_STATE
    # a checkpoint on a sequence's last token is its final state, bit for bit
    cu = inp.cu_seqlens.numpy()
    sN_np = sN.cpu().numpy()
    for n in range(inp.N):
        L = int(cu[n + 1] - cu[n])
        if counts[n] and L % interval == 0:
            assert np.array_equal(ck_np[offs[n] + counts[n] - 1].astype(np.float32), sN_np[n])
    return o, ck


def test_checkpoints_batch_form():
    inp = workloads.prefill_inputs([320, 320], H=4, dk=128, dv=128, dtype="bf16", seed=31,
                                   s0_std=0.02, name="ck_batch")
    _check(inp, 128, use_cu=False)
    _check(inp, 64, use_cu=False)


def test_checkpoints_varlen_edge_lengths():
    # lengths below one interval (no checkpoint), exactly one interval (= final state),
    # ragged, and an empty sequence
    inp = workloads.prefill_inputs([100, 128, 0, 300, 512, 65], H=2, dk=128, dv=128,
                                   dtype="bf16", seed=32, s0_std=0.02, name="ck_varlen")
    _check(inp, 128, use_cu=True)


def test_checkpoints_many_sequences():
    """300 sequences of 0-200 tokens (600 bf16 chains: the fused kernel on a 256-CU GPU, with
    empty sequences among them), and most sequences hold zero to three checkpoints at their
    own offsets."""
    lens = [int(x) for x in np.random.default_rng(35).integers(0, 201, 300)]
    lens[:4] = [0, 64, 63, 128]
    inp = workloads.prefill_inputs(lens, H=2, dk=128, dv=128, dtype="bf16", seed=35,
                                   s0_std=0.02, name="ck_many")
    _check(inp, 64, use_cu=True)


def test_checkpoints_fused_d64():
    """300 sequences of 0-200 tokens at d = 64, one head (the fused kernel at d = 64)."""
    lens = [int(x) for x in np.random.default_rng(36).integers(0, 201, 300)]
    lens[:4] = [0, 64, 63, 128]
    inp = workloads.prefill_inputs(lens, H=1, dk=64, dv=64, dtype="bf16", seed=36,
                                   s0_std=0.02, name="ck_fused_d64")
    _check(inp, 64, use_cu=True)


def test_checkpoints_fused_batch_form():
    """Eight equal sequences of 320 tokens at 32 heads: 256 chains, the fused kernel given
    n_seqs and no cu_seqlens, so each sequence's checkpoints start at n * (320 // interval)."""
    inp = workloads.prefill_inputs([320] * 8, H=32, dk=128, dv=128, dtype="bf16", seed=37,
                                   s0_std=0.02, name="ck_fused_batch")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if inp.N * inp.H < cus:
        pytest.skip(f"{inp.N * inp.H} chains do not reach the fused form on {cus} CUs")
    _check(inp, 128, use_cu=False)


def test_checkpoints_d64_fp32():
    inp = workloads.prefill_inputs([200, 256], H=3, dk=64, dv=64, dtype="fp32", seed=33,
                                   s0_std=0.02, name="ck_d64_fp32")
    _check(inp, 64, use_cu=True)


def test_resume_from_checkpoint_reproduces_outputs():
    """Prefix hit: restore checkpoint j as the initial state and prefill the remaining tokens;
    their outputs and the final state must equal the uninterrupted run exactly."""
    interval = 128
    inp = workloads.prefill_inputs([384, 448], H=4, dk=128, dv=128, dtype="bf16", seed=34,
                                   s0_std=0.02, name="ck_resume")
    o_full, ck = _check(inp, interval, use_cu=True)
    sN_full = torch.empty((inp.N, inp.H, inp.dk, inp.dv), device="cuda")
    kda.kda_prefill_fwd(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.beta), dev(inp.z),
                        dev(inp.A), initial_state=dev(inp.S0), final_state=sN_full,
                        cu_seqlens=dev(inp.cu_seqlens))
    cu = inp.cu_seqlens.numpy()
    # resume both sequences at their second checkpoint (256 tokens in)
    j = 1
    cut = (j + 1) * interval
    counts = [int(cu[n + 1] - cu[n]) // interval for n in range(inp.N)]
    offs = np.concatenate([[0], np.cumsum(counts)])
    s0 = torch.stack([ck[int(offs[n]) + j] for n in range(inp.N)]).contiguous()
    idx = np.concatenate([np.arange(cu[n] + cut, cu[n + 1]) for n in range(inp.N)])
    rest_lens = [int(cu[n + 1] - cu[n]) - cut for n in range(inp.N)]
    rest_cu = torch.tensor(np.concatenate([[0], np.cumsum(rest_lens)]), dtype=torch.int32)
    t = lambda x: x[torch.from_numpy(idx)].contiguous().cuda()
    sN = torch.empty_like(s0)
    o_rest = kda.kda_prefill_fwd(t(inp.q), t(inp.k), t(inp.v), t(inp.beta), t(inp.z), dev(inp.A),
                                 initial_state=s0, final_state=sN, cu_seqlens=rest_cu.cuda())
    torch.cuda.synchronize()
    assert torch.equal(o_rest, o_full[torch.from_numpy(idx).cuda()])
    assert torch.equal(sN, sN_full)
