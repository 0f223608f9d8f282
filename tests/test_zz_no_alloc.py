"""kda_prefill_fwd_noalloc -- the prefill with its workspace in the library's static
per-device scratch array, for callers that cannot allocate -- against kda_prefill_fwd with a
caller workspace.  Both run the same kernels on the same inputs, so outputs and final states
must agree bit for bit.  The calls come in a row on one device, each smaller than the one
before, so every later call runs on scratch that still holds the previous call's contents."""
from __future__ import annotations

import pytest
import torch

from linear_attention_sequence_chunkwise_amd import kda, workloads
from tests.gpu_util import note

pytestmark = pytest.mark.gpu


def _compare(inp):
    c = lambda t: None if t is None else t.cuda()
    q, k, v, beta, z, A = map(c, (inp.q, inp.k, inp.v, inp.beta, inp.z, inp.A))
    s0 = c(inp.S0)
    cu = None if inp.equal_length else c(inp.cu_seqlens)
    n = None if cu is not None else inp.N
    shape = (inp.N, inp.H, inp.dk, inp.dv)
    need = kda.kda_prefill_workspace_size(inp.total, inp.N, inp.H, inp.dk, inp.dv, q.dtype)
    note(f"[noalloc] {inp.name}: {inp.total} tokens, H={inp.H}, d={inp.dk}, {inp.dtype}, "
         f"workspace {need} of {kda.NOALLOC_SCRATCH_BYTES} bytes")
    assert need <= kda.NOALLOC_SCRATCH_BYTES
    if inp.dtype == "bf16" and inp.N * inp.H >= 256:
        assert need == (inp.N + 1 + 63) // 64 * 256, "the fused form needs only the chain-order table"
    s_ref = torch.empty(shape, dtype=torch.float32, device="cuda")
    o_ref = kda.kda_prefill_fwd(q, k, v, beta, z, A, initial_state=s0, final_state=s_ref,
                                cu_seqlens=cu, n_seqs=n)
    s_na = torch.full(shape, float("nan"), device="cuda")
    o_na = torch.full_like(o_ref, float("nan"))
    kda.kda_prefill_fwd_noalloc(q, k, v, beta, z, A, initial_state=s0, final_state=s_na,
                                cu_seqlens=cu, n_seqs=n, o=o_na)
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ref), "outputs differ from the caller-workspace entry point"
    assert torch.equal(s_na, s_ref), "final states differ from the caller-workspace entry point"


def test_noalloc_equals_workspace_entry_on_calls_in_a_row():
    # 16 sequences x 16 heads: a chain per compute unit of MI355X (256), so the fused kernel,
    # whose scratch is the chain-order table alone (the two-kernel form would need about
    # 250 MB here, beyond the scratch)
    assert torch.cuda.get_device_properties(0).multi_processor_count <= 256
    calls = [
        workloads.prefill_inputs([1500, 700, 1024, 64, 2100, 999, 1, 1200, 640, 1024, 333,
                                  1777, 900, 1030, 2000, 1000], H=16, dk=128, dv=128,
                                 dtype="bf16", seed=60, s0_std=0.2, name="noalloc_fused_varlen"),
        # the largest named single-GPU prefill that fits the scratch: one 4096-token sequence
        workloads.make(workloads.PREFILL_B1),
        # varlen with slow decay and initial states
        workloads.prefill_inputs([300, 1000, 64, 77, 513], H=8, dk=128, dv=128, dtype="bf16",
                                 seed=61, z_mean=-4.0, s0_std=0.5, name="noalloc_varlen"),
        # smaller, other kernels (fp32 inputs, d = 64), equal lengths
        workloads.prefill_inputs([130, 130], H=4, dk=64, dv=64, dtype="fp32", seed=62,
                                 s0_std=0.02, name="noalloc_b2_d64_fp32"),
        # smaller still
        workloads.prefill_inputs([70, 0, 5], H=2, dk=128, dv=128, dtype="bf16", seed=63,
                                 s0_std=0.02, name="noalloc_small"),
    ]
    for inp in calls:
        _compare(inp)


def test_noalloc_rejects_a_call_beyond_the_scratch():
    inp = workloads.prefill_inputs([4096 + 512], H=16, dk=128, dv=128, dtype="bf16", seed=64,
                                   name="noalloc_too_large")
    c = lambda t: t.cuda()
    o = torch.zeros((inp.total, inp.H, inp.dv), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kda.KDAError) as err:
        kda.kda_prefill_fwd_noalloc(c(inp.q), c(inp.k), c(inp.v), c(inp.beta), c(inp.z),
                                    c(inp.A), o=o)
    assert err.value.code == kda.KDA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert not o.any(), "a rejected call wrote its output"
