"""GPU parity of the fused output epilogue y = Sigmoid(gate) * RMSNorm(o)
([K3 note] §3.2, the K3 output path before W_o) against the oracle.

Tolerance: max-abs 2e-2 (the output bound of the forward pass).  Guard: the kernel computes
in fp32 and rounds y once to the element type, so every bf16 output is within one rounding
(2^-9 |y|, round to nearest even) plus fp32 arithmetic error of the exact value: |dy| <=
2^-8 |y| + 1e-6 elementwise; fp32 outputs agree to 1e-5.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_chunkwise_amd import kda
from tests.gpu_util import OUT_TOL, max_abs, note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dv,dtype,rows", [(128, torch.bfloat16, 4096 * 3 + 5), (64, torch.bfloat16, 77),
                                           (128, torch.float32, 1000), (64, torch.float32, 1)])
def test_output_gate_parity(dv, dtype, rows):
    g = torch.Generator().manual_seed(90 + dv + rows)
    o = (torch.randn(rows, dv, generator=g) * 0.05).to(dtype)
    gate = torch.randn(rows, dv, generator=g).to(dtype)
    w = (1.0 + 0.1 * torch.randn(dv, generator=g)).float()
    y = kda.kda_output_gate(o.cuda(), gate.cuda(), w.cuda(), eps=1e-6)
    torch.cuda.synchronize()
    ref = oracle.load().output_gate(o.float().numpy(), gate.float().numpy(), w.numpy(), eps=1e-6)
    e = max_abs(y.float().cpu().numpy(), ref)
    note(f"[output gate] dv={dv} {dtype} rows={rows}: max|dy| = {e:.3e}")
    assert e <= OUT_TOL
    if dtype == torch.bfloat16:
        assert np.all(np.abs(y.float().cpu().numpy() - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)
    else:
        assert e <= 1e-5


def test_output_gate_in_place_on_prefill_layout():
    """y may overwrite o; a [tokens, H, dv] readout is rows = tokens * H."""
    T, H, dv = 300, 4, 128
    g = torch.Generator().manual_seed(99)
    o = (torch.randn(T, H, dv, generator=g) * 0.1).to(torch.bfloat16).cuda()
    gate = torch.randn(T, H, dv, generator=g).to(torch.bfloat16).cuda()
    w = torch.ones(dv).cuda()
    ref = oracle.load().output_gate(o.float().cpu().numpy(), gate.float().cpu().numpy(),
                                    w.cpu().numpy(), eps=1e-6)
    kda.kda_output_gate(o, gate, w, eps=1e-6, y=o)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy()
    assert max_abs(got, ref) <= OUT_TOL
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)
