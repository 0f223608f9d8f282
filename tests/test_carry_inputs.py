"""CPU checks that the state-carry parity cases (tests/carry_cases.py) can fail: on their
inputs, the oracle's outputs and final states move far beyond the tolerances when the
initial state is dropped or when the state is not carried from one 64-token chunk to the
next.  A GPU path with either mistake would therefore fail those parity tests."""
from __future__ import annotations

import numpy as np
import pytest

from tests import carry_cases
from tests.gpu_util import OUT_TOL, STATE_TOL, state_rel_err


def _chunked_restart(orc, inp):
    """The oracle on every 64-token chunk as a sequence of its own: the first chunk of each
    sequence starts from the initial state, every later chunk from zero (carry dropped)."""
    f = lambda t: t.float().numpy()
    cu = inp.cu_seqlens.numpy()
    starts, owner = [], []
    for n in range(inp.N):
        for s in range(int(cu[n]), int(cu[n + 1]), 64):
            starts.append(s)
            owner.append(n if s == cu[n] else -1)
    cu_c = np.array(starts + [inp.total], np.int32)
    S0 = np.zeros((len(starts), inp.H, inp.dk, inp.dv), np.float32)
    for i, n in enumerate(owner):
        if n >= 0:
            S0[i] = inp.S0[n].numpy()
    o, _ = orc.prefill(f(inp.q), f(inp.k), f(inp.v), f(inp.beta), z=inp.z.numpy(),
                       A=inp.A.numpy(), S0=S0, cu_seqlens=cu_c)
    return o


@pytest.mark.parametrize("d,ncw,z_mean", [(128, 1, -4.0), (128, 1, -8.0), (64, 2, -4.0)])
def test_carry_cases_expose_dropped_state(oracle_lib, d, ncw, z_mean):
    inp = carry_cases.make_case(ncw, d, "bf16", z_mean, cus=256)
    f = lambda t: t.float().numpy()
    args = (f(inp.q), f(inp.k), f(inp.v), f(inp.beta))
    kw = dict(z=inp.z.numpy(), A=inp.A.numpy(), cu_seqlens=inp.cu_seqlens.numpy())
    o, S = oracle_lib.prefill(*args, S0=inp.S0.numpy(), **kw)
    o_nos0, S_nos0 = oracle_lib.prefill(*args, S0=None, **kw)
    o_nocarry = _chunked_restart(oracle_lib, inp)
    d_s0 = float(np.abs(o - o_nos0).max())
    d_s0_state = state_rel_err(S_nos0, S)
    d_carry = float(np.abs(o - o_nocarry).max())
    # outputs past the first chunk of each sequence: only the carry reaches them
    cu = inp.cu_seqlens.numpy()
    late = np.concatenate([np.arange(cu[n] + 64, cu[n + 1]) for n in range(inp.N)])
    d_s0_late = float(np.abs(o[late] - o_nos0[late]).max())
    print(f"{inp.name}: no S0 max|do| {d_s0:.3f} (after chunk 0: {d_s0_late:.3f}), "
          f"rel dS {d_s0_state:.3f}; no carry max|do| {d_carry:.3f}")
    assert d_s0 > 10 * OUT_TOL and d_s0_late > 4 * OUT_TOL
    assert d_s0_state > 10 * STATE_TOL
    assert d_carry > 4 * OUT_TOL


def test_carry_cases_land_on_every_form():
    """With 256 compute units, the case shapes select the form they name."""
    for d in (64, 128):
        for ncw in (1, 2, 4):
            lens, H = carry_cases.case_shape(ncw, d, 256)
            P = len(lens) * H
            assert carry_cases.state_pass_waves(P, d, 256) == ncw, (d, ncw, P)
            assert carry_cases.form_name(P, d, "bf16", 256) == ("lagged" if ncw == 1 else f"waves{ncw}")
        lens, H = carry_cases.case_shape(0, d, 256)
        assert carry_cases.form_name(len(lens) * H, d, "bf16", 256) == "fused"
        assert carry_cases.form_name(len(lens) * H, d, "fp32", 256) == "waves4"
    assert carry_cases.form_name(32, 128, "fp32", 256) == "waves1"
