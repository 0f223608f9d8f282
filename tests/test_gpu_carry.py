"""GPU parity where the carried state decides the outputs, on every state-pass form.

The cases (tests/carry_cases.py) use slow-decay gates with a unit-scale initial state, or
gates near the 16-token bound, and pair counts that make the library pick each form of the
state pass: the lagged 16-column kernel, and one, two or four compute waves per workgroup.
tests/test_carry_inputs.py shows on the CPU that, on these inputs, a dropped initial state
or a dropped chunk-to-chunk carry moves the outputs far beyond the tolerance.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from tests import carry_cases
from tests.gpu_util import (OUT_TOL, STATE_TOL, gpu_prefill, max_abs, note, oracle_prefill,
                            state_rel_err)

pytestmark = pytest.mark.gpu

# regression guard: bf16 operands round by 2^-9 relative; with a unit-scale state the outputs
# are sums of O(1) terms of size <= ~0.5
GUARD_OUT = 1e-2
GUARD_STATE = 5e-3


def _cus() -> int:
    return torch.cuda.get_device_properties(0).multi_processor_count


# every (form, d, dtype) that exists: the fused form (ncw 0) runs bf16 inputs only
_FORMS = [(ncw, d, dt) for ncw in (0, 1, 2, 4) for d, dt in ((128, "bf16"), (128, "fp32"), (64, "bf16"), (64, "fp32"))
          if ncw != 0 or dt == "bf16"]


@pytest.mark.parametrize("z_mean", [-4.0, -8.0, 6.0])
@pytest.mark.parametrize("ncw,d,dtype", _FORMS)
def test_prefill_carry_every_state_pass_form(ncw, d, dtype, z_mean):
    cus = _cus()
    inp = carry_cases.make_case(ncw, d, dtype, z_mean, cus)
    P = inp.N * inp.H
    form = carry_cases.form_name(P, d, dtype, cus)
    if ncw == 0:
        assert form == "fused"
    else:
        assert carry_cases.state_pass_waves(P, d, cus) == ncw and form != "fused"
    note(f"[carry] {inp.name}: {P} pairs on {cus} CUs -> {form}; lens {inp.lengths}")
    o, S = gpu_prefill(inp, use_cu=True)
    o_ref, S_ref = oracle_prefill(inp)
    e_o, e_s = max_abs(o, o_ref), state_rel_err(S, S_ref)
    note(f"    max|do| = {e_o:.3e}  max rel dS = {e_s:.3e}  max|o| = {np.abs(o_ref).max():.3f}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    assert e_o <= OUT_TOL and e_s <= STATE_TOL
    assert e_o <= GUARD_OUT and e_s <= GUARD_STATE
