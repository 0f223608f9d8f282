"""A seeded sweep of random prefill shapes over every form the library can pick, against the
oracle: random sequence counts, head counts (powers of two and not), ragged lengths with
empty and one-token sequences among them, equal-length batches, initial state present or
absent, final state requested or not, and gates from slow decay to the 16-token bound.

Each case names the form it is drawn for (the fused kernel, or the state pass with four,
two or one compute waves) and asserts that the library picks it on this device: the chain
count is chosen inside that form's band for the device's compute units.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from linear_attention_sequence_chunkwise_amd import workloads
from tests import carry_cases
from tests.gpu_util import OUT_TOL, STATE_TOL, gpu_prefill, max_abs, note, oracle_prefill, state_rel_err

pytestmark = pytest.mark.gpu

# (form, d, dtype): every form at both head sizes, both element types where they exist
COMBOS = [(f, d, dt) for f in ("fused", "waves4", "waves2", "one") for d in (128, 64)
          for dt in ("bf16", "fp32") if not (f == "fused" and dt == "fp32")]
CASES_PER_COMBO = 2


def _chain_band(form: str, d: int, cus: int):
    """[lo, hi] chain counts that select `form` (bf16 and fp32 alike below the fused form)."""
    if form == "fused":
        return cus, cus + cus // 4
    # four waves while chains x d/32 > cus, two while chains x d/16 > cus, else one
    four_lo = cus * 32 // d + 1
    two_lo = cus * 16 // d + 1
    if form == "waves4":
        return four_lo, min(cus - 1, four_lo + 40)
    if form == "waves2":
        return two_lo, four_lo - 1
    return 1, two_lo - 1


def _case(idx: int, cus: int):
    form, d, dtype = COMBOS[idx // CASES_PER_COMBO]
    rng = np.random.default_rng(5000 + idx)
    lo, hi = _chain_band(form, d, cus)
    target = int(rng.integers(lo, hi + 1))
    # a head count that divides a chain count inside the band
    heads = [h for h in (1, 2, 3, 4, 5, 6, 8, 12, 16, 24, 32, 48) if lo <= (target // h) * h <= hi and target // h >= 1]
    H = int(rng.choice(heads))
    N = target // H
    equal = bool(rng.random() < 0.3)
    budget = 40_000 if d == 128 else 90_000          # token-heads, to keep the oracle quick
    lmax = max(2, min(1200, budget // max(1, N * H)))
    if equal:
        lens = [int(rng.integers(1, lmax + 1))] * N
    else:
        lens = [int(x) for x in rng.integers(0, lmax + 1, N)]
        if N >= 5:  # the edge lengths, with real sequences beside them
            for j, edge in enumerate((0, 1, 64, 65)):
                if edge <= lmax:
                    lens[j] = edge
        lens[-1] = max(lens[-1], lmax // 2)  # never an all-empty batch
    z_mean = float(rng.choice([-8.0, -4.0, 0.0, 0.0, 3.0, 6.0]))
    s0 = None if rng.random() < 0.25 else (1.0 if z_mean < 0 else 0.02)
    with_state = bool(rng.random() < 0.8)
    inp = workloads.prefill_inputs(lens, H=H, dk=d, dv=d, dtype=dtype, seed=6000 + idx, z_mean=z_mean,
                                   s0_std=s0, name=f"sweep{idx}_{form}_d{d}_{dtype}",
                                   equal_length=equal)
    return form, inp, with_state


@pytest.mark.parametrize("idx", range(len(COMBOS) * CASES_PER_COMBO))
def test_prefill_sweep(idx):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    form, inp, with_state = _case(idx, cus)
    P = inp.N * inp.H
    got = carry_cases.form_name(P, inp.dk, inp.dtype, cus)
    want = {"fused": ["fused"], "waves4": ["waves4"], "waves2": ["waves2"],
            "one": ["lagged", "waves1"]}[form]
    note(f"[sweep] {inp.name}: N={inp.N} H={inp.H} P={P} -> {got}; lens {inp.lengths[:6]}"
         f"{'...' if inp.N > 6 else ''} equal={inp.equal_length} S0={inp.S0 is not None} "
         f"final={with_state} z_mean={inp.meta['z_mean']}")
    assert got in want
    o, S = gpu_prefill(inp, with_state=with_state)
    o_ref, S_ref = oracle_prefill(inp)
    e_o = max_abs(o, o_ref)
    assert np.all(np.isfinite(o))
    assert e_o <= OUT_TOL, f"max|do| = {e_o}"
    if with_state:
        e_s = state_rel_err(S, S_ref)
        assert np.all(np.isfinite(S))
        assert e_s <= STATE_TOL, f"max rel dS = {e_s}"
        note(f"    max|do| = {e_o:.3e}  max rel dS = {e_s:.3e}")
    else:
        note(f"    max|do| = {e_o:.3e}  (no final state)")
