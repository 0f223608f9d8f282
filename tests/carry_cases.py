"""Prefill cases in which the state carried between chunks, and the initial state, decide the
outputs -- one for every state-pass form the library can pick.

At the named workloads' gates (z ~ N(0, 1), so g averages about -2.5) every 64-token chunk
decays the state by e^-100 or more in every key channel, so a dropped carry or a wrong
initial-state load stays far below the output tolerance.  These cases shift the gate:
  * z ~ N(-4, 1) or N(-8, 1): slow decay (g about -0.26 or less); many channels keep their
    state over dozens of chunks, and an initial state of unit scale dominates early outputs;
  * z ~ N(+6, 1): decay near the floor, 16-token sums near the -80 bound ("Kimi K3:
    Architecture, Training, and Million-Token Agentic RL" §3.3).

The state pass runs one workgroup per (sequence, head, dv slice) with 1, 2 or 4 compute
waves of 16 dv columns; the library halves the waves while the (sequence, head) pairs times
slices still fit the compute units.  The rule, for dk = dv = d and P pairs on a device with
U compute units: four waves if P * d / 32 > U, else two if P * d / 16 > U, else one.  With
one wave, bf16 inputs (and every d = 64 call) take the lagged two-wave form.  With bf16
inputs and P >= U, the fused single-kernel prefill runs instead (one workgroup per pair).
Each case's pair count is derived from U so that it lands on the form it names (ncw = 0
names the fused form).
"""
from __future__ import annotations

from typing import List, Tuple

from linear_attention_sequence_chunkwise_amd import workloads

# cycled sequence lengths: several chunks each, ragged tails, one long chain (1,000 tokens)
LENGTHS = [581, 300, 1000, 129, 64, 777, 450, 2, 333, 700]


def state_pass_waves(pairs: int, d: int, cus: int) -> int:
    ncw = 4
    while ncw > 1 and pairs * (d // (8 * ncw)) <= cus:
        ncw //= 2
    return ncw


def uses_fused(pairs: int, dtype: str, cus: int) -> bool:
    return dtype == "bf16" and pairs >= cus


def form_name(pairs: int, d: int, dtype: str, cus: int) -> str:
    if uses_fused(pairs, dtype, cus):
        return "fused"
    ncw = state_pass_waves(pairs, d, cus)
    if ncw == 1 and (dtype == "bf16" or d == 64):
        return "lagged"
    return f"waves{ncw}"


def pairs_for(ncw: int, d: int, cus: int) -> int:
    """A pair count that selects `ncw` compute waves (0: the fused form, bf16 only): just
    inside each band."""
    if ncw == 0:
        return cus
    if ncw == 1:
        return cus * 16 // d
    if ncw == 2:
        return cus * 24 // d
    return cus * 40 // d


def case_shape(ncw: int, d: int, cus: int) -> Tuple[List[int], int]:
    """(lengths, H) with len(lengths) * H == pairs_for(ncw, d, cus)."""
    P = pairs_for(ncw, d, cus)
    H = 16 if P % 16 == 0 else 8 if P % 8 == 0 else 1
    if ncw == 0:
        H = 32 if P % 32 == 0 else H   # shorter chains for the oracle
    N = P // H
    return [LENGTHS[i % len(LENGTHS)] for i in range(N)], H


def make_case(ncw: int, d: int, dtype: str, z_mean: float, cus: int, seed: int = 900):
    lens, H = case_shape(ncw, d, cus)
    s0 = 1.0 if z_mean < 0 else 0.02   # slow decay: the initial state dominates
    return workloads.prefill_inputs(lens, H=H, dk=d, dv=d, dtype=dtype,
                                    seed=seed + 10 * ncw + d + (0 if dtype == "bf16" else 1),
                                    z_mean=z_mean, s0_std=s0,
                                    name=f"carry_w{ncw}_d{d}_{dtype}_z{z_mean:+g}")
