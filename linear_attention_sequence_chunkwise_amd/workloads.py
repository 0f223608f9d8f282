"""Seeded synthetic inputs for the KDA forward pass.

This module only draws random numbers and shapes them; it holds none of the method's
arithmetic (no gate, no decay, no recurrence).  Both the HIP path's tests/benchmark and the
CPU oracle consume what it produces, so the two sides see bit-identical inputs.

Recipe (numpy PCG64 ``default_rng(seed)``, float32 draws, fixed draw order):
  lengths (varlen only) -> q -> k -> v -> beta -> z -> A -> S0
  Each tensor after the lengths is cut, along its leading axes, into blocks of about 4M
  elements; block b is drawn from the b-th PCG64 stream spawned from the generator (streams
  spawned in draw order), so the values do not depend on how many host threads draw them.
  * q, k ~ N(0, 1), each (token, head) vector L2-normalised over d_k in fp32; q then scaled
    by 1/sqrt(d_k).  (The KDA input branch normalises q and k per head; the scale is the
    usual attention scale, applied here because o = S^T q carries none.)
  * v ~ N(0, 1);  beta = Sigmoid(N(0, 1)) per (token, head)
  * z ~ N(z_mean, z_std) per (token, head, key channel), fp32
  * A ~ N(0, 0.5) per (head, key channel), fp32
  * S0 ~ N(0, s0_std) fp32 [N, H, d_k, d_v] when s0_std is given, else no initial state
  * bf16 inputs are rounded from the fp32 draws with round-to-nearest-even (torch CPU).
  Varlen lengths: L = round(exp(U(ln lo, ln hi))) per sequence, not rescaled.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional

import numpy as np
import torch

_DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


_BLOCK_ELEMS = 1 << 22   # elements per independently seeded block (fixed: part of the recipe)
_pool: Optional[ThreadPoolExecutor] = None


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal(rng: np.random.Generator, shape, mean: float = 0.0, std: float = 1.0,
            post: Optional[Callable[[np.ndarray], np.ndarray]] = None) -> np.ndarray:
    """float32 N(mean, std) draws of `shape`, block by block (see the recipe); `post` maps
    each block of whole last-axis rows (applied after the scale and shift)."""
    shape = tuple(int(x) for x in shape)
    last = shape[-1]
    rows = int(np.prod(shape[:-1], dtype=np.int64)) if len(shape) > 1 else 1
    out = np.empty((rows, last), dtype=np.float32)
    brows = max(1, _BLOCK_ELEMS // max(last, 1))
    nblk = max(1, -(-rows // brows))
    streams = rng.spawn(nblk)

    def fill(b):
        r0, r1 = b * brows, min(rows, (b + 1) * brows)
        if r1 <= r0:
            return
        x = streams[b].standard_normal(size=(r1 - r0, last), dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        if mean != 0.0:
            x += np.float32(mean)
        out[r0:r1] = post(x) if post is not None else x

    global _pool
    if nblk == 1:
        fill(0)
    else:
        if _pool is None:
            _pool = ThreadPoolExecutor(max_workers=_threads())
        list(_pool.map(fill, range(nblk)))
    return out.reshape(shape)


def _l2norm_lastdim(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.einsum("...d,...d->...", x, x, dtype=np.float32))
    n = np.maximum(n, np.float32(1e-12))
    return x / n[..., None]


def _l2norm_scaled(scale: float):
    s = np.float32(scale)
    return lambda x: _l2norm_lastdim(x) * s


def _sigmoid_f32(x: np.ndarray) -> np.ndarray:
    return (np.float32(1.0) / (np.float32(1.0) + np.exp(-x))).astype(np.float32)


def _to(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(_DT[dtype])


@dataclass
class PrefillInputs:
    """Packed prefill batch: q,k,z [total,H,dk]; v [total,H,dv]; beta [total,H]; A [H,dk];
    S0 [N,H,dk,dv] or None; cu_seqlens [N+1] int32 (always filled, also for equal lengths)."""
    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    beta: torch.Tensor
    z: torch.Tensor
    A: torch.Tensor
    S0: Optional[torch.Tensor]
    cu_seqlens: torch.Tensor
    lengths: List[int]
    equal_length: bool
    dtype: str
    meta: Dict = field(default_factory=dict)

    @property
    def total(self) -> int:
        return int(self.q.shape[0])

    @property
    def H(self) -> int:
        return int(self.q.shape[1])

    @property
    def dk(self) -> int:
        return int(self.q.shape[2])

    @property
    def dv(self) -> int:
        return int(self.v.shape[2])

    @property
    def N(self) -> int:
        return len(self.lengths)

    def pair_slice(self, n: int, h: int):
        """fp32 numpy views of one (sequence, head) pair, shaped for the oracle with H=1."""
        s, e = int(self.cu_seqlens[n]), int(self.cu_seqlens[n + 1])
        f = lambda t: t[s:e, h:h + 1].float().numpy()
        out = dict(q=f(self.q), k=f(self.k), v=f(self.v),
                   beta=self.beta[s:e, h:h + 1].float().numpy(),
                   z=self.z[s:e, h:h + 1].numpy(), A=self.A[h:h + 1].numpy())
        out["S0"] = None if self.S0 is None else self.S0[n:n + 1, h:h + 1].numpy()
        return out


def prefill_inputs(lengths: List[int], H: int, dk: int, dv: int, dtype: str, seed: int,
                   z_mean: float = 0.0, z_std: float = 1.0, s0_std: Optional[float] = None,
                   name: str = "custom", equal_length: Optional[bool] = None,
                   rng: Optional[np.random.Generator] = None) -> PrefillInputs:
    rng = rng if rng is not None else np.random.default_rng(seed)
    total = int(sum(lengths))
    q = _normal(rng, (total, H, dk), post=_l2norm_scaled(1.0 / math.sqrt(dk)))
    k = _normal(rng, (total, H, dk), post=_l2norm_lastdim)
    v = _normal(rng, (total, H, dv))
    beta = _normal(rng, (total, H), post=_sigmoid_f32)
    z = _normal(rng, (total, H, dk), z_mean, z_std)
    A = _normal(rng, (H, dk), 0.0, 0.5)
    S0 = _normal(rng, (len(lengths), H, dk, dv), 0.0, s0_std) if s0_std is not None else None
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    if equal_length is None:
        equal_length = len(set(lengths)) <= 1
    return PrefillInputs(
        name=name, q=_to(q, dtype), k=_to(k, dtype), v=_to(v, dtype), beta=_to(beta, dtype),
        z=torch.from_numpy(z), A=torch.from_numpy(A),
        S0=None if S0 is None else torch.from_numpy(S0),
        cu_seqlens=torch.from_numpy(cu), lengths=[int(x) for x in lengths],
        equal_length=bool(equal_length), dtype=dtype,
        meta=dict(seed=seed, z_mean=z_mean, z_std=z_std, s0_std=s0_std))


def varlen_lengths(rng: np.random.Generator, n: int, lo: int, hi: int) -> List[int]:
    u = rng.uniform(math.log(lo), math.log(hi), size=n)
    return [int(x) for x in np.rint(np.exp(u))]


@dataclass
class DecodeInputs:
    """`steps` consecutive single-token decode steps: q,k,z [steps,N,H,dk]; v [steps,N,H,dv];
    beta [steps,N,H]; A [H,dk]; S0 [N,H,dk,dv] fp32."""
    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    beta: torch.Tensor
    z: torch.Tensor
    A: torch.Tensor
    S0: torch.Tensor
    dtype: str
    meta: Dict = field(default_factory=dict)

    @property
    def steps(self) -> int:
        return int(self.q.shape[0])

    @property
    def N(self) -> int:
        return int(self.q.shape[1])

    @property
    def H(self) -> int:
        return int(self.q.shape[2])

    @property
    def dk(self) -> int:
        return int(self.q.shape[3])

    @property
    def dv(self) -> int:
        return int(self.v.shape[3])


def decode_inputs(N: int, H: int, dk: int, dv: int, steps: int, dtype: str, seed: int,
                  z_mean: float = 0.0, z_std: float = 1.0, s0_std: float = 0.02,
                  name: str = "custom") -> DecodeInputs:
    """Draw order: q, k, v, beta, z (all steps at once), A, S0."""
    rng = np.random.default_rng(seed)
    q = _normal(rng, (steps, N, H, dk), post=_l2norm_scaled(1.0 / math.sqrt(dk)))
    k = _normal(rng, (steps, N, H, dk), post=_l2norm_lastdim)
    v = _normal(rng, (steps, N, H, dv))
    beta = _normal(rng, (steps, N, H), post=_sigmoid_f32)
    z = _normal(rng, (steps, N, H, dk), z_mean, z_std)
    A = _normal(rng, (H, dk), 0.0, 0.5)
    S0 = _normal(rng, (N, H, dk, dv), 0.0, s0_std)
    return DecodeInputs(name=name, q=_to(q, dtype), k=_to(k, dtype), v=_to(v, dtype),
                        beta=_to(beta, dtype), z=torch.from_numpy(z), A=torch.from_numpy(A),
                        S0=torch.from_numpy(S0), dtype=dtype,
                        meta=dict(seed=seed, z_mean=z_mean, z_std=z_std, s0_std=s0_std))


# --- the five named workloads ------------------------------------------------------------
# Names state what each workload is; seeds are fixed per workload.

PREFILL_TINY = "prefill_b1_h2_t256_d64_fp32"
PREFILL_B1 = "prefill_b1_h16_t4096_d128_bf16"
PREFILL_B4 = "prefill_b4_h32_t32768_d128_bf16"
PREFILL_VARLEN = "prefill_varlen64_h32_d128_bf16_s0"
DECODE = "decode_n512_h32_d128_bf16_256steps"

WORKLOADS = (PREFILL_TINY, PREFILL_B1, PREFILL_B4, PREFILL_VARLEN, DECODE)


def make(name: str, **overrides):
    """Build one of the named workloads (``overrides`` only for reduced test variants)."""
    if name == PREFILL_TINY:
        kw = dict(lengths=[256], H=2, dk=64, dv=64, dtype="fp32", seed=0)
    elif name == PREFILL_B1:
        kw = dict(lengths=[4096], H=16, dk=128, dv=128, dtype="bf16", seed=1)
    elif name == PREFILL_B4:
        kw = dict(lengths=[32768] * 4, H=32, dk=128, dv=128, dtype="bf16", seed=2)
    elif name == PREFILL_VARLEN:
        rng = np.random.default_rng(3)
        lens = varlen_lengths(rng, 64, 512, 16384)
        kw = dict(lengths=lens, H=32, dk=128, dv=128, dtype="bf16", seed=3, s0_std=0.02,
                  rng=rng, equal_length=False)
    elif name == DECODE:
        kw = dict(N=512, H=32, dk=128, dv=128, steps=256, dtype="bf16", seed=4)
        kw.update(overrides)
        return decode_inputs(name=name, **kw)
    else:
        raise KeyError(f"unknown workload {name!r}; known: {WORKLOADS}")
    kw.update(overrides)
    return prefill_inputs(name=name, **kw)
