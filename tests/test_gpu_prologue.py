"""GPU parity of the input prologue y = Swish(ShortConv(x)) (+ L2Norm per head) with the
short-convolution cache ([K3 note] §3.2), against the oracle.

Tolerance: max-abs 2e-2 (the output bound of the forward pass).  Guard: the kernel computes in
fp32 and rounds y once, so bf16 outputs are within one rounding of the exact value,
|dy| <= 2^-8 |y| + 1e-5 elementwise; fp32 outputs within 1e-5 (1 + |y|).  The cache holds the
raw inputs and must match exactly.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_chunkwise_amd import kda
from tests.gpu_util import OUT_TOL, note

pytestmark = pytest.mark.gpu


def _inputs(lengths, C, width, dtype, seed, with_cache=True):
    g = torch.Generator().manual_seed(seed)
    total = int(sum(lengths))
    x = torch.randn(total, C, generator=g).to(dtype)
    w = (torch.randn(C, width, generator=g) * 0.5).float()
    cache = (torch.randn(len(lengths), C, width - 1, generator=g)).to(dtype).float() if with_cache else None
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    return x, w, cache, cu


def _check(y, co, x, w, cache, cu, l2, dtype):
    y_ref, co_ref = oracle.load().short_conv(x.float().numpy(), w.numpy(),
                                             None if cache is None else cache.numpy(),
                                             cu_seqlens=cu.numpy(), l2_group=l2)
    got = y.float().cpu().numpy()
    d = np.abs(got - y_ref)
    assert d.max(initial=0.0) <= OUT_TOL
    if dtype == torch.bfloat16:
        assert np.all(d <= 2.0 ** -8 * np.abs(y_ref) + 1e-5)
    else:
        assert np.all(d <= 1e-5 * (1.0 + np.abs(y_ref)))
    if co is not None:
        assert np.array_equal(co.cpu().numpy(), co_ref.astype(np.float32))
    return d.max(initial=0.0)


# C = 2304: two 2048-channel workgroup blocks, the second one partial
@pytest.mark.parametrize("C,width,l2,dtype", [(256, 4, 128, torch.bfloat16), (192, 3, 64, torch.float32),
                                              (4096, 4, 128, torch.bfloat16), (128, 2, 0, torch.bfloat16),
                                              (64, 1, 64, torch.float32), (2304, 4, 128, torch.bfloat16)])
def test_short_conv_varlen_parity(C, width, l2, dtype):
    lengths = [0, 1, 2, 3, 31, 32, 33, 100, 0, 7]
    x, w, cache, cu = _inputs(lengths, C, width, dtype, seed=100 + C + width)
    co = torch.full((len(lengths), C, width - 1), float("nan")).cuda() if width > 1 else None
    y = kda.kda_short_conv(x.cuda(), w.cuda(), cache_in=None if cache is None else cache.cuda(),
                           cache_out=co, cu_seqlens=cu.cuda(), l2_group=l2)
    torch.cuda.synchronize()
    e = _check(y, co, x, w, cache, cu, l2, dtype)
    note(f"[short conv] C={C} width={width} l2={l2} {dtype}: max|dy| = {e:.3e}")


def test_short_conv_many_short_sequences():
    """1,100 sequences of 0-5 tokens at width 4: most windows reach into the cache, and the
    cache out of a sequence shorter than width - 1 keeps part of the cache in."""
    lengths = [int(x) for x in np.random.default_rng(12).integers(0, 6, 1100)]
    lengths[:6] = [0, 1, 2, 3, 4, 5]
    C, width, l2, dtype = 256, 4, 128, torch.bfloat16
    x, w, cache, cu = _inputs(lengths, C, width, dtype, seed=77)
    co = torch.full((len(lengths), C, width - 1), float("nan")).cuda()
    y = kda.kda_short_conv(x.cuda(), w.cuda(), cache_in=cache.cuda(), cache_out=co,
                           cu_seqlens=cu.cuda(), l2_group=l2)
    torch.cuda.synchronize()
    e = _check(y, co, x, w, cache, cu, l2, dtype)
    note(f"[short conv] 1,100 short sequences, {int(sum(lengths))} tokens: max|dy| = {e:.3e}")


def test_short_conv_equal_length_without_cache():
    x, w, _, cu = _inputs([70, 70, 70], 512, 4, torch.bfloat16, seed=7, with_cache=False)
    y = kda.kda_short_conv(x.cuda(), w.cuda(), n_seqs=3, l2_group=128)
    torch.cuda.synchronize()
    _check(y, None, x, w, None, cu, 128, torch.bfloat16)


def test_short_conv_decode_steps_match_prefill():
    """Decode: one token per sequence per call, the cache updated in place, reproduces the
    prefill over the same tokens exactly (same fp32 arithmetic per element)."""
    N, C, width, steps = 5, 256, 4, 6
    x, w, cache, _ = _inputs([steps] * N, C, width, torch.bfloat16, seed=11)
    xs = x.reshape(N, steps, C)
    cache_d = cache.clone().cuda()
    outs = []
    for t in range(steps):
        outs.append(kda.kda_short_conv(xs[:, t].contiguous().cuda(), w.cuda(), cache_in=cache_d,
                                       cache_out=cache_d, n_seqs=N, l2_group=128))
    y_dec = torch.stack(outs, 1).reshape(N * steps, C)
    co = torch.empty_like(cache_d)
    y_pre = kda.kda_short_conv(x.cuda(), w.cuda(), cache_in=cache.cuda(), cache_out=co, n_seqs=N,
                               l2_group=128)
    torch.cuda.synchronize()
    assert torch.equal(y_dec, y_pre)
    assert torch.equal(cache_d, co)
