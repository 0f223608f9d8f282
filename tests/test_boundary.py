"""CPU tests of the C ABI: the library loads, exports every symbol include/kda.h declares,
and rejects invalid arguments on the host before anything is launched (no GPU needed: every
call below fails validation, so no HIP call is made)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from linear_attention_sequence_chunkwise_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, ENULL, ESHAPE, EUNSUP, EALIGN, EWS, EHIP, ESCRATCH = 0, -1, -2, -3, -4, -5, -6, -7
F32, BF16 = 0, 1
P = ctypes.c_void_p(0x10000)   # aligned, never dereferenced: validation fails first
MIS = ctypes.c_void_p(0x10004)  # misaligned


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return kda.load_library()


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(kda.SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"libkda.so does not export {name}"


def test_status_strings(lib):
    for code in (OK, ENULL, ESHAPE, EUNSUP, EALIGN, EWS, EHIP, ESCRATCH):
        s = kda.status_str(code)
        assert s.startswith("KDA_"), s
    assert "unknown" in kda.status_str(42)


def prefill(lib, dt=BF16, q=P, k=P, v=P, beta=P, z=P, A=P, g_min=-5.0, s0=None, sN=None,
            cu=None, N=1, T=64, H=2, dk=128, dv=128, o=P, ws=None, wsb=0):
    return lib.kda_prefill_fwd(dt, q, k, v, beta, z, A, g_min, s0, sN, cu, N, T, H, dk, dv, o,
                               ws, wsb, None)


def test_prefill_rejects_bad_arguments(lib):
    assert prefill(lib, dt=7) == EUNSUP
    assert prefill(lib, A=None) == ENULL
    assert prefill(lib, T=0, q=None, k=None, v=None, beta=None, z=None, o=None) == OK
    for name in ("q", "k", "v", "beta", "z", "A", "o"):
        assert prefill(lib, **{name: None}) == ENULL, name
    assert prefill(lib, N=0) == ESHAPE
    assert prefill(lib, T=-1) == ESHAPE
    assert prefill(lib, H=0) == ESHAPE
    assert prefill(lib, dk=96, dv=96) == EUNSUP
    assert prefill(lib, dk=128, dv=64) == EUNSUP
    assert prefill(lib, g_min=-5.5) == EUNSUP      # outside the 16-token tile bound
    assert prefill(lib, g_min=0.0) == EUNSUP
    assert prefill(lib, g_min=float("nan")) == EUNSUP
    assert prefill(lib, q=MIS) == EALIGN
    assert prefill(lib, s0=MIS) == EALIGN
    assert prefill(lib, cu=ctypes.c_void_p(0x10002)) == EALIGN
    # a final state that partially overlaps the initial state
    assert prefill(lib, s0=ctypes.c_void_p(0x100000), sN=ctypes.c_void_p(0x100010)) == ESHAPE
    assert prefill(lib, T=1 << 45, N=1 << 10) == ESHAPE
    # (chunk slots) x heads intra-chunk workgroups must fit one 1-D grid
    assert prefill(lib, H=65535, T=64 * 40000) == ESHAPE


def test_noalloc_prefill_scratch_limit(lib):
    """The allocation-free prefill states its scratch limit in the header, rejects a call
    whose workspace would exceed it on the host (before any HIP call, so this runs without a
    GPU), and applies the ordinary argument checks first."""
    src = open(HEADER).read()
    m = re.search(r"#define KDA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == kda.NOALLOC_SCRATCH_BYTES
    assert kda.KDA_ERR_SCRATCH == ESCRATCH

    def call(T, H=16, dk=128, N=1, dt=BF16, A=P):
        return lib.kda_prefill_fwd_noalloc(dt, P, P, P, P, P, A, -5.0, None, None, None, N, T,
                                           H, dk, dk, P, None)

    # a 4096-token, 16-head d = 128 call fits; 512 more tokens do not
    fits = lib.kda_prefill_workspace_size(4096, 1, 16, 128, 128, BF16)
    assert fits <= kda.NOALLOC_SCRATCH_BYTES
    assert lib.kda_prefill_workspace_size(4096 + 512, 1, 16, 128, 128, BF16) > kda.NOALLOC_SCRATCH_BYTES
    assert call(4096 + 512) == ESCRATCH
    assert call(1 << 20, H=32) == ESCRATCH
    # ordinary checks come first
    assert call(64, dt=7) == EUNSUP
    assert call(64, A=None) == ENULL
    assert call(64, dk=96) == EUNSUP
    # nothing to compute and nothing to write: accepted without touching the device
    assert lib.kda_prefill_fwd_noalloc(BF16, None, None, None, None, None, P, -5.0, None, None,
                                       None, 1, 0, 2, 128, 128, None, None) == OK


def test_checkpointed_prefill_rejects_bad_arguments(lib):
    def ck(states=P, offs=None, interval=128, cu=None, T=256, ws=None, wsb=0):
        return lib.kda_prefill_fwd_checkpointed(BF16, P, P, P, P, P, P, -5.0, None, None, cu, 1, T,
                                                2, 128, 128, P, states, offs, interval, ws, wsb, None)
    assert ck(states=None) == ENULL
    assert ck(interval=0) == ESHAPE
    assert ck(interval=100) == ESHAPE                  # not a multiple of the 64-token chunk
    assert ck(interval=-64) == ESHAPE
    assert ck(cu=P, offs=None) == ENULL                # varlen needs the per-sequence offsets
    assert ck(states=MIS) == EALIGN
    assert ck(cu=P, offs=ctypes.c_void_p(0x10002)) == EALIGN
    assert ck() == EWS                                 # valid so far; no workspace given
    assert ck(T=0) == OK                               # nothing to compute


def test_gate_rejects_bad_arguments(lib):
    def gate(z=P, A=P, g=P, gc=P, T=64, H=2, dk=128, cu=None, N=1, chunk=64, g_min=-5.0):
        return lib.kda_gate(z, A, g, gc, T, H, dk, cu, N, chunk, g_min, None)
    assert gate(z=None) == ENULL
    assert gate(g=None, gc=None) == ENULL
    assert gate(T=-1) == ESHAPE
    assert gate(dk=6) == EUNSUP
    assert gate(chunk=0) == ESHAPE
    assert gate(chunk=4096) == ESHAPE
    assert gate(g_min=1.0) == EUNSUP
    assert gate(T=65, N=2) == ESHAPE
    assert gate(z=MIS) == EALIGN
    assert gate(T=0) == OK  # nothing to do, nothing launched
    assert gate(T=0, z=None, g=None, gc=None) == OK  # no tokens: per-token pointers unused
    assert gate(A=None) == ENULL
    # (token windows) x (column blocks) workgroups of 256 threads must fit one grid
    assert gate(T=1 << 25, chunk=1) == ESHAPE


def test_decode_rejects_bad_arguments(lib):
    def dec(dt=BF16, q=P, state=P, N=4, H=2, dk=128, dv=128, g_min=-5.0, o=P):
        return lib.kda_decode_step(dt, q, P, P, P, P, P, g_min, state, N, H, dk, dv, o, None)
    assert dec(q=None) == ENULL
    assert dec(state=None) == ENULL
    assert dec(N=-1) == ESHAPE
    assert dec(dk=32, dv=32) == EUNSUP
    assert dec(state=MIS) == EALIGN
    assert dec(dt=3) == EUNSUP
    assert dec(N=0) == OK
    assert dec(N=0, q=None, state=None, o=None) == OK


def test_verify_and_commit_reject_bad_arguments(lib):
    def ver(q=P, state=P, N=4, K=4, dk=128, dv=128, o=P):
        return lib.kda_decode_verify(BF16, q, P, P, P, P, P, -5.0, state, N, K, 2, dk, dv, o, None)
    def com(k=P, state=P, acc=P, N=4, K=4, dk=128, dv=128):
        return lib.kda_decode_commit(BF16, k, P, P, P, P, -5.0, state, N, K, 2, dk, dv, acc, None)
    assert ver(q=None) == ENULL and ver(state=None) == ENULL and ver(o=None) == ENULL
    assert ver(K=0) == ESHAPE and ver(K=17) == ESHAPE and ver(N=-1) == ESHAPE
    assert ver(dk=96, dv=96) == EUNSUP
    assert ver(state=MIS) == EALIGN
    assert ver(N=0) == OK
    assert com(k=None) == ENULL and com(acc=None) == ENULL
    assert com(K=0) == ESHAPE and com(K=17) == ESHAPE
    assert com(acc=ctypes.c_void_p(0x10002)) == EALIGN
    assert com(N=0) == OK


def test_output_gate_rejects_bad_arguments(lib):
    def og(dt=BF16, o=P, gate=P, w=P, eps=1e-6, rows=16, dv=128, y=P):
        return lib.kda_output_gate(dt, o, gate, w, eps, rows, dv, y, None)
    assert og(o=None) == ENULL and og(gate=None) == ENULL and og(y=None) == ENULL
    assert og(w=None) == ENULL
    assert og(rows=-1) == ESHAPE
    assert og(dv=96) == EUNSUP and og(dt=5) == EUNSUP
    assert og(eps=-1.0) == EUNSUP and og(eps=float("inf")) == EUNSUP
    assert og(o=MIS) == EALIGN
    assert og(rows=0, o=None, gate=None, y=None) == OK


def test_short_conv_rejects_bad_arguments(lib):
    def sc(dt=BF16, x=P, w=P, width=4, cin=None, cout=None, cu=None, N=1, T=64, C=256, l2=128, y=ctypes.c_void_p(0x20000)):
        return lib.kda_short_conv(dt, x, w, width, cin, cout, cu, N, T, C, l2, y, None)
    assert sc(x=None) == ENULL and sc(w=None) == ENULL and sc(y=None) == ENULL
    assert sc(width=0) == EUNSUP and sc(width=5) == EUNSUP
    assert sc(C=260) == EUNSUP                    # not a multiple of 8
    assert sc(l2=32) == EUNSUP and sc(C=192, l2=128) == EUNSUP
    assert sc(N=0) == ESHAPE and sc(T=-1) == ESHAPE
    assert sc(x=MIS) == EALIGN and sc(cu=ctypes.c_void_p(0x10002)) == EALIGN
    assert sc(y=P) == ESHAPE                      # y must not be x
    assert sc(T=0) == OK
    # (64-token segments) x (2048-channel blocks) workgroups of 256 threads must fit one grid
    assert sc(T=1 << 31, C=8, l2=0) == ESHAPE


def test_workspace_size_is_aligned(lib):
    for args in [(4096, 1, 16, 128, 128, BF16), (293000, 64, 32, 128, 128, BF16), (256, 1, 2, 64, 64, F32)]:
        assert lib.kda_prefill_workspace_size(*args) % 256 == 0


def test_workspace_size_follows_the_prefill_form(lib):
    """Without a device the library sizes for 256 compute units (MI355X's count).  bf16 with a
    (sequence, head) chain per compute unit takes the fused kernel, which keeps its factors on
    chip and needs only the n_seqs + 1 int32 chain-order table (rounded up to 256 bytes);
    fp32, or fewer chains, take the two-kernel form with one factor block per chunk and head
    (58.5 KiB at d = 128, 34.25 KiB at d = 64) after that table."""
    table = lambda n: ((n + 1) * 4 + 255) // 256 * 256
    block = {128: 59904, 64: 35072}
    split = lambda T, n, H, d: table(n) + (-(-T // 64) + n) * H * block[d]
    assert block[128] == 58.5 * 1024 and block[64] == 34.25 * 1024
    for T, n, H, d in [(293000, 64, 32, 128), (16384, 16, 16, 128), (4096, 256, 1, 64)]:
        assert n * H >= 256
        assert lib.kda_prefill_workspace_size(T, n, H, d, d, BF16) == table(n)
        assert lib.kda_prefill_workspace_size(T, n, H, d, d, F32) == split(T, n, H, d)
    # one chain short of the compute units: the two-kernel form
    assert lib.kda_prefill_workspace_size(16320, 15, 17, 128, 128, BF16) == split(16320, 15, 17, 128)
    # so a bf16 batch far beyond the scratch in the two-kernel form fits it when fused
    assert lib.kda_prefill_workspace_size(293000, 64, 32, 128, 128, F32) > kda.NOALLOC_SCRATCH_BYTES
    assert lib.kda_prefill_workspace_size(293000, 64, 32, 128, 128, BF16) <= kda.NOALLOC_SCRATCH_BYTES


def test_binding_fails_loudly_without_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    z = torch.zeros(4, 1, 4)
    with pytest.raises(Exception):
        kda.kda_gate(z, torch.zeros(1, 4))
