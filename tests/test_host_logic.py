"""CPU tests of the host-side logic around the kernels: the seeded input recipe, the
roofline accounting that bench.py reports, and the readers of the rocprofv3 summaries under
profiles/ (which must drop a summary taken for other kernel sources)."""
from __future__ import annotations

import math
import os
import re
import shutil

import numpy as np
import pytest
import torch

import bench
from linear_attention_sequence_chunkwise_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# --- input recipe ------------------------------------------------------------------------

def test_prefill_inputs_follow_the_recipe():
    inp = workloads.prefill_inputs([70, 0, 130], H=3, dk=64, dv=32, dtype="fp32", seed=9,
                                   s0_std=0.02)
    assert inp.total == 200 and inp.N == 3 and inp.H == 3
    assert inp.cu_seqlens.tolist() == [0, 70, 70, 200]
    # q, k L2-normalised per (token, head); q then carries 1/sqrt(dk)
    kn = np.linalg.norm(inp.k.numpy(), axis=-1)
    qn = np.linalg.norm(inp.q.numpy(), axis=-1)
    assert np.allclose(kn, 1.0, atol=1e-5)
    assert np.allclose(qn, 1.0 / math.sqrt(64), atol=1e-5)
    b = inp.beta.numpy()
    assert b.shape == (200, 3) and np.all((b > 0) & (b < 1))
    assert inp.z.dtype == torch.float32 and inp.A.shape == (3, 64)
    assert inp.S0.shape == (3, 3, 64, 32) and abs(float(inp.S0.std()) - 0.02) < 2e-3
    assert not inp.equal_length


def test_inputs_are_reproducible_and_seed_dependent():
    a = workloads.prefill_inputs([64], H=2, dk=64, dv=64, dtype="bf16", seed=5)
    b = workloads.prefill_inputs([64], H=2, dk=64, dv=64, dtype="bf16", seed=5)
    c = workloads.prefill_inputs([64], H=2, dk=64, dv=64, dtype="bf16", seed=6)
    for x, y in [(a.q, b.q), (a.k, b.k), (a.v, b.v), (a.beta, b.beta), (a.z, b.z)]:
        assert torch.equal(x, y)
    assert not torch.equal(a.q, c.q)
    assert a.q.dtype == torch.bfloat16 and a.z.dtype == torch.float32


def test_bf16_inputs_round_the_fp32_draws_to_nearest_even():
    f = workloads.prefill_inputs([32], H=1, dk=64, dv=64, dtype="fp32", seed=11)
    h = workloads.prefill_inputs([32], H=1, dk=64, dv=64, dtype="bf16", seed=11)
    assert torch.equal(f.v.to(torch.bfloat16), h.v)
    assert torch.equal(f.z, h.z)  # the gate input stays fp32


def test_blocked_draws_do_not_depend_on_threads(monkeypatch):
    """Each block of rows comes from its own stream spawned in order from the generator, so
    the thread pool that fills them changes nothing: the draws equal a serial fill."""
    monkeypatch.setattr(workloads, "_BLOCK_ELEMS", 256)
    got = workloads._normal(np.random.default_rng(77), (37, 5, 64), -4.0, 2.0,
                            post=workloads._l2norm_lastdim)
    streams = np.random.default_rng(77).spawn(-(-37 * 5 // 4))  # 4 rows of 64 per block
    rows = []
    for s in streams:
        x = s.standard_normal(size=(4, 64), dtype=np.float32) * np.float32(2.0) + np.float32(-4.0)
        rows.append(workloads._l2norm_lastdim(x))
    want = np.concatenate(rows)[:37 * 5].reshape(37, 5, 64)
    assert np.array_equal(got, want)


def test_varlen_lengths_are_log_uniform_in_range():
    rng = np.random.default_rng(3)
    lens = workloads.varlen_lengths(rng, 2000, 512, 16384)
    assert min(lens) >= 512 and max(lens) <= 16384
    logs = np.log(lens)
    # log-uniform: the median of log L sits at the middle of [ln 512, ln 16384]
    assert abs(np.median(logs) - 0.5 * (math.log(512) + math.log(16384))) < 0.1


def test_decode_inputs_shapes():
    d = workloads.decode_inputs(N=3, H=2, dk=64, dv=64, steps=5, dtype="bf16", seed=1)
    assert d.q.shape == (5, 3, 2, 64) and d.beta.shape == (5, 3, 2)
    assert d.S0.shape == (3, 2, 64, 64) and d.S0.dtype == torch.float32
    assert d.steps == 5 and d.N == 3 and d.H == 2


def test_unknown_workload_is_rejected():
    with pytest.raises(KeyError):
        workloads.make("no_such_workload")


# --- roofline accounting -----------------------------------------------------------------

def test_prefill_algorithmic_work_per_token_head():
    # d = 128, chunk 64: 6 C dk dv + C(C-1) dk + 2 C(C+1) dk + 2 C(C+1) dv + C^3 / 3, per C
    fl, by = bench.prefill_algorithmic(128, 128, 2)
    C = 64
    expect = (6 * C * 128 * 128 + C * (C - 1) * 128 + 2 * C * (C + 1) * 128
              + 2 * C * (C + 1) * 128 + C ** 3 / 3) / C
    assert fl == pytest.approx(expect) and round(fl) == 141013
    # bf16 q, k, v, beta, o plus fp32 z
    assert by == 3 * 128 * 2 + 2 + 4 * 128 + 128 * 2 == 1538
    fl64, _ = bench.prefill_algorithmic(64, 64, 2)
    assert round(fl64) == 46613


def test_decode_bytes_per_pair():
    # fp32 state read and written, plus one token's inputs and output
    assert bench.decode_bytes_per_pair(128, 128, 2) == 2 * 128 * 128 * 4 + 1538 == 132610


# --- profile summaries -------------------------------------------------------------------

def test_committed_summaries_name_their_sources_and_command():
    # a summary's figures are used only while its hash matches the kernel sources (the
    # readers below check that); here: every summary records a hash and the command it ran
    found = 0
    for f in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        txt = open(os.path.join(ROOT, "profiles", f)).read()
        assert re.search(r"kernel_source_hash:\s*[0-9a-f]{16}", txt), f"{f} names no kernel_source_hash"
        assert "rocprofv3 " in txt and "bench.py" in txt, f"{f} gives no command"
        found += 1
    assert found > 0


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    csrc = os.path.join(ROOT, "linear_attention_sequence_chunkwise_amd", "csrc")
    fake_root = tmp_path / "r"
    dst = fake_root / "linear_attention_sequence_chunkwise_amd" / "csrc"
    shutil.copytree(csrc, dst)
    monkeypatch.setattr(bench, "ROOT", str(fake_root))
    h0 = bench.kernel_source_hash()
    f = dst / "kda_gate.hip"
    f.write_text(f.read_text() + "\n// a new comment\n/* and a block one */\n")
    assert bench.kernel_source_hash() == h0
    f.write_text(f.read_text().replace("acc.x += gv.x;", "acc.x += gv.x * 1.0f;"))
    assert bench.kernel_source_hash() != h0
    # a summary depends only on its own kernels' sources: the gate change above leaves the
    # decode summaries' hash alone and changes the gate summaries' one
    h_dec = bench.kernel_source_hash(bench.summary_sources("decode_n512_h32_d128_bf16_256steps"))
    h_gate = bench.kernel_source_hash(bench.summary_sources("gate_b4_t32768_h32_d128_f32"))
    f.write_text(f.read_text().replace("acc.x += gv.x * 1.0f;", "acc.x += gv.x * 2.0f;"))
    assert bench.kernel_source_hash(bench.summary_sources("decode_n512_h32_d128_bf16_256steps")) == h_dec
    assert bench.kernel_source_hash(bench.summary_sources("gate_b4_t32768_h32_d128_f32")) != h_gate


def test_summary_readers_drop_stale_summaries(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    h = bench.kernel_source_hash()
    (prof / "w_traffic.txt").write_text(f"kernel_source_hash: {h}\ntraffic_bytes_per_launch: 1.5e+09\n")
    (prof / "w_mfma.txt").write_text(f"kernel_source_hash: {h}\nexecuted_bf16_flops_per_launch: 2e+10\n"
                                     "mfma_busy_frac_per_launch: 0.05\n")
    (prof / "old_traffic.txt").write_text("kernel_source_hash: 0000000000000000\n"
                                          "traffic_bytes_per_launch: 1e9\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda files=None: h)
    assert bench.read_traffic("w") == 1.5e9
    m = bench.read_mfma("w")
    assert m["executed_bf16_flops_per_launch"] == 2e10 and m["mfma_busy_frac"] == 0.05
    assert bench.read_traffic("old") is None
    assert bench.read_traffic("missing") is None and bench.read_mfma("missing") is None


def test_summarize_profiles_from_rocprof_csv(tmp_path, monkeypatch):
    """bench.py --summarize-profiles turns rocprofv3 CSV output into the summaries the readers
    use: kernel trace rows, counter means scaled by the calibration copy, the launch's total."""
    raw = tmp_path / "raw"
    w = "prefill_b1_h16_t4096_d128_bf16"
    (raw / f"{w}_kt").mkdir(parents=True)
    (raw / f"{w}_kt" / "kt_kernel_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"void kda::prefill_intra_kernel<128, unsigned short>(kda::SplitArgs)",2,60000,30000,60,29000,31000,1\n'
        '"void kda::prefill_state_lagged_kernel<128, 4, unsigned short>(kda::SplitArgs)",2,40000,20000,40,19000,21000,1\n'
        '"__amd_rocclr_copyBuffer",1,10,10,0.01,10,10,0\n')
    head = '"Dispatch_Id","Kernel_Name","Grid_Size","Counter_Name","Counter_Value"\n'
    for c, cal, vals in (("FETCH_SIZE", 524288.0, (1000.0, 3000.0)), ("WRITE_SIZE", 1048576.0, (500.0, 700.0))):
        d = raw / f"{w}_{c}"
        d.mkdir()
        rows = [f'1,"__amd_rocclr_copyBuffer",131072,"{c}",{cal}',
                f'2,"void kda::prefill_intra_kernel<128, unsigned short>(kda::SplitArgs)",262144,"{c}",{vals[0]}',
                f'3,"void kda::prefill_state_lagged_kernel<128, 4, unsigned short>(kda::SplitArgs)",256,"{c}",{vals[1]}']
        (d / "p_counter_collection.csv").write_text(head + "\n".join(rows) + "\n")
    out = tmp_path / "profiles"
    out.mkdir()
    done = bench.summarize_profiles(str(raw), str(out))
    assert sorted(done) == [f"{w}_kernel_trace", f"{w}_traffic"]
    kt = (out / f"{w}_kernel_trace.txt").read_text()
    assert "| `void kda::prefill_intra_kernel<128, unsigned short>` | 2 | 30.00 |" in kt
    assert "__amd_rocclr_copyBuffer" not in kt and "rocprofv3 --kernel-trace --stats" in kt
    tr = (out / f"{w}_traffic.txt").read_text()
    # FETCH_SIZE reads half the copied bytes: scale 2; WRITE_SIZE all of them: scale 1
    want = (1000 + 3000) * 1024 * 2 + (500 + 700) * 1024 * 1
    got = float(re.search(r"traffic_bytes_per_launch:\s*([0-9.e+]+)", tr).group(1))
    assert abs(got - want) / want < 1e-4
    h = bench.kernel_source_hash(bench.summary_sources(w))
    assert f"kernel_source_hash: {h}" in tr
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda files=None: h)
    assert bench.read_traffic(w) == got


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one MI355X" in r.stderr


# --- binding argument checks -------------------------------------------------------------
# The kernels take plain pointers, so the binding checks every tensor's shape and dtype
# against the call's sizes before anything is launched (these raise on the CPU, before the
# device check).

def _prefill_args(T=64, H=2, d=64):
    bf = torch.bfloat16
    return dict(q=torch.zeros(T, H, d, dtype=bf), k=torch.zeros(T, H, d, dtype=bf),
                v=torch.zeros(T, H, d, dtype=bf), beta=torch.zeros(T, H, dtype=bf),
                z=torch.zeros(T, H, d), A=torch.zeros(H, d))


def test_binding_rejects_mismatched_prefill_tensors():
    from linear_attention_sequence_chunkwise_amd import kda
    bad = [("v", torch.zeros(63, 2, 64, dtype=torch.bfloat16), "v: shape"),
           ("beta", torch.zeros(64, 2, 1, dtype=torch.bfloat16), "beta: shape"),
           ("z", torch.zeros(64, 2, 64, dtype=torch.bfloat16), "z: dtype"),
           ("A", torch.zeros(2, 32), "A: shape"),
           ("k", torch.zeros(64, 2, 64), "k: dtype")]
    for name, t, msg in bad:
        a = _prefill_args()
        a[name] = t
        with pytest.raises(ValueError, match=msg):
            kda.kda_prefill_fwd(**a)
    with pytest.raises(ValueError, match="initial_state: shape"):
        kda.kda_prefill_fwd(**_prefill_args(), initial_state=torch.zeros(2, 2, 64, 64))
    with pytest.raises(ValueError, match="o: shape"):
        kda.kda_prefill_fwd(**_prefill_args(), o=torch.zeros(64, 2, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="cu_seqlens: dtype"):
        kda.kda_prefill_fwd(**_prefill_args(), cu_seqlens=torch.tensor([0, 64]))
    with pytest.raises(ValueError, match="checkpoints"):
        kda.kda_prefill_fwd(**_prefill_args(), checkpoints=torch.zeros(0, 2, 64, 64),
                            checkpoint_interval=64)
    with pytest.raises(ValueError, match="GPU"):   # right shapes: only the device is wrong
        kda.kda_prefill_fwd(**_prefill_args())


def test_binding_rejects_mismatched_decode_tensors():
    from linear_attention_sequence_chunkwise_amd import kda
    bf = torch.bfloat16
    N, K, H, d = 3, 2, 2, 64
    q = torch.zeros(N, H, d, dtype=bf)
    args = dict(k=q.clone(), v=q.clone(), beta=torch.zeros(N, H, dtype=bf),
                z=torch.zeros(N, H, d), A=torch.zeros(H, d))
    with pytest.raises(ValueError, match="state: shape"):
        kda.kda_decode_step(q, **args, state=torch.zeros(N, H, d, 32))
    with pytest.raises(ValueError, match="z: dtype"):
        kda.kda_decode_step(q, **{**args, "z": torch.zeros(N, H, d, dtype=bf)},
                            state=torch.zeros(N, H, d, d))
    qk = torch.zeros(N, K, H, d, dtype=bf)
    margs = dict(v=qk.clone(), beta=torch.zeros(N, K, H, dtype=bf), z=torch.zeros(N, K, H, d),
                 A=torch.zeros(H, d), state=torch.zeros(N, H, d, d))
    with pytest.raises(ValueError, match="k: shape"):
        kda.kda_decode_verify(qk, torch.zeros(N, K + 1, H, d, dtype=bf), **margs)
    with pytest.raises(ValueError, match="accepted: dtype"):
        kda.kda_decode_commit(qk, **margs, accepted=torch.zeros(N, dtype=torch.int64))


def test_binding_rejects_mismatched_elementwise_tensors():
    from linear_attention_sequence_chunkwise_amd import kda
    with pytest.raises(ValueError, match="A: shape"):
        kda.kda_gate(torch.zeros(8, 2, 64), torch.zeros(3, 64))
    with pytest.raises(ValueError, match="g: dtype"):
        kda.kda_gate(torch.zeros(8, 2, 64), torch.zeros(2, 64),
                     g=torch.zeros(8, 2, 64, dtype=torch.bfloat16))
    o = torch.zeros(10, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="gate: dtype"):
        kda.kda_output_gate(o, torch.zeros(10, 128), torch.ones(128))
    with pytest.raises(ValueError, match="weight: shape"):
        kda.kda_output_gate(o, o.clone(), torch.ones(64))
    x = torch.zeros(70, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="weight: shape"):
        kda.kda_short_conv(x, torch.zeros(128, 4))
    with pytest.raises(ValueError, match="cache_in: shape"):
        kda.kda_short_conv(x, torch.zeros(256, 4), cache_in=torch.zeros(1, 256, 4))


def test_binding_calls_run_on_their_tensors_device(monkeypatch):
    """Each binding call makes its tensors' GPU current first (the library launches on, and sizes
    the prefill workspace for, the current device).  Checked on the host with a stand-in tensor
    that reports cuda:1 and a recording stand-in for torch.cuda.device."""
    import contextlib

    from linear_attention_sequence_chunkwise_amd import kda

    class OnCuda1(torch.Tensor):
        @property
        def is_cuda(self):
            return True

        @property
        def device(self):
            return torch.device("cuda", 1)

    seen = []

    @contextlib.contextmanager
    def record(dev):
        seen.append(dev)
        yield

    monkeypatch.setattr(torch.cuda, "device", record)

    @kda._on_tensor_device
    def call(a, b=None):
        return "ran"

    x = torch.zeros(2).as_subclass(OnCuda1)
    assert call(torch.zeros(1), b=x) == "ran" and seen == [torch.device("cuda", 1)]
    seen.clear()
    assert call(torch.zeros(1)) == "ran" and seen == []  # no GPU tensor: no device switch
