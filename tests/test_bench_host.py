"""Host logic of bench.py that needs no GPU: the roofline pass's call order, the CPU
baseline's report, the algorithmic bytes the roofline divides by, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from rank_latent_kv_amd.roofline import algorithmic_bytes  # noqa: E402
from rank_latent_kv_amd.workloads import PRESETS, default_seq_lens  # noqa: E402


class _FakeLib:
    """Stands in for the library's decode entry point: records which argument structs it got."""

    def __init__(self):
        self.calls = []

    def __call__(self, ref, stream):
        self.calls.append(ref._obj)
        return 0


@pytest.mark.parametrize("samples", [20, 40])
def test_event_pass_brackets_every_sample_once_after_its_warmup(samples):
    """The roofline pass runs its warm-up, then each event-bracketed call followed by a plain
    one, so a driver run with --steps 20 still yields at least 20 samples."""
    fn = _FakeLib()
    import ctypes
    plain = [ctypes.c_int(k) for k in range(3)]
    ev = [ctypes.c_int(100 + j) for j in range(samples)]
    bench.event_pass(fn, plain, ev, None, warm=7, samples=samples)
    assert all(fn.calls[k] is plain[k % 3] for k in range(7))
    tail = fn.calls[7:]
    assert len(tail) == 2 * samples
    assert all(a is b for a, b in zip(tail[0::2], ev)) and all(any(c is p for p in plain) for c in tail[1::2])


def test_timing_events_drop_the_system_fence():
    """The roofline events are created with hipEventDisableSystemFence: the flag value bench.py
    passes is the one the installed HIP header defines."""
    import re
    hdr = "/opt/rocm/include/hip/hip_runtime_api.h"
    if not os.path.exists(hdr):
        pytest.skip("no HIP headers on this host")
    m = re.search(r"#define\s+hipEventDisableSystemFence\s+(0x[0-9a-fA-F]+)", open(hdr).read())
    assert m and int(m.group(1), 16) == bench.HIP_EVENT_DISABLE_SYSTEM_FENCE


def test_driver_style_run_gets_twenty_event_samples():
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert "n_ev = max(20, args.event_samples)" in src


def test_cpu_baseline_reports_cores_threads_and_materialised_subset():
    """The oracle's timing on a tiny workload: cores from the affinity set, a single-thread
    time, and the materialised form on a subset of rows agreeing with the absorbed form."""
    from rank_latent_kv_amd.workloads import make_inputs
    w = PRESETS["mlra4_b16_l32k"].replace(batch=2, seq_len=300)
    inp = make_inputs(w)
    cb, ys = bench.cpu_baseline(w, inp, 0.2)
    assert cb["cores"] == len(os.sched_getaffinity(0)) and cb["kind"] == "oracle"
    assert cb["value"] > 0 and cb["single_thread"]["value"] > 0 and cb["blas_threads"] >= 1
    assert cb["materialised_subset"]["max_rel_diff_vs_absorbed"] < 1e-10
    assert ys.shape == (2, 64, 128)


def test_headline_algorithmic_bytes():
    """16 x 32768 cache rows of 320 bytes plus the bf16 queries (16 x 64 x 160 x 2 bytes)."""
    w = PRESETS["mlra4_b16_l32k"]
    ab = algorithmic_bytes(w, default_seq_lens(w).tolist())
    assert ab["cache"] == 16 * 32768 * 320
    assert ab["queries"] == 16 * 64 * 160 * 2
    assert ab["attention_kernel"] == 168_099_840


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_kernel_hash_ignores_comments_and_whitespace():
    """The stored counter figures stay valid across comment edits, not across code edits."""
    code = 'int f(int x) {  // doubles\n  /* note */ return 2 * x; }\nconst char* s = "a // b";\n'
    same = 'int f(int x) {\n  return 2 * x;   // twice\n}\nconst char* s = "a // b";\n'
    other = 'int f(int x) { return 3 * x; }\nconst char* s = "a // b";\n'
    assert bench.code_tokens(code) == bench.code_tokens(same)
    assert bench.code_tokens(code) != bench.code_tokens(other)
    assert '"a // b"' in bench.code_tokens(code)

