"""Host logic of bench.py that needs no GPU: which timed calls carry the attention kernel's
events, the algorithmic bytes the roofline divides by, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from rank_latent_kv_amd.roofline import algorithmic_bytes  # noqa: E402
from rank_latent_kv_amd.workloads import PRESETS, default_seq_lens  # noqa: E402


@pytest.mark.parametrize("steps,every", [(400, 16), (20, 16), (5, 16), (1, 16), (9, 16), (8, 16),
                                         (17, 16), (400, 1), (3, 0), (100, 7)])
def test_event_schedule_covers_exactly_the_sampled_calls(steps, every):
    ev, phase, n = bench.event_schedule(steps, every)
    sampled = [k for k in range(steps) if k % ev == phase]
    assert len(sampled) == n >= 1
    # sample j sits at call phase + j * every, so k // every indexes the event list densely
    assert [k // ev for k in sampled] == list(range(n))
    assert 0 <= phase < ev


def test_event_schedule_skips_the_first_call_when_it_can():
    ev, phase, n = bench.event_schedule(400, 16)
    assert (ev, phase, n) == (16, 8, 25)


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
