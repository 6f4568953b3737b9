"""GPU parity at the benchmark's full sizes and at the size limits.

The four benchmark workloads run exactly as bench.py launches them (the default
seeded inputs, automatic context split, host-side lengths). The CPU oracle
checks every sequence where that takes seconds and a spread of sequences
otherwise; every output must be finite. The limit cases are a single
2^20-token context, the largest split count (4096 one-stage splits), a wide
batch of short ragged contexts and paged caches with pages smaller and larger
than a stage. Tolerance as in the other parity tests: max row relative error
1e-2 for bf16.
"""
import numpy as np
import pytest
import torch

from rank_latent_kv_amd.workloads import PRESETS, make_inputs

from gpu_helpers import f64, gpu_decode, oracle_decode, row_rel_err, say

pytestmark = pytest.mark.gpu

TOL = 1e-2


def check_sampled(w, inp, seqs, **kw):
    y = f64(gpu_decode(w, inp, **kw))
    assert np.all(np.isfinite(y))
    ref = oracle_decode(w, inp, seqs=seqs)
    err = row_rel_err(y[seqs], ref)
    say(f"{w.name}: {len(seqs)} sequences checked, row rel err {err:.3e}")
    assert err <= TOL, err
    return y


@pytest.mark.parametrize("preset,mla,seqs", [
    ("mlra4_b16_l32k", False, None),
    ("mla_b16_l32k", True, None),
    ("mlra2_b16_l32k", False, None),
    ("mlra4_paged_b4_l64k_128k", False, None),
    ("mlra4_tp_shard_b64_l64k", False, list(range(0, 64, 4)) + [63]),
    ("mla_tp_shard_b64_l64k", True, list(range(0, 64, 8)) + [63]),
    ("mlra4_branch_shard_b64_l64k", False, list(range(0, 64, 8)) + [63]),
])
def test_benchmark_workload_full_size(preset, mla, seqs):
    w = PRESETS[preset]
    say(f"full size {preset}")
    inp = make_inputs(w)
    seqs = list(range(w.batch)) if seqs is None else seqs
    check_sampled(w, inp, seqs, mla=mla)


def test_peaked_logits_at_full_length():
    """Planted dominant logits over whole 32k contexts: the running-max rescales and the split
    merge at the benchmark's launch configuration."""
    w = PRESETS["mlra4_b16_l32k"].replace(batch=4, name="mlra4_b4_l32k_peaked")
    say("peaked logits, 4 x 32768 tokens")
    check_sampled(w, make_inputs(w, peaked=True), [0, 1, 2, 3])


def test_single_context_of_a_million_tokens():
    w = PRESETS["mlra4_b16_l32k"].replace(batch=1, seq_len=1 << 20, name="mlra4_b1_l1m")
    say("single 2^20-token context")
    check_sampled(w, make_inputs(w), [0])


def test_largest_split_count():
    """4096 splits of one 128-token stage each, the last one ragged."""
    w = PRESETS["mlra4_b16_l32k"].replace(batch=2, name="mlra4_max_splits")
    L = 4096 * 128
    inp = make_inputs(w, seq_lens=[L, L - 77])
    say("4096 one-stage splits")
    check_sampled(w, inp, [0, 1], num_splits=4096)


def test_wide_batch_of_short_contexts():
    w = PRESETS["mlra4_b16_l32k"].replace(batch=512, name="mlra4_b512_short")
    rng = np.random.default_rng(5)
    lens = rng.integers(1, 400, size=512).tolist()
    say("512 short ragged contexts")
    check_sampled(w, make_inputs(w, seq_lens=lens), list(range(0, 512, 8)) + [511])


@pytest.mark.parametrize("page_size", [16, 128, 1024])
def test_paged_page_sizes(page_size):
    w = PRESETS["mlra4_paged_b4_l64k_128k"].replace(batch=3, page_size=page_size,
                                                   name=f"mlra4_paged_ps{page_size}")
    inp = make_inputs(w, seq_lens=[20000, 4097, 300])
    say(f"paged, page_size {page_size}")
    check_sampled(w, inp, [0, 1, 2])
