"""GPU parity: the HIP library (through the C ABI) against the CPU fp64 oracle on
the same seeded inputs.

Tolerance (bf16 inputs, fp32 accumulation): per output row (sequence, head),
max_j |y_gpu - y_ref| / max_j |y_ref| <= 1e-2. The fp32 path must reach 1e-5.
Index and page-table work is compared bit for bit.
"""
import numpy as np
import pytest
import torch

import rank_latent_kv_amd as R
from oracle import mlra_oracle as O
from rank_latent_kv_amd.workloads import PRESETS, make_inputs

from gpu_helpers import DEV, f64, gpu_decode, oracle_decode, row_rel_err, say

pytestmark = pytest.mark.gpu

TOL_BF16 = 1e-2
TOL_F32 = 1e-5


def check(w, inp, tol=TOL_BF16, **kw):
    y = f64(gpu_decode(w, inp, **kw))
    ref = oracle_decode(w, inp)
    err = row_rel_err(y, ref)
    say(f"{w.name}: row rel err {err:.3e}")
    assert np.all(np.isfinite(y))
    assert err <= tol, err
    return y, ref


def test_tiny_f32():
    w = PRESETS["tiny_f32"]
    say("tiny_f32 generic fp32")
    y, _ = check(w, make_inputs(w), tol=TOL_F32, out_dtype=torch.float32)
    golden = np.load("tests/golden/tiny_f32_y.npy")
    assert row_rel_err(y, golden) <= TOL_F32


@pytest.mark.parametrize("lens", [[1000, 777, 2049], [1, 33, 129], [4096]])
def test_mlra4_bf16_ragged(lens):
    w = PRESETS["mlra4_b16_l32k"].replace(batch=len(lens))
    say(f"mlra4 bf16 lens={lens}")
    check(w, make_inputs(w, seq_lens=lens))


def test_mlra4_fp32_output():
    w = PRESETS["mlra4_b16_l32k"].replace(batch=2)
    say("mlra4 bf16 in, fp32 out")
    check(w, make_inputs(w, seq_lens=[1500, 600]), out_dtype=torch.float32)


@pytest.mark.parametrize("lens", [[1500, 333], [1, 2, 4095]])
def test_mla_bf16(lens):
    w = PRESETS["mla_b16_l32k"].replace(batch=len(lens))
    say(f"mla bf16 lens={lens}")
    check(w, make_inputs(w, seq_lens=lens), mla=True)


def test_mla_equals_single_branch_mlra_entry():
    w = PRESETS["mla_b16_l32k"].replace(batch=2)
    inp = make_inputs(w, seq_lens=[900, 1300])
    say("mla_decode vs mlra_decode with one branch")
    a = gpu_decode(w, inp, mla=True)
    b = gpu_decode(w, inp, mla=False)
    assert torch.equal(a, b)


@pytest.mark.parametrize("lens", [[700, 2000, 64, 5]])
def test_tp_shard_16_heads(lens):
    w = PRESETS["mlra4_tp_shard_b64_l64k"].replace(batch=len(lens))
    say(f"tp shard h=16 lens={lens}")
    check(w, make_inputs(w, seq_lens=lens))


@pytest.mark.parametrize("lens", [[700, 2000, 64, 5]])
def test_mla_tp_shard_16_heads(lens):
    w = PRESETS["mla_tp_shard_b64_l64k"].replace(batch=len(lens))
    say(f"mla tp shard h=16 lens={lens}")
    check(w, make_inputs(w, seq_lens=lens), mla=True)


@pytest.mark.parametrize("lens", [[1, 33, 129, 2049]])
def test_mlra2_bf16_ragged(lens):
    w = PRESETS["mlra2_b16_l32k"].replace(batch=len(lens))
    say(f"mlra2 bf16 lens={lens}")
    check(w, make_inputs(w, seq_lens=lens))


@pytest.mark.parametrize("preset,mla", [("mlra4_tp_shard_b64_l64k", False), ("mla_tp_shard_b64_l64k", True)])
def test_tp_shard_fp32_output(preset, mla):
    w = PRESETS[preset].replace(batch=3)
    say(f"{preset} fp32 out")
    check(w, make_inputs(w, seq_lens=[3000, 257, 1]), mla=mla, out_dtype=torch.float32)


@pytest.mark.parametrize("nb,db,heads", [(1, 32, 64), (2, 64, 64)])
def test_other_mfma_shapes(nb, db, heads):
    w = PRESETS["mlra4_b16_l32k"].replace(batch=2, branches=nb, branch_dim=db, heads=heads, name=f"nb{nb}_db{db}")
    say(f"mfma shape nb={nb} db={db} h={heads}")
    check(w, make_inputs(w, seq_lens=[1234, 3000]))


def test_generic_bf16_shape():
    w = PRESETS["mlra4_b16_l32k"].replace(batch=2, heads=8, branches=3, branch_dim=16, rope_dim=16, head_dim=48,
                                           name="generic_bf16")
    say("generic bf16 nb=3 db=16")
    check(w, make_inputs(w, seq_lens=[300, 700]))


@pytest.mark.parametrize("nb,db,dh", [(4, 32, 64), (4, 32, 256), (8, 32, 128), (2, 32, 128)])
def test_mfma_merge_shapes(nb, db, dh):
    """Every MFMA merge build beyond the workloads' own (d_c, d_h): (128, 64), (128, 256),
    (256, 128) and (64, 128). Eight heads have no attention build, so the generic attention
    kernel writes the fp32 split records and the MFMA merge (W^V operands requested before the
    records, one 16-wide output tile per wave and tile slot) applies W^V; several splits per
    sequence exercise its log-sum-exp merge."""
    w = PRESETS["mlra4_b16_l32k"].replace(batch=3, heads=8, branches=nb, branch_dim=db, head_dim=dh,
                                           name=f"merge_dc{nb * db}_dh{dh}")
    inp = make_inputs(w, seq_lens=[1300, 520, 77])
    say(f"mfma merge d_c={nb * db} d_h={dh}")
    for ns in (0, 5):
        check(w, inp, num_splits=ns)


@pytest.mark.parametrize("preset,mla", [("mlra4_b16_l32k", False), ("mla_b16_l32k", True),
                                        ("mlra4_tp_shard_b64_l64k", False), ("mla_tp_shard_b64_l64k", True),
                                        ("mlra2_b16_l32k", False)])
def test_peaked_logits(preset, mla):
    w = PRESETS[preset].replace(batch=2)
    inp = make_inputs(w, seq_lens=[4096, 2500], peaked=True)
    say(f"peaked {preset}")
    y = f64(gpu_decode(w, inp, mla=mla))
    ref = oracle_decode(w, inp)
    err = row_rel_err(y, ref)
    say(f"peaked {preset}: {err:.3e}")
    assert err <= TOL_BF16


@pytest.mark.parametrize("offset", [-300.0, 300.0])
@pytest.mark.parametrize("preset,mla", [("mlra4_b16_l32k", False), ("mla_b16_l32k", True)])
def test_logit_offset(offset, preset, mla):
    """Adding one constant to every logit of a head leaves its softmax unchanged. Here the
    RoPE key is the same vector for every token, so q^R . k^R shifts all logits by `offset`
    (natural-log units): far past where exp over- or underflows in fp32 unless a reference
    max is subtracted. The oracle subtracts the exact max in fp64."""
    lens = [3000, 700]
    w = PRESETS[preset].replace(batch=len(lens))
    inp = make_inputs(w, seq_lens=lens)
    dc, k0 = w.latent_dim, 16.0
    kv = inp["kv"].float()
    kv[..., dc:] = 0.0
    kv[..., dc] = k0
    q_rope = torch.zeros(inp["q_rope"].shape)
    q_rope[..., 0] = offset / (w.sm_scale * k0)
    inp = dict(inp, kv=kv.to(inp["kv"].dtype), q_rope=q_rope.to(inp["q_rope"].dtype))
    say(f"logit offset {offset} {preset}")
    check(w, inp, mla=mla)


def test_split_invariance():
    w = PRESETS["mlra4_b16_l32k"].replace(batch=2)
    inp = make_inputs(w, seq_lens=[3000, 2900])
    ref = oracle_decode(w, inp)
    ys = {}
    for s in (1, 2, 7, 16, 24):
        say(f"split invariance num_splits={s}")
        ys[s] = f64(gpu_decode(w, inp, num_splits=s, out_dtype=torch.float32))
        assert row_rel_err(ys[s], ref) <= TOL_BF16
    for s in ys:
        assert row_rel_err(ys[s], ys[1]) <= 5e-3


def test_deterministic():
    w = PRESETS["mlra4_b16_l32k"].replace(batch=3)
    inp = make_inputs(w, seq_lens=[2000, 100, 5000])
    say("determinism")
    a = gpu_decode(w, inp)
    b = gpu_decode(w, inp)
    assert torch.equal(a, b)


def test_context_length_one_gpu():
    w = PRESETS["mlra4_b16_l32k"].replace(batch=2)
    inp = make_inputs(w, seq_lens=[1, 1])
    say("L = 1")
    y = f64(gpu_decode(w, inp, out_dtype=torch.float32))
    kv = f64(inp["kv"])
    wv = f64(inp["w_v"])
    db = w.branch_dim
    expect = np.zeros_like(y)
    for beta in range(2):
        for b in range(w.branches):
            expect[beta] += np.einsum("inj,j->in", wv[:, :, b * db:(b + 1) * db], kv[beta, 0, b * db:(b + 1) * db])
    expect *= w.alpha
    assert row_rel_err(y, expect) <= 1e-3


def test_materialised_oracle_subset():
    """The GPU against the materialised oracle (per-branch K and V built from the
    non-absorbed up-projections) on a few (sequence, head) rows."""
    w = PRESETS["mlra4_b16_l32k"].replace(batch=2)
    inp = make_inputs(w, seq_lens=[1500, 700])
    say("materialised oracle subset")
    y = f64(gpu_decode(w, inp))
    rng = np.random.default_rng(11)
    q_nope, w_k = O.absorption_consistent_query(f64(inp["q_lat"]), w.head_dim, rng)
    kv = f64(inp["kv"])
    dc = w.latent_dim
    heads = [0, 17, 63]
    ref = O.mlra_decode_materialised(q_nope, w_k, f64(inp["q_rope"]), kv[:, :, :dc], kv[:, :, dc:],
                                     inp["seq_lens"].numpy(), f64(inp["w_v"]), w.sm_scale, w.alpha,
                                     num_branches=w.branches, seqs=[0, 1], heads=heads)
    assert row_rel_err(y[:, heads], ref[:, heads]) <= TOL_BF16


def test_error_flag_for_long_seq_len():
    """A device seq_len above max_seq_len is clamped on the device and flagged."""
    w = PRESETS["mlra4_b16_l32k"].replace(batch=2)
    inp = make_inputs(w, seq_lens=[512, 512])
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    bad = torch.tensor([512, 100000], dtype=torch.int32, device=DEV)
    say("error flag: seq_len > max_seq_len")
    y = gpu_decode(w, inp, host_lens=False, seq_lens_dev=bad, error_flags=flags, max_seq_len=512)
    assert int(flags.item()) & R.FLAG_SEQ_LEN_CLAMPED
    ref = oracle_decode(w, inp)
    assert row_rel_err(f64(y), ref) <= TOL_BF16


@pytest.mark.parametrize("preset,mla", [("mlra4_b16_l32k", False), ("mla_b16_l32k", True),
                                        ("mlra4_tp_shard_b64_l64k", False)])
def test_device_lengths_below_the_host_copy(preset, mla):
    """The host copy says every sequence holds 3000 rows (and they exist), so each split's first
    stage below row 3000 is read before the device length arrives. The device lengths are
    shorter: 100 rows (a ragged first stage, read again over the same slots, and empty splits
    that leave early), 2500 (a ragged last split) and 129 (a one-row split). The output must
    follow the device lengths."""
    w = PRESETS[preset].replace(batch=3)
    inp = make_inputs(w, seq_lens=[3000, 3000, 3000])
    dev_lens = [100, 2500, 129]
    say(f"{preset}: device lengths {dev_lens} below the host copy 3000")
    y = gpu_decode(w, inp, mla=mla, seq_lens_dev=torch.tensor(dev_lens, dtype=torch.int32, device=DEV))
    ref = oracle_decode(w, dict(inp, seq_lens=torch.tensor(dev_lens, dtype=torch.int32)))
    assert row_rel_err(f64(y), ref) <= TOL_BF16


@pytest.mark.parametrize("preset,out_dtype", [("mlra4_b16_l32k", torch.bfloat16), ("tiny_f32", torch.float32)])
def test_empty_device_lengths_give_zero_rows(preset, out_dtype):
    """Device lengths of 0 and below are clamped to an empty context and flagged: those
    sequences' outputs are exact zeros (no token contributes, nothing is NaN), and the other
    sequences are unaffected (matrix-core path and generic fp32 path)."""
    w = PRESETS[preset].replace(batch=3)
    inp = make_inputs(w, seq_lens=[200, 200, 200])
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    bad = torch.tensor([0, -5, 200], dtype=torch.int32, device=DEV)
    say(f"{preset}: device lengths 0 and -5")
    y = gpu_decode(w, inp, host_lens=False, seq_lens_dev=bad, error_flags=flags, out_dtype=out_dtype)
    assert int(flags.item()) & R.FLAG_SEQ_LEN_CLAMPED
    assert bool(torch.all(y[:2] == 0))
    tol = TOL_F32 if out_dtype == torch.float32 else TOL_BF16
    assert row_rel_err(f64(y[2:]), oracle_decode(w, inp, seqs=[2])) <= tol


def test_caller_workspace_reuse():
    w = PRESETS["mlra4_b16_l32k"].replace(batch=2)
    inp = make_inputs(w, seq_lens=[3000, 3000])
    d = {k: v.to(DEV) for k, v in inp.items()}
    dc = w.latent_dim
    args = R.make_args(d["q_lat"], d["q_rope"], d["kv"][..., :dc], d["kv"][..., dc:], d["seq_lens"], d["w_v"],
                       sm_scale=w.sm_scale, alpha=w.alpha)
    ws = torch.full((R.workspace_size(args),), 0xAB, dtype=torch.uint8, device=DEV)
    say("caller workspace (poisoned)")
    y1 = gpu_decode(w, inp, workspace=ws)
    y2 = gpu_decode(w, inp, workspace=ws)
    assert torch.equal(y1, y2)
    assert row_rel_err(f64(y1), oracle_decode(w, inp)) <= TOL_BF16


@pytest.mark.parametrize("fill", [float("nan"), float("inf"), float("-inf"), 1e30])
@pytest.mark.parametrize("preset,mla", [("mlra4_b16_l32k", False), ("mla_b16_l32k", True),
                                        ("mlra4_paged_b4_l64k_128k", False)])
def test_unwritten_split_records_are_ignored(fill, preset, mla):
    """With ragged lengths the shorter sequences leave split records of the workspace
    unwritten; whatever the caller's workspace held there (NaN, infinities, huge values)
    must not reach the output."""
    lens = [9000, 300, 5000, 2100]
    w = PRESETS[preset].replace(batch=len(lens))
    inp = make_inputs(w, seq_lens=lens)
    d = {k: v.to(DEV) for k, v in inp.items()}
    dc = w.latent_dim
    if w.paged:
        pool = d["pool"]
        args = R.make_args(d["q_lat"], d["q_rope"], pool[..., :dc], pool[..., dc:], d["seq_lens"], d["w_v"],
                           sm_scale=w.sm_scale, alpha=w.alpha, page_table=d["page_table"], page_size=w.page_size,
                           num_pages=pool.shape[0], row_stride=pool.shape[-1], max_seq_len=max(lens),
                           seq_lens_host=inp["seq_lens"].to(torch.int32), num_splits=12)
    else:
        q_lat = d["q_lat"]
        args = R.make_args(q_lat, d["q_rope"], d["kv"][..., :dc], d["kv"][..., dc:], d["seq_lens"], d["w_v"],
                           sm_scale=w.sm_scale, alpha=w.alpha, seq_lens_host=inp["seq_lens"].to(torch.int32),
                           num_splits=12)
    n = R.workspace_size(args)
    ws = torch.full((n // 4,), fill, dtype=torch.float32, device=DEV)
    say(f"unwritten records filled with {fill}, {preset}")
    y = f64(gpu_decode(w, inp, mla=mla, num_splits=12, workspace=ws))
    assert np.all(np.isfinite(y))
    assert row_rel_err(y, oracle_decode(w, inp)) <= TOL_BF16
