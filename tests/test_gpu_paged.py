"""GPU tests of the paged cache: append / gather are bit-exact against NumPy
indexing through the page table, paged decode matches the oracle and equals the
contiguous decode bit for bit on the same split boundaries (MLRA-4 and MLA)."""
import numpy as np
import pytest
import torch

import rank_latent_kv_amd as R
from rank_latent_kv_amd.workloads import PRESETS, make_inputs

from gpu_helpers import DEV, f64, gpu_decode, oracle_decode, row_rel_err, say

pytestmark = pytest.mark.gpu


def small_paged(lens, seed=None, peaked=False):
    w = PRESETS["mlra4_paged_b4_l64k_128k"].replace(batch=len(lens))
    return w, make_inputs(w, seq_lens=lens, seed=seed, peaked=peaked)


def test_paged_decode_matches_oracle():
    w, inp = small_paged([3000, 9000, 64, 4097])
    say("paged decode vs oracle")
    y = f64(gpu_decode(w, inp))
    err = row_rel_err(y, oracle_decode(w, inp))
    say(f"paged err {err:.3e}")
    assert err <= 1e-2


@pytest.mark.parametrize("num_splits", [1, 3, 8])
def test_paged_split_invariance(num_splits):
    """Explicit split counts through the page table: splits start on page boundaries of any
    count, and the result stays within the bf16 bound of the oracle."""
    w, inp = small_paged([3000, 9000, 64, 4097])
    say(f"paged num_splits={num_splits}")
    y = f64(gpu_decode(w, inp, num_splits=num_splits, out_dtype=torch.float32))
    err = row_rel_err(y, oracle_decode(w, inp))
    say(f"paged num_splits={num_splits} err {err:.3e}")
    assert err <= 1e-2


@pytest.mark.parametrize("page_size", [32, 256])
def test_paged_mla(page_size):
    """The single-latent kernel through a page table of other page sizes."""
    w = PRESETS["mlra4_paged_b4_l64k_128k"].replace(batch=3, branches=1, branch_dim=128, page_size=page_size,
                                                      name=f"mla_paged_ps{page_size}")
    inp = make_inputs(w, seq_lens=[2500, 700, 4096])
    say(f"mla paged page_size={page_size}")
    y = f64(gpu_decode(w, inp, mla=True))
    err = row_rel_err(y, oracle_decode(w, inp))
    say(f"mla paged page_size={page_size} err {err:.3e}")
    assert err <= 1e-2


def test_paged_peaked():
    w, inp = small_paged([5000, 2048], peaked=True)
    say("paged peaked")
    y = f64(gpu_decode(w, inp))
    assert row_rel_err(y, oracle_decode(w, inp)) <= 1e-2


def identity_paged(w, inp):
    """The same rows as `inp`, moved into a pool in sequence order (sequence b's page j at pool
    page b * max_pages + j) with the matching page table."""
    pool = inp["pool"]
    pt = inp["page_table"].numpy()
    B, mp = pt.shape
    ident = torch.zeros((B * mp,) + tuple(pool.shape[1:]), dtype=pool.dtype)
    table = np.full((B, mp), -1, dtype=np.int32)
    for b in range(B):
        for j in range(mp):
            if pt[b, j] >= 0:
                ident[b * mp + j] = pool[int(pt[b, j])]
                table[b, j] = b * mp + j
    return dict(inp, pool=ident, page_table=torch.from_numpy(table))


def gather_contiguous(w, inp):
    pool = inp["pool"]
    pt = inp["page_table"].numpy()
    lens = inp["seq_lens"].numpy()
    kv = torch.zeros((w.batch, int(lens.max()), pool.shape[-1]), dtype=pool.dtype)
    flat = pool.reshape(-1, pool.shape[-1])
    for b in range(w.batch):
        idx = [int(pt[b][s // w.page_size]) * w.page_size + s % w.page_size for s in range(int(lens[b]))]
        kv[b, :lens[b]] = flat[idx]
    return {"kv": kv, "q_lat": inp["q_lat"], "q_rope": inp["q_rope"], "w_v": inp["w_v"], "seq_lens": inp["seq_lens"]}


def test_paged_translation_is_exact():
    """A shuffled pool and the same rows laid out in sequence order give bit-identical
    outputs: the page table changes only where rows are read from."""
    w, inp = small_paged([2500, 6000, 128])
    ident = identity_paged(w, inp)
    say("paged: shuffled pool vs pool in sequence order, same splits")
    for ns in (3, 10):
        a = gpu_decode(w, inp, num_splits=ns)
        b = gpu_decode(w, ident, num_splits=ns)
        assert torch.equal(a, b), ns


def test_paged_equals_contiguous_bitwise_mlra4():
    """The paged and contiguous MLRA-4 instances split the work between waves identically, so
    on the same split boundaries they agree bit for bit (ragged last pages included)."""
    w, inp = small_paged([2500, 6000, 128])
    wc = w.replace(paged=False)
    say("paged vs contiguous, same splits (MLRA-4)")
    for ns in (3, 10):
        a = gpu_decode(w, inp, num_splits=ns)
        b = gpu_decode(wc, gather_contiguous(w, inp), num_splits=ns)
        assert torch.equal(a, b), ns


def test_paged_equals_contiguous_bitwise_mla():
    """The same for MLA (one branch per wave)."""
    w = PRESETS["mla_b16_l32k"].replace(batch=3, paged=True, page_size=64, name="mla_paged_small")
    inp = make_inputs(w, seq_lens=[2500, 6000, 128])
    wc = w.replace(paged=False)
    say("paged vs contiguous, same splits (MLA)")
    for ns in (3, 10):
        a = gpu_decode(w, inp, num_splits=ns, mla=True)
        b = gpu_decode(wc, gather_contiguous(w, inp), num_splits=ns, mla=True)
        assert torch.equal(a, b), ns


def test_long_splits_rotate_their_stage_order():
    """Splits of 64 or more full stages start at a per-sequence stage and wrap around. One
    split per sequence of 8,229-12,000 tokens (64-93 full stages and a ragged tail): the
    output follows the oracle, and the paged and contiguous instances, which rotate alike,
    still agree bit for bit (MLA: its page ids of up to 255 pages per split sit in LDS)."""
    w = PRESETS["mla_b16_l32k"].replace(batch=3, paged=True, page_size=64, name="mla_paged_long")
    lens = [8229, 12000, 8192]
    inp = make_inputs(w, seq_lens=lens)
    wc = w.replace(paged=False)
    say(f"rotated long splits, MLA lens {lens}")
    a = gpu_decode(w, inp, num_splits=1, mla=True)
    b = gpu_decode(wc, gather_contiguous(w, inp), num_splits=1, mla=True)
    assert torch.equal(a, b)
    assert row_rel_err(f64(a), oracle_decode(w, inp)) <= 1e-2
    w4 = PRESETS["mlra4_b16_l32k"].replace(batch=3)
    inp4 = make_inputs(w4, seq_lens=lens)
    say(f"rotated long splits, MLRA-4 lens {lens}")
    y = gpu_decode(w4, inp4, num_splits=1)
    assert row_rel_err(f64(y), oracle_decode(w4, inp4)) <= 1e-2


def test_append_and_gather_bitexact():
    rng = np.random.default_rng(3)
    ps, P, Rw = 64, 37, 160
    B = 4
    pool = torch.from_numpy(rng.standard_normal((P, ps, Rw)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    perm = rng.permutation(P)
    max_pages = 9
    pt = np.full((B, max_pages), -1, dtype=np.int32)
    lens = np.array([500, 64, 1, 300], dtype=np.int32)
    off = 0
    for b in range(B):
        n = -(-int(lens[b]) // ps)
        pt[b, :n] = perm[off:off + n]
        off += n
    R.page_table_check(torch.from_numpy(pt), torch.from_numpy(lens), ps, P)
    pt_d = torch.from_numpy(pt).to(DEV)
    # append the row for position lens-1 of each sequence
    rows = torch.from_numpy(rng.standard_normal((B, Rw)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    pos = torch.from_numpy(lens - 1).to(DEV)
    before = pool.clone()
    say("paged append")
    R.paged_append(pool, pt_d, pos, rows, page_size=ps)
    torch.cuda.synchronize()
    expect = before.clone().reshape(-1, Rw)
    for b in range(B):
        s = int(lens[b]) - 1
        expect[int(pt[b][s // ps]) * ps + s % ps] = rows[b]
    assert torch.equal(pool.reshape(-1, Rw), expect)
    say("paged gather")
    out = R.paged_gather(pool, pt_d, torch.from_numpy(lens).to(DEV), int(lens.max()), page_size=ps)
    torch.cuda.synchronize()
    flat = pool.reshape(-1, Rw).cpu()
    for b in range(B):
        idx = [int(pt[b][s // ps]) * ps + s % ps for s in range(int(lens[b]))]
        assert torch.equal(out[b, :lens[b]].cpu(), flat[idx])
        assert torch.all(out[b, lens[b]:] == 0)


def test_append_bad_page_flagged():
    ps, P, Rw = 64, 4, 160
    pool = torch.zeros((P, ps, Rw), dtype=torch.bfloat16, device=DEV)
    pt = torch.tensor([[0, 1], [2, 9]], dtype=torch.int32, device=DEV)     # 9 is outside the pool
    rows = torch.ones((2, Rw), dtype=torch.bfloat16, device=DEV)
    pos = torch.tensor([70, 70], dtype=torch.int32, device=DEV)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    say("append with a bad page id")
    R.paged_append(pool, pt, pos, rows, page_size=ps, error_flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) & R.FLAG_BAD_PAGE
    assert torch.all(pool[1, 6] == 1) and int((pool != 0).sum()) == Rw


def test_bad_page_in_decode_flagged():
    w, inp = small_paged([300, 200])
    inp = dict(inp)
    pt = inp["page_table"].clone()
    pt[1, 1] = 10 ** 6
    inp["page_table"] = pt
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    say("decode with a bad page id")
    y = gpu_decode(w, inp, error_flags=flags)
    assert int(flags.item()) & R.FLAG_BAD_PAGE
    assert torch.all(torch.isfinite(y.float()))
