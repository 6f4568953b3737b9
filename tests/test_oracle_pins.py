"""Pins for the CPU oracle: checks against facts that the pages and the
mathematics fix, none of which re-types the oracle's own formula.

  absorbed == materialised       absorption identity ([MLA-LR] §3.3, [MLRA] §1.3 / §二)
  n_b = 1 reduces to MLA          [MLRA] §1.3 three-step MLA decode (independent code)
  each branch == torch SDPA       MQA-style attention per branch, library routine in fp64
  L = 1                           output is the up-projected latent, independent of queries
  L = 2                           closed form via the logistic function
  permutation / equal rows        softmax is a convex, order-free weighting
  RoPE-key shift                  adding a vector to every k^R shifts each logit row by a constant
  independent softmax             MLRA != one shared softmax (the [MLRA] §三 change)
  split / merge                   log-sum-exp identity for any chunking
  brute force                     scalar loops, math.exp, fsum, no max shift
  paged gather                    page-table translation by hand-written indexing
  linearity                       alpha and W^V enter linearly
  planted mistakes                mutants of the oracle fail at least one pin
  RoPE                            complex multiplication by exp(i m theta_j), relative-position
                                  invariance of scores, frequencies, identity at position 0
  query absorption                q~ . c == q^N . (W^UK c) for random latents c
  prepare + decode                rotated cache and query == attention with the rotation in the score

Page keys: [MLRA] "原生支持张量并行的多分支低秩注意力MLRA：优化KV缓存，实现2.8倍解码加速";
[MLA-LR] "Multi-Head Latent Attention：低秩近似优化Transformer计算效率".
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import mlra_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_problem(seed=0, B=2, h=3, nb=4, db=5, dr=3, dh=7, lens=(9, 4), scale=1.0):
    rng = np.random.default_rng(seed)
    Lmax = max(lens)
    dc = nb * db
    return dict(
        q_lat=rng.standard_normal((B, h, nb, db)) * scale,
        q_rope=rng.standard_normal((B, h, dr)) * scale,
        kv_lat=rng.standard_normal((B, Lmax, dc)) * scale,
        kv_rope=rng.standard_normal((B, Lmax, dr)) * scale,
        seq_lens=np.array(lens),
        w_v=rng.standard_normal((h, dh, dc)),
        sm_scale=0.37,
        alpha=0.61,
    )


def absorbed(p, **kw):
    q = dict(p)
    q.update(kw)
    return O.mlra_decode_absorbed(q["q_lat"], q["q_rope"], q["kv_lat"], q["kv_rope"], q["seq_lens"],
                                  q["w_v"], q["sm_scale"], q["alpha"])


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---- pins that use library routines or independent code ---------------------------------

def sdpa_reference(p):
    """y from torch's scaled_dot_product_attention (fp64, CPU) run once per branch
    with query [q~_b ; q^R], one key/value head broadcast to all query heads
    (K = [c_b ; k^R], V = c_b), then W^V per branch, summed and scaled."""
    B, h, nb, db = p["q_lat"].shape
    dh = p["w_v"].shape[1]
    y = np.zeros((B, h, dh))
    for beta in range(B):
        L = int(p["seq_lens"][beta])
        for b in range(nb):
            cb = p["kv_lat"][beta, :L, b * db:(b + 1) * db]
            q = torch.from_numpy(np.concatenate([p["q_lat"][beta, :, b, :], p["q_rope"][beta]], axis=1))
            k = torch.from_numpy(np.concatenate([cb, p["kv_rope"][beta, :L]], axis=1))
            v = torch.from_numpy(np.ascontiguousarray(cb))
            out = torch.nn.functional.scaled_dot_product_attention(
                q[None, :, None, :], k[None, None].expand(1, h, L, k.shape[1]),
                v[None, None].expand(1, h, L, db), scale=p["sm_scale"])[0, :, 0, :].numpy()  # [h, d_b]
            for i in range(h):
                y[beta, i] += p["w_v"][i, :, b * db:(b + 1) * db] @ out[i]
    return p["alpha"] * y


def test_branch_equals_sdpa():
    for seed in range(3):
        p = rand_problem(seed)
        assert rel(absorbed(p), sdpa_reference(p)) < 1e-12


def test_bruteforce_tiny():
    for seed in range(3):
        p = rand_problem(seed, B=2, h=2, nb=2, db=3, dr=2, dh=3, lens=(5, 3))
        bf = O.mlra_decode_bruteforce(p["q_lat"], p["q_rope"], p["kv_lat"], p["kv_rope"], p["seq_lens"],
                                      p["w_v"], p["sm_scale"], p["alpha"])
        assert rel(absorbed(p), bf) < 1e-12


def test_absorbed_equals_materialised():
    rng = np.random.default_rng(5)
    p = rand_problem(1, B=2, h=3, nb=4, db=3, dr=2, dh=16, lens=(11, 6))
    q_nope, w_k = O.absorption_consistent_query(p["q_lat"], 16, rng)
    # absorption really reproduces q~ (W^K_i^T q^N_i == q~_i)
    back = np.einsum("inc,bin->bic", w_k, q_nope).reshape(p["q_lat"].shape)
    assert np.max(np.abs(back - p["q_lat"])) < 1e-12
    mat = O.mlra_decode_materialised(q_nope, w_k, p["q_rope"], p["kv_lat"], p["kv_rope"], p["seq_lens"],
                                     p["w_v"], p["sm_scale"], p["alpha"], num_branches=4)
    assert rel(absorbed(p), mat) < 1e-12


def test_materialised_subset_rows():
    rng = np.random.default_rng(6)
    p = rand_problem(2, B=3, h=4, nb=4, db=2, dr=2, dh=8, lens=(7, 3, 5))
    q_nope, w_k = O.absorption_consistent_query(p["q_lat"], 8, rng)
    mat = O.mlra_decode_materialised(q_nope, w_k, p["q_rope"], p["kv_lat"], p["kv_rope"], p["seq_lens"],
                                     p["w_v"], p["sm_scale"], p["alpha"], num_branches=4,
                                     seqs=[0, 2], heads=[1, 3])
    full = absorbed(p)
    for beta in (0, 2):
        for i in (1, 3):
            assert rel(mat[beta, i], full[beta, i]) < 1e-12
    assert np.all(mat[1] == 0) and np.all(mat[:, 0] == 0)


def test_single_branch_is_mla():
    p = rand_problem(3, nb=1, db=12)
    y_mla = O.mla_decode(p["q_lat"][:, :, 0, :], p["q_rope"], p["kv_lat"], p["kv_rope"], p["seq_lens"],
                         p["w_v"], p["sm_scale"], p["alpha"])
    assert rel(absorbed(p), y_mla) < 1e-12


def test_mla_three_step_against_sdpa():
    """MLA itself pinned to SDPA with the concatenated key [c ; k^R] and value c."""
    p = rand_problem(4, nb=1, db=12)
    assert rel(O.mla_decode(p["q_lat"], p["q_rope"], p["kv_lat"], p["kv_rope"], p["seq_lens"], p["w_v"],
                            p["sm_scale"], p["alpha"]), sdpa_reference(p)) < 1e-12


# ---- closed forms and invariants ---------------------------------------------------------

def test_context_length_one():
    p = rand_problem(7, lens=(1, 1))
    nb, db = p["q_lat"].shape[2], p["q_lat"].shape[3]
    expect = np.zeros((2, 3, 7))
    for beta in range(2):
        for i in range(3):
            for b in range(nb):
                expect[beta, i] += p["w_v"][i, :, b * db:(b + 1) * db] @ p["kv_lat"][beta, 0, b * db:(b + 1) * db]
    expect *= p["alpha"]
    assert rel(absorbed(p), expect) < 1e-13
    # independent of the queries
    p2 = dict(p, q_lat=p["q_lat"] * -3.0 + 1.0, q_rope=p["q_rope"] * 5.0)
    assert rel(absorbed(p2), expect) < 1e-13


def test_context_length_two_closed_form():
    p = rand_problem(8, lens=(2, 2))
    B, h, nb, db = p["q_lat"].shape
    expect = np.zeros((B, h, 7))
    for beta in range(B):
        for i in range(h):
            for b in range(nb):
                c0 = p["kv_lat"][beta, 0, b * db:(b + 1) * db]
                c1 = p["kv_lat"][beta, 1, b * db:(b + 1) * db]
                z = [p["sm_scale"] * (p["q_lat"][beta, i, b] @ c + p["q_rope"][beta, i] @ p["kv_rope"][beta, s])
                     for s, c in ((0, c0), (1, c1))]
                p0 = 1.0 / (1.0 + math.exp(z[1] - z[0]))        # logistic(z0 - z1)
                u = p0 * c0 + (1.0 - p0) * c1
                expect[beta, i] += p["w_v"][i, :, b * db:(b + 1) * db] @ u
    assert rel(absorbed(p), p["alpha"] * expect) < 1e-13


def test_permutation_invariance():
    p = rand_problem(9, lens=(9, 9))
    rng = np.random.default_rng(1)
    perm = rng.permutation(9)
    q = dict(p, kv_lat=p["kv_lat"][:, perm], kv_rope=p["kv_rope"][:, perm])
    assert rel(absorbed(q), absorbed(p)) < 1e-13


def test_equal_rows_give_the_row():
    p = rand_problem(10, lens=(6, 6))
    kv_lat = np.repeat(p["kv_lat"][:, :1], 6, axis=1)
    kv_rope = np.random.default_rng(3).standard_normal(p["kv_rope"].shape)   # logits still differ
    q = dict(p, kv_lat=kv_lat, kv_rope=kv_rope, seq_lens=np.array([6, 6]))
    y1 = absorbed(dict(q, seq_lens=np.array([1, 1]), kv_rope=kv_rope[:, :1]))
    assert rel(absorbed(q), y1) < 1e-13


def test_rope_key_shift_invariance():
    p = rand_problem(11)
    shift = np.random.default_rng(4).standard_normal(p["kv_rope"].shape[2])
    q = dict(p, kv_rope=p["kv_rope"] + shift)
    assert rel(absorbed(q), absorbed(p)) < 1e-12


def test_rope_term_matters():
    """The RoPE score is part of every branch's logit (shift by a per-token vector changes y)."""
    p = rand_problem(12)
    q = dict(p, kv_rope=p["kv_rope"] * 2.0)
    assert rel(absorbed(q), absorbed(p)) > 1e-3


def test_independent_softmax_differs_from_shared():
    p = rand_problem(13, lens=(9, 7))
    shared = O.shared_softmax_decode(p["q_lat"], p["q_rope"], p["kv_lat"], p["kv_rope"], p["seq_lens"],
                                     p["w_v"], p["sm_scale"], p["alpha"])
    assert rel(absorbed(p), shared) > 1e-1
    p1 = dict(p, seq_lens=np.array([1, 1]))
    shared1 = O.shared_softmax_decode(p1["q_lat"], p1["q_rope"], p1["kv_lat"], p1["kv_rope"], p1["seq_lens"],
                                      p1["w_v"], p1["sm_scale"], p1["alpha"])
    assert rel(absorbed(p1), shared1) < 1e-13


def test_split_merge_identity():
    p = rand_problem(14, lens=(37, 20), scale=2.0)
    rng = np.random.default_rng(7)
    for beta in range(2):
        L = int(p["seq_lens"][beta])
        whole = O.merge_partials([O.branch_partials(p["q_lat"], p["q_rope"], p["kv_lat"], p["kv_rope"], beta, 0, L,
                                                    p["sm_scale"])])
        # whole-context state equals the softmax-weighted latent (checked against SDPA via y below)
        for trial in range(5):
            cuts = sorted(set(rng.integers(1, L, size=rng.integers(1, 6)).tolist()))
            bounds = [0] + cuts + [L]
            parts = [O.branch_partials(p["q_lat"], p["q_rope"], p["kv_lat"], p["kv_rope"], beta, a, b,
                                       p["sm_scale"]) for a, b in zip(bounds[:-1], bounds[1:])]
            assert np.max(np.abs(O.merge_partials(parts) - whole)) < 1e-12
        # chunks of one token each
        parts = [O.branch_partials(p["q_lat"], p["q_rope"], p["kv_lat"], p["kv_rope"], beta, s, s + 1,
                                   p["sm_scale"]) for s in range(L)]
        assert np.max(np.abs(O.merge_partials(parts) - whole)) < 1e-12
        nb, db = p["q_lat"].shape[2], p["q_lat"].shape[3]
        y = sum(np.einsum("inj,ij->in", p["w_v"][:, :, b * db:(b + 1) * db], whole[:, b, :]) for b in range(nb))
        assert rel(p["alpha"] * y, sdpa_reference(p)[beta]) < 1e-12


def test_linearity_in_alpha_and_wv():
    p = rand_problem(15)
    y = absorbed(p)
    assert rel(absorbed(p, alpha=2.5 * p["alpha"]), 2.5 * y) < 1e-13
    assert rel(absorbed(p, w_v=-0.75 * p["w_v"]), -0.75 * y) < 1e-13


def test_empty_context_rejected():
    p = rand_problem(16, lens=(3, 0))
    with pytest.raises(ValueError):
        absorbed(p)


def test_large_logits_stable():
    """Max-shifted softmax: huge logits give the one-hot limit, not NaN."""
    p = rand_problem(17, lens=(5, 5))
    p["sm_scale"] = 1e4
    y = absorbed(p)
    assert np.all(np.isfinite(y))
    beta, i, b = 0, 1, 2
    db = p["q_lat"].shape[3]
    z = [p["q_lat"][beta, i, b] @ p["kv_lat"][beta, s, b * db:(b + 1) * db] + p["q_rope"][beta, i] @ p["kv_rope"][beta, s]
         for s in range(5)]
    s_star = int(np.argmax(z))
    o = O.branch_partials(p["q_lat"], p["q_rope"], p["kv_lat"], p["kv_rope"], beta, 0, 5, p["sm_scale"])
    u = O.merge_partials([o])
    assert np.max(np.abs(u[i, b] - p["kv_lat"][beta, s_star, b * db:(b + 1) * db])) < 1e-12


# ---- paged cache -------------------------------------------------------------------------

def test_paged_gather_by_hand():
    rng = np.random.default_rng(18)
    ps, P, R = 4, 9, 5
    pool = rng.standard_normal((P, ps, R))
    table = np.array([[3, 7, 0, -1], [8, 1, 5, 2]])
    lens = [10, 13]
    rows = O.paged_gather(pool, table, lens, ps)
    flat = pool.reshape(P * ps, R)
    for beta in range(2):
        idx = [table[beta][s // ps] * ps + s % ps for s in range(lens[beta])]
        assert np.array_equal(rows[beta, :lens[beta]], flat[idx])
    assert np.all(rows[0, 10:] == 0)


def test_paged_decode_equals_contiguous():
    p = rand_problem(19, lens=(13, 6))
    ps = 4
    B, Lmax = 2, 13
    R = p["kv_lat"].shape[2] + p["kv_rope"].shape[2]
    rows = np.concatenate([p["kv_lat"], p["kv_rope"]], axis=2)
    npages = [4, 2]
    perm = np.random.default_rng(2).permutation(6)
    pool = np.zeros((6, ps, R))
    table = np.full((B, 4), -1)
    off = 0
    for beta in range(B):
        for j in range(npages[beta]):
            pid = perm[off + j]
            table[beta, j] = pid
            seg = rows[beta, j * ps:(j + 1) * ps]
            pool[pid, :seg.shape[0]] = seg
        off += npages[beta]
    dc = p["kv_lat"].shape[2]
    y = O.mlra_decode_paged(p["q_lat"], p["q_rope"], pool, table, p["seq_lens"], ps, dc, p["w_v"],
                            p["sm_scale"], p["alpha"])
    assert rel(y, absorbed(p)) < 1e-14


# ---- golden fixtures ---------------------------------------------------------------------

def test_golden_tp_load_formula():
    """Per-device load per token under 4-way TP ([MLRA] §3.2): MLRA-4 d_k^R + d_h/4,
    MLA d_k^R + d_h; at the Qwen3-32B widths (d_h = 128, d_k^R = 32)."""
    from rank_latent_kv_amd.roofline import tp_per_device_load
    with open(os.path.join(GOLDEN, "tp_load_qwen3_32b.json")) as f:
        g = json.load(f)
    got = tp_per_device_load(g["head_dim"], g["rope_dim"], g["ways"])
    assert got["mlra"] == g["mlra_elements_per_token"]
    assert got["mla"] == g["mla_elements_per_token"]


def test_golden_tiny_f32_regression():
    """Oracle output on the tiny fp32 workload, stored by tests/golden/make_golden.py
    (which calls only the oracle and the input generator)."""
    from rank_latent_kv_amd.workloads import PRESETS, make_inputs
    w = PRESETS["tiny_f32"]
    inp = make_inputs(w)
    kv = inp["kv"].double().numpy()
    dc = w.latent_dim
    y = O.mlra_decode_absorbed(inp["q_lat"].double().numpy(), inp["q_rope"].double().numpy(), kv[:, :, :dc],
                               kv[:, :, dc:], inp["seq_lens"].numpy(), inp["w_v"].double().numpy(),
                               w.sm_scale, w.alpha)
    g = np.load(os.path.join(GOLDEN, "tiny_f32_y.npy"))
    assert np.max(np.abs(y - g)) < 1e-12


# ---- planted mistakes: each mutant must fail at least one pin ------------------------------

def _mutant(kind):
    def f(q_lat, q_rope, kv_lat, kv_rope, seq_lens, w_v, sm_scale, alpha):
        B, h, nb, db = q_lat.shape
        y = np.zeros((B, h, w_v.shape[1]))
        for beta in range(B):
            L = int(seq_lens[beta])
            C = kv_lat[beta, :L].reshape(L, nb, db)
            KR = kv_rope[beta, :L]
            rope = q_rope[beta] @ KR.T
            if kind == "drop_rope":
                rope = 0 * rope
            if kind == "rope_sign":
                rope = -rope
            for b in range(nb):
                cb = C[:, b, :]
                if kind == "strided_branch":
                    cb = kv_lat[beta, :L, b::nb]
                z = sm_scale * (q_lat[beta, :, b, :] @ cb.T + rope)
                if kind == "no_scale":
                    z = z / sm_scale
                if kind == "softmax_over_heads":
                    e = np.exp(z - z.max(axis=0, keepdims=True))
                    pr = e / e.sum(axis=0, keepdims=True)
                else:
                    e = np.exp(z - z.max(axis=1, keepdims=True))
                    pr = e / e.sum(axis=1, keepdims=True)
                if kind == "shared_softmax":
                    continue
                u = pr @ cb
                bw = (b + 1) % nb if kind == "wrong_wv_block" else b
                Wb = w_v[:, :, bw * db:(bw + 1) * db]
                if kind == "transposed_wv":          # W^V_{i,b} applied transposed (square blocks)
                    Wb = Wb.transpose(0, 2, 1)
                y[beta] += np.einsum("inj,ij->in", Wb, u)
            if kind == "shared_softmax":            # one softmax over every branch's logits of a head
                zs = np.concatenate([sm_scale * (q_lat[beta, :, b, :] @ C[:, b, :].T + rope) for b in range(nb)], 1)
                e = np.exp(zs - zs.max(axis=1, keepdims=True))
                pr = e / e.sum(axis=1, keepdims=True)
                for b in range(nb):
                    u = pr[:, b * L:(b + 1) * L] @ C[:, b, :]
                    y[beta] += np.einsum("inj,ij->in", w_v[:, :, b * db:(b + 1) * db], u)
        a = 1.0 if kind == "no_alpha" else alpha
        return a * y
    return f


@pytest.mark.parametrize("kind", ["drop_rope", "rope_sign", "strided_branch", "no_scale",
                                  "softmax_over_heads", "wrong_wv_block", "no_alpha", "shared_softmax",
                                  "transposed_wv"])
def test_planted_mistakes_are_caught(kind):
    # square W^V blocks (d_h = d_b) so that the transposed-W^V mutant is well formed
    p = rand_problem(20, B=2, h=3, nb=4, db=4, dr=2, dh=4, lens=(6, 5))
    mutant = _mutant(kind)
    y = mutant(p["q_lat"], p["q_rope"], p["kv_lat"], p["kv_rope"], p["seq_lens"], p["w_v"], p["sm_scale"],
               p["alpha"])
    ref_sdpa = sdpa_reference(p)
    ref_bf = O.mlra_decode_bruteforce(p["q_lat"], p["q_rope"], p["kv_lat"], p["kv_rope"], p["seq_lens"],
                                      p["w_v"], p["sm_scale"], p["alpha"])
    assert rel(y, ref_sdpa) > 1e-3 or rel(y, ref_bf) > 1e-3
    # and the oracle itself passes both
    assert rel(absorbed(p), ref_sdpa) < 1e-12 and rel(absorbed(p), ref_bf) < 1e-12


def test_block_identity():
    """Branch slicing ([MLRA] §二, reading A5): with branch b owning latent columns
    [b*d_b, (b+1)*d_b), the branch dot products q~_b . c_b sum to the full-width q~ . c; the
    oracle run with the whole latent as one branch is MLA decode (which never slices), and
    with four branches (independent softmaxes) it is not."""
    p = rand_problem(23, B=2, h=3, nb=4, db=5, dr=3, dh=7, lens=(9, 6))
    B, h, nb, db = p["q_lat"].shape
    dc = nb * db
    z_blocks = np.einsum("bhnd,bsnd->bhs", p["q_lat"], p["kv_lat"].reshape(B, -1, nb, db))
    z_full = np.einsum("bhc,bsc->bhs", p["q_lat"].reshape(B, h, dc), p["kv_lat"])
    assert np.max(np.abs(z_blocks - z_full)) < 1e-12
    y_mla = O.mla_decode(p["q_lat"].reshape(B, h, 1, dc), p["q_rope"], p["kv_lat"], p["kv_rope"], p["seq_lens"],
                         p["w_v"], p["sm_scale"], p["alpha"])
    # MLA over the full latent == per-branch attention only when there is one branch
    one = O.mlra_decode_absorbed(p["q_lat"].reshape(B, h, 1, dc), p["q_rope"], p["kv_lat"], p["kv_rope"],
                                 p["seq_lens"], p["w_v"], p["sm_scale"], p["alpha"])
    assert rel(one, y_mla) < 1e-12
    assert rel(absorbed(p), y_mla) > 1e-3


def test_bruteforce_on_tiny_f32_workload():
    """The tiny fp32 workload (B=1, h=8, 4 branches of 16, d_R=16, L=256) end to end
    against the scalar brute force."""
    from rank_latent_kv_amd.workloads import PRESETS, make_inputs
    w = PRESETS["tiny_f32"]
    inp = make_inputs(w)
    kv = inp["kv"].double().numpy()
    dc = w.latent_dim
    args = (inp["q_lat"].double().numpy(), inp["q_rope"].double().numpy(), kv[:, :, :dc], kv[:, :, dc:],
            inp["seq_lens"].numpy(), inp["w_v"].double().numpy(), w.sm_scale, w.alpha)
    assert rel(O.mlra_decode_absorbed(*args), O.mlra_decode_bruteforce(*args)) < 1e-12


# ---- the step before attention: RoPE rotation and query absorption ----------------------------

def test_rope_rotation_is_complex_multiplication():
    """Pair (x_2j, x_2j+1) at position m equals (x_2j + i x_2j+1) * exp(i m theta_j) with
    theta_j = 10000^(-2j/d_R), computed here with numpy complex arithmetic."""
    rng = np.random.default_rng(21)
    dr, B = 8, 5
    x = rng.standard_normal((B, 3, dr))
    pos = np.array([0, 1, 7, 1000, 123457])
    got = O.rope_rotate(x, pos)
    theta = np.array([10000.0 ** (-2.0 * j / dr) for j in range(dr // 2)])
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * pos[:, None, None] * theta[None, None, :])
    assert np.allclose(got[..., 0::2], z.real, atol=1e-12)
    assert np.allclose(got[..., 1::2], z.imag, atol=1e-12)


def test_rope_frequencies_and_identity():
    ang = O.rope_angles([1], 32)[0]
    assert ang[0] == 1.0 and math.isclose(ang[1], 10.0 ** -0.25, rel_tol=1e-14)
    assert math.isclose(ang[15], 10000.0 ** (-30.0 / 32.0), rel_tol=1e-14)
    x = np.random.default_rng(2).standard_normal((3, 2, 32))
    assert np.array_equal(O.rope_rotate(x, [0, 0, 0]), x)


def test_rope_scores_depend_on_relative_position_only():
    """rot(q, m) . rot(k, n) depends on m - n alone, and each pair keeps its length."""
    rng = np.random.default_rng(22)
    q, k = rng.standard_normal((1, 16)), rng.standard_normal((1, 16))
    def score(m, n):
        return float(np.sum(O.rope_rotate(q, [m]) * O.rope_rotate(k, [n])))
    for m, n in [(5, 2), (1003, 1000), (70000, 69997)]:
        assert math.isclose(score(m, n), score(3, 0), rel_tol=1e-9, abs_tol=1e-9)
    r = O.rope_rotate(q, [12345])
    assert np.allclose(r[..., 0::2] ** 2 + r[..., 1::2] ** 2, q[..., 0::2] ** 2 + q[..., 1::2] ** 2)


def test_absorbed_query_scores_like_the_up_projected_key():
    """q~_i . c == q^N_i . (W^UK_i c) for random latents c (a transposed W fails this)."""
    rng = np.random.default_rng(23)
    B, h, dh, nb, db = 2, 3, 12, 4, 2
    dc = nb * db
    q_nope = rng.standard_normal((B, h, dh))
    w = rng.standard_normal((h, dh, dc))                 # W^UK_i: latent -> key
    q_lat = O.absorb_query(q_nope, np.transpose(w, (0, 2, 1)), nb)
    assert q_lat.shape == (B, h, nb, db)
    c = rng.standard_normal((4, dc))
    for b in range(B):
        for i in range(h):
            lhs = q_lat[b, i].reshape(dc) @ c.T
            rhs = q_nope[b, i] @ (w[i] @ c.T)
            assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_prepared_decode_equals_attention_on_rotated_keys():
    """End to end: keys stored rotated by the prepare step, the query rotated to its own
    position, then decoded, equals attention written directly on un-rotated keys with
    the rotation applied inside each score (materialised per-branch keys)."""
    rng = np.random.default_rng(24)
    B, h, nb, db, dr, dh = 2, 2, 2, 4, 6, 8
    dc = nb * db
    L = 9
    c_all = rng.standard_normal((B, L, dc))
    kpe_raw = rng.standard_normal((B, L, dr))
    q_nope = rng.standard_normal((B, h, dh))
    q_pe = rng.standard_normal((B, h, dr))
    w = rng.standard_normal((h, dh, dc)) / 3.0
    w_v = rng.standard_normal((h, dh, dc)) / 3.0
    pos = np.array([L - 1, L - 1])
    # cache rows 0 .. L-2 already rotated; the prepare step writes row L-1
    kv = np.zeros((B, L, dc + dr))
    for s in range(L - 1):
        kv[:, s, :dc] = c_all[:, s]
        kv[:, s, dc:] = O.rope_rotate(kpe_raw[:, s], [s, s])
    q_lat, q_rope, row = O.prepare_decode(q_nope, q_pe, np.transpose(w, (0, 2, 1)), nb,
                                          c_all[:, L - 1], kpe_raw[:, L - 1], pos)
    kv[:, L - 1] = row
    lens = np.array([L, L])
    y = O.mlra_decode_absorbed(q_lat, q_rope, kv[:, :, :dc], kv[:, :, dc:], lens, w_v, 0.3, 0.5)
    ref = np.zeros((B, h, dh))
    for b in range(B):
        for i in range(h):
            for br in range(nb):
                sl = slice(br * db, (br + 1) * db)
                z = np.empty(L)
                for s in range(L):
                    k_nope = w[i][:, sl] @ c_all[b, s, sl]                     # materialised key
                    qr = O.rope_rotate(q_pe[b:b + 1, i], [L - 1])[0]
                    kr = O.rope_rotate(kpe_raw[b:b + 1, s], [s])[0]
                    z[s] = 0.3 * (q_nope[b, i] @ k_nope + qr @ kr)
                p = np.exp(z - z.max())
                p /= p.sum()
                u = p @ c_all[b, :, sl]
                ref[b, i] += w_v[i][:, sl] @ u
    assert np.allclose(y, 0.5 * ref, rtol=1e-10, atol=1e-12)
