"""GPU parity of the step before a decode call (mlra_decode_prepare): query absorption,
the RoPE query rotated to the new token's position, and the new cache row, each
against the CPU oracle on the same seeded values; then prepare followed by decode
against the oracle end to end.

Tolerances: bf16 outputs are rounded once from fp32 arithmetic, so the absorbed query
is checked per row to 1e-2 relative (as the decode) and the rotated vectors elementwise
to 2^-7 of the row's largest magnitude; fp32 to 1e-5. The latent copy is bit-exact.
"""
import numpy as np
import pytest
import torch

import rank_latent_kv_amd as R
from oracle import mlra_oracle as O

from gpu_helpers import DEV, f64, row_rel_err, say

pytestmark = pytest.mark.gpu


def inputs(B, h, nb, db, dr, dh, seed, dtype=torch.bfloat16):
    rng = np.random.default_rng(seed)
    dc = nb * db
    f = lambda *shape, s=1.0: torch.from_numpy((rng.standard_normal(shape) * s).astype(np.float32)).to(dtype)
    return dict(q_nope=f(B, h, dh), q_pe=f(B, h, dr), w_uk_t=f(h, dc, dh, s=dh ** -0.5),
                c_new=f(B, dc, s=0.125), k_pe_new=f(B, dr, s=0.125))


def run_prepare(d, positions, kv, dc, nb, **kw):
    dd = {k: v.to(DEV) for k, v in d.items()}
    pos = torch.tensor(positions, dtype=torch.int32)
    q_lat, q_rope = R.prepare(dd["q_nope"], dd["q_pe"], dd["w_uk_t"], dd["c_new"], dd["k_pe_new"], pos.to(DEV),
                              kv[..., :dc], kv[..., dc:], num_branches=nb, positions_host=pos, **kw)
    torch.cuda.synchronize()
    return q_lat, q_rope


def rot_err(got, ref):
    """max |got - ref| / max |ref| per row, rows along the last axis."""
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)
    return float(np.max(num / den))


@pytest.mark.parametrize("B", [16, 20])
def test_prepare_bf16_mfma_path(B):
    h, nb, db, dr, dh = 64, 4, 32, 32, 128
    dc = nb * db
    d = inputs(B, h, nb, db, dr, dh, seed=31 + B)
    L = 64
    kv = torch.zeros((B, L, dc + dr), dtype=torch.bfloat16, device=DEV)
    positions = [(7 * b) % L for b in range(B)]
    say(f"prepare bf16 B={B}")
    q_lat, q_rope = run_prepare(d, positions, kv, dc, nb)
    ql_ref, qr_ref, row_ref = O.prepare_decode(f64(d["q_nope"]), f64(d["q_pe"]), f64(d["w_uk_t"]), nb,
                                               f64(d["c_new"]), f64(d["k_pe_new"]), positions)
    err = row_rel_err(f64(q_lat).reshape(B, h, dc), ql_ref.reshape(B, h, dc))
    say(f"absorbed query row rel err {err:.3e}")
    assert err <= 1e-2
    assert rot_err(f64(q_rope), qr_ref) <= 2 ** -7
    kvh = kv.cpu()
    for b in range(B):
        m = positions[b]
        assert torch.equal(kvh[b, m, :dc], d["c_new"][b])
        assert rot_err(f64(kvh[b, m, dc:])[None], row_ref[b:b + 1, dc:]) <= 2 ** -7
        others = torch.cat([kvh[b, :m], kvh[b, m + 1:]])
        assert torch.all(others == 0)


def test_prepare_long_positions():
    """Angles up to 2^20 rad keep their accuracy (fp64 angle, sine and cosine). The
    rows go through a page table whose only valid entries are the new tokens' pages."""
    B, h, nb, db, dr, dh = 4, 16, 1, 32, 32, 64
    dc = nb * db
    d = inputs(B, h, nb, db, dr, dh, seed=37)
    positions = [0, 1, 65535, (1 << 20) - 1]
    ps = 64
    pt = torch.full((B, (1 << 20) // ps), -1, dtype=torch.int32)
    for b, m in enumerate(positions):
        pt[b, m // ps] = b
    pool = torch.zeros((B, ps, dc + dr), dtype=torch.bfloat16, device=DEV)
    say("prepare long positions")
    q_lat, q_rope = run_prepare(d, positions, pool.view(-1, dc + dr)[None], dc, nb, page_table=pt.to(DEV),
                                page_size=ps, num_pages=B)
    _, qr_ref, row_ref = O.prepare_decode(f64(d["q_nope"]), f64(d["q_pe"]), f64(d["w_uk_t"]), nb,
                                          f64(d["c_new"]), f64(d["k_pe_new"]), positions)
    assert rot_err(f64(q_rope), qr_ref) <= 2 ** -7
    flat = pool.view(-1, dc + dr).cpu()
    for b, m in enumerate(positions):
        r = b * ps + m % ps
        assert torch.equal(flat[r, :dc], d["c_new"][b])
        assert rot_err(f64(flat[r, dc:])[None], row_ref[b:b + 1, dc:]) <= 2 ** -7


def test_prepare_fp32_valu_path():
    B, h, nb, db, dr, dh = 3, 4, 2, 8, 16, 24
    dc = nb * db
    d = inputs(B, h, nb, db, dr, dh, seed=41, dtype=torch.float32)
    L = 12
    kv = torch.zeros((B, L, dc + dr), dtype=torch.float32, device=DEV)
    positions = [0, 5, 11]
    say("prepare fp32")
    q_lat, q_rope = run_prepare(d, positions, kv, dc, nb)
    ql_ref, qr_ref, row_ref = O.prepare_decode(f64(d["q_nope"]), f64(d["q_pe"]), f64(d["w_uk_t"]), nb,
                                               f64(d["c_new"]), f64(d["k_pe_new"]), positions)
    assert row_rel_err(f64(q_lat).reshape(B, h, dc), ql_ref.reshape(B, h, dc)) <= 1e-5
    assert rot_err(f64(q_rope), qr_ref) <= 1e-5
    kvh = kv.cpu()
    for b in range(B):
        assert torch.equal(kvh[b, positions[b], :dc], d["c_new"][b])
        assert rot_err(f64(kvh[b, positions[b], dc:])[None], row_ref[b:b + 1, dc:]) <= 1e-5


def test_prepare_paged_and_bad_page():
    B, h, nb, db, dr, dh = 3, 64, 4, 32, 32, 128
    dc = nb * db
    d = inputs(B, h, nb, db, dr, dh, seed=43)
    ps, P = 64, 8
    pool = torch.zeros((P, ps, dc + dr), dtype=torch.bfloat16, device=DEV)
    pt = torch.tensor([[3, 5], [0, 7], [1, 99]], dtype=torch.int32)      # entry 99 is outside the pool
    positions = [70, 3, 64]                                             # sequence 2 uses page 99
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    say("prepare paged")
    run_prepare(d, positions, pool.view(-1, dc + dr)[None], dc, nb, page_table=pt.to(DEV), page_size=ps,
                num_pages=P, error_flags=flags)
    assert int(flags.item()) & R.FLAG_BAD_PAGE
    flat = pool.view(-1, dc + dr).cpu()
    _, _, row_ref = O.prepare_decode(f64(d["q_nope"]), f64(d["q_pe"]), f64(d["w_uk_t"]), nb,
                                     f64(d["c_new"]), f64(d["k_pe_new"]), positions)
    written = {0: 5 * ps + 70 % ps, 1: 0 * ps + 3}
    for b, r in written.items():
        assert torch.equal(flat[r, :dc], d["c_new"][b])
        assert rot_err(f64(flat[r, dc:])[None], row_ref[b:b + 1, dc:]) <= 2 ** -7
    assert int((flat != 0).any(dim=1).sum()) == len(written)


def test_prepare_then_decode_matches_oracle():
    """The new token's absorbed query, rotated query and cache row, then the decode over
    the whole context including that row, against the oracle."""
    B, h, nb, db, dr, dh = 3, 64, 4, 32, 32, 128
    dc = nb * db
    lens = [1500, 777, 64]
    rng = np.random.default_rng(47)
    d = inputs(B, h, nb, db, dr, dh, seed=47)
    L = max(lens)
    kv_np = (rng.standard_normal((B, L, dc + dr)) * 0.125).astype(np.float32)
    kv = torch.from_numpy(kv_np).to(torch.bfloat16)
    w_v = torch.from_numpy((rng.standard_normal((h, dh, dc)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    positions = [n - 1 for n in lens]
    kv_d = kv.to(DEV)
    say("prepare then decode")
    q_lat, q_rope = run_prepare(d, positions, kv_d, dc, nb)
    seq_lens = torch.tensor(lens, dtype=torch.int32)
    y = R.decode(q_lat, q_rope, kv_d[..., :dc], kv_d[..., dc:], seq_lens.to(DEV), w_v.to(DEV),
                 sm_scale=0.125, alpha=0.5, seq_lens_host=seq_lens)
    torch.cuda.synchronize()
    ql_ref, qr_ref, row_ref = O.prepare_decode(f64(d["q_nope"]), f64(d["q_pe"]), f64(d["w_uk_t"]), nb,
                                               f64(d["c_new"]), f64(d["k_pe_new"]), positions)
    kv_ref = f64(kv)
    for b in range(B):
        kv_ref[b, positions[b]] = row_ref[b]
    ref = O.mlra_decode_absorbed(ql_ref, qr_ref, kv_ref[:, :, :dc], kv_ref[:, :, dc:], np.array(lens), f64(w_v),
                                 0.125, 0.5)
    err = row_rel_err(f64(y), ref)
    say(f"prepare + decode row rel err {err:.3e}")
    assert err <= 1e-2
