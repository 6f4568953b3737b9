"""The attention kernel's split records, read back from the workspace (a white-box check).

With several branches, or one branch over four phases (MLA), the kernel stores each split's
unnormalised output o in fp16, scaled
by 2^-e where l = f 2^e with f in [0.5, 1), and adds e to m: every record it writes must then
hold l in [0.5, 1), a finite m, and |o| <= l * max|c| (o is an l-weighted mean of cache
values). The workspace starts as NaN bytes, so a record left unwritten, or written with
stale lanes, shows. The benchmark workloads at full size, all sequences full length (every
split holds tokens)."""
import numpy as np
import pytest
import torch

import rank_latent_kv_amd as R
from rank_latent_kv_amd.workloads import PRESETS, make_inputs
from gpu_helpers import DEV, f64, oracle_decode, row_rel_err, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("preset", ["mlra4_b16_l32k", "mlra2_b16_l32k", "mla_b16_l32k"])
def test_every_fp16_record_is_a_finite_in_range_softmax_state(preset):
    w = PRESETS[preset]
    inp = make_inputs(w)
    assert int(inp["seq_lens"].min()) == w.seq_len
    d = to_dev(inp)
    dc = w.latent_dim
    kv = d["kv"]
    kw = dict(sm_scale=w.sm_scale, alpha=w.alpha, seq_lens_host=inp["seq_lens"].to(torch.int32).contiguous())
    args = R.make_args(d["q_lat"], d["q_rope"], kv[..., :dc], kv[..., dc:], d["seq_lens"], d["w_v"], **kw)
    plan = R.plan(args)
    assert plan["kernel"] == "mfma"
    n = R.workspace_size(args)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device=DEV)   # NaN in fp16 and fp32
    say(f"records of {preset}, {plan['num_splits']} splits")
    fn = R.mla_decode if w.branches == 1 else R.decode
    y = fn(d["q_lat"], d["q_rope"], kv[..., :dc], kv[..., dc:], d["seq_lens"], d["w_v"], workspace=ws, **kw)
    torch.cuda.synchronize()

    B, S, H, NB, DB = w.batch, plan["num_splits"], w.heads, w.branches, w.branch_dim
    recs = B * S * H * NB
    o_bytes = -(-recs * DB * 2 // 256) * 256
    assert n == o_bytes + -(-recs * 2 * 4 // 256) * 256
    o = ws[:recs * DB * 2].view(torch.float16).float().cpu().numpy().reshape(B, S, H, NB, DB)
    ml = ws[o_bytes:o_bytes + recs * 8].view(torch.float32).cpu().numpy().reshape(B, S, H, NB, 2)
    m, l = ml[..., 0], ml[..., 1]
    assert np.isfinite(m).all() and np.isfinite(l).all()
    assert (l >= 0.5).all() and (l < 1.0).all(), (l.min(), l.max())
    assert np.isfinite(o).all()
    cmax = float(kv[..., :dc].abs().max())
    bound = l[..., None] * cmax * (1 + 2.0 ** -10) + 2.0 ** -24   # fp16 rounding of o
    assert (np.abs(o) <= bound).all(), float((np.abs(o) / bound).max())

    yy = f64(y)
    assert np.isfinite(yy).all()
    seqs = [0, w.batch - 1]
    assert row_rel_err(yy[seqs], oracle_decode(w, inp, seqs=seqs)) <= 1e-2
