"""Stray writes: the output and the workspace sit inside larger buffers whose surrounding
bytes hold a canary pattern; after a decode call every canary byte must be unchanged and the
output must still match the oracle. These are correct kernels checked for writes outside
their buffers (an out-of-bounds store by the attention, merge or prepare kernels would land
in a guard)."""
import numpy as np
import pytest
import torch

import rank_latent_kv_amd as R
from rank_latent_kv_amd.workloads import PRESETS, make_inputs
from gpu_helpers import DEV, f64, oracle_decode, row_rel_err, say

pytestmark = pytest.mark.gpu

GUARD = 64 * 1024          # canary bytes on each side
CANARY = 0xA5


def _guarded(nbytes: int):
    """A uint8 buffer of GUARD + nbytes + GUARD canary bytes and the middle region's offset
    (GUARD is a multiple of 256, so the region keeps the allocator's alignment)."""
    buf = torch.full((GUARD + nbytes + GUARD,), CANARY, dtype=torch.uint8, device=DEV)
    return buf, GUARD


def _guards_intact(buf: torch.Tensor, nbytes: int) -> bool:
    head = buf[:GUARD]
    tail = buf[GUARD + nbytes:]
    return bool(torch.all(head == CANARY)) and bool(torch.all(tail == CANARY))


@pytest.mark.parametrize("preset,lens,out_dtype,num_splits", [
    ("mlra4_b16_l32k", [9000, 300, 5000, 2100], torch.bfloat16, 0),
    ("mlra4_b16_l32k", [4096, 4096], torch.float32, 7),
    ("mla_b16_l32k", [6000, 1500, 3333], torch.bfloat16, 0),
    ("mlra4_paged_b4_l64k_128k", [5000, 700, 2048], torch.bfloat16, 0),
    ("mlra4_tp_shard_b64_l64k", [3000, 100, 4097, 64], torch.bfloat16, 0),
    ("tiny_f32", [256], torch.float32, 3),
])
def test_no_write_outside_output_and_workspace(preset, lens, out_dtype, num_splits):
    w = PRESETS[preset].replace(batch=len(lens))
    inp = make_inputs(w, seq_lens=lens)
    d = {k: v.to(DEV) for k, v in inp.items()}
    dc = w.latent_dim
    lens_host = inp["seq_lens"].to(torch.int32).contiguous()
    kw = dict(sm_scale=w.sm_scale, alpha=w.alpha, seq_lens_host=lens_host, num_splits=num_splits)
    if w.paged:
        pool = d["pool"]
        kv_lat, kv_rope = pool[..., :dc], pool[..., dc:]
        kw.update(page_table=d["page_table"], page_size=w.page_size, num_pages=pool.shape[0],
                  row_stride=pool.shape[-1], max_seq_len=max(lens))
    else:
        kv_lat, kv_rope = d["kv"][..., :dc], d["kv"][..., dc:]
    esz = torch.tensor([], dtype=out_dtype).element_size()
    out_bytes = w.batch * w.heads * w.head_dim * esz
    obuf, off = _guarded(out_bytes)
    out = obuf[off:off + out_bytes].view(out_dtype).view(w.batch, w.heads, w.head_dim)
    args = R.make_args(d["q_lat"], d["q_rope"], kv_lat, kv_rope, d["seq_lens"], d["w_v"], out=out, **kw)
    ws_bytes = R.workspace_size(args)
    wbuf, woff = _guarded(ws_bytes)
    ws = wbuf[woff:woff + ws_bytes]
    say(f"guard bytes: {preset} lens {lens} out {out_dtype} splits {num_splits}")
    y = R.decode(d["q_lat"], d["q_rope"], kv_lat, kv_rope, d["seq_lens"], d["w_v"], out=out, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert y.data_ptr() == out.data_ptr()
    assert _guards_intact(obuf, out_bytes), "a kernel wrote outside the output"
    assert _guards_intact(wbuf, ws_bytes), "a kernel wrote outside the workspace"
    tol = 1e-5 if w.dtype == "f32" else 1e-2
    assert row_rel_err(f64(y), oracle_decode(w, inp)) <= tol


def test_prepare_writes_only_its_rows():
    """The prepare step writes q_lat, q_rope and one cache row per sequence: the rest of a
    guarded cache is unchanged byte for byte."""
    w = PRESETS["mlra4_b16_l32k"].replace(batch=3)
    B, H, dc, dr, dh, L = 3, w.heads, w.latent_dim, w.rope_dim, w.head_dim, 700
    g = torch.Generator().manual_seed(5)
    bf = lambda *s: torch.randn(s, generator=g).to(torch.bfloat16).to(DEV)
    kv = torch.full((B, L, dc + dr), 3.0, dtype=torch.bfloat16, device=DEV)
    before = kv.clone()
    q_lat = torch.empty(B, H, w.branches, w.branch_dim, dtype=torch.bfloat16, device=DEV)
    q_rope = torch.empty(B, H, dr, dtype=torch.bfloat16, device=DEV)
    pos = torch.tensor([0, 350, 699], dtype=torch.int32)
    say("guard bytes: prepare")
    R.prepare(bf(B, H, dh), bf(B, H, dr), bf(H, dc, dh), bf(B, dc), bf(B, dr), pos.to(DEV), kv[..., :dc], kv[..., dc:],
              num_branches=w.branches, q_lat=q_lat, q_rope=q_rope, positions_host=pos)
    torch.cuda.synchronize()
    changed = {tuple(r) for r in (kv != before).any(dim=-1).nonzero().tolist()}
    assert changed and changed <= {(0, 0), (1, 350), (2, 699)}
