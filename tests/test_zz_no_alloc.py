"""The allocation-free decode entry point (mlra_decode_noalloc) against mlra_decode on the same
inputs: the same kernels with the split state in the library's own device array, so the
outputs must agree bit for bit, call after call, including a smaller call right after a
larger one (the array keeps the previous call's records), and both stay within the oracle's
tolerance. A call whose split state exceeds the array is refused on the host."""
import numpy as np
import pytest
import torch

import rank_latent_kv_amd as R
from rank_latent_kv_amd.workloads import PRESETS, make_inputs
from gpu_helpers import DEV, f64, gpu_decode, oracle_decode, row_rel_err, say

TOL_BF16 = 1e-2

pytestmark = pytest.mark.gpu


def _noalloc(w, inp, out):
    d = {k: v.to(DEV) for k, v in inp.items()}
    dc = w.latent_dim
    lens_host = inp["seq_lens"].to(torch.int32).contiguous()
    if w.paged:
        pool = d["pool"]
        y = R.decode_noalloc(d["q_lat"], d["q_rope"], pool[..., :dc], pool[..., dc:], d["seq_lens"], d["w_v"],
                             sm_scale=w.sm_scale, alpha=w.alpha, out=out, page_table=d["page_table"],
                             page_size=w.page_size, num_pages=pool.shape[0], row_stride=pool.shape[-1],
                             max_seq_len=int(inp["seq_lens"].max()), seq_lens_host=lens_host)
    else:
        kv = d["kv"]
        y = R.decode_noalloc(d["q_lat"], d["q_rope"], kv[..., :dc], kv[..., dc:], d["seq_lens"], d["w_v"],
                             sm_scale=w.sm_scale, alpha=w.alpha, out=out, seq_lens_host=lens_host)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("preset,lens_list", [
    ("mlra4_b16_l32k", ([9000, 4000, 700, 12000], [900, 300])),
    ("mla_b16_l32k", ([5000, 3000, 800], [1000])),
    ("mlra4_paged_b4_l64k_128k", ([7000, 2000], [500, 1200])),
])
def test_noalloc_matches_decode_call_after_call(preset, lens_list):
    for lens in lens_list:   # the second call is smaller than the first
        w = PRESETS[preset].replace(batch=len(lens))
        inp = make_inputs(w, seq_lens=lens)
        say(f"noalloc vs decode: {preset} lens {lens}")
        ref = gpu_decode(w, inp)
        out = torch.full_like(ref, float("nan"))
        y = _noalloc(w, inp, out)
        assert y.data_ptr() == out.data_ptr()
        assert torch.equal(y, ref)
        assert row_rel_err(f64(y), oracle_decode(w, inp)) <= TOL_BF16


def test_noalloc_refuses_split_state_beyond_its_array():
    """256 sequences with 64 splits each need 256*64*64*4*34*4 bytes of split state, beyond the
    16 MiB array: refused before anything is enqueued, and the output is untouched."""
    w = PRESETS["mlra4_b16_l32k"].replace(batch=256)
    B, H, NB, DB, DR = 256, 64, 4, 32, 32
    q_lat = torch.zeros(B, H, NB, DB, dtype=torch.bfloat16, device=DEV)
    q_rope = torch.zeros(B, H, DR, dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros(B, 8192, NB * DB + DR, dtype=torch.bfloat16, device=DEV)
    lens = torch.full((B,), 8192, dtype=torch.int32, device=DEV)
    w_v = torch.zeros(H, 128, NB * DB, dtype=torch.bfloat16, device=DEV)
    out = torch.full((B, H, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    say("noalloc: oversize split state refused")
    with pytest.raises(R.MlraError) as e:
        R.decode_noalloc(q_lat, q_rope, kv[..., :NB * DB], kv[..., NB * DB:], lens, w_v, sm_scale=w.sm_scale,
                         alpha=w.alpha, out=out, num_splits=64)
    assert e.value.status == R.MLRA_ERR_WORKSPACE and "device array" in str(e.value)
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))


def test_noalloc_under_graph_capture():
    """The caller the entry point exists for: a decode captured into a HIP graph (no device
    allocation is allowed while capturing). The graph is replayed several times, with the
    program's own eager work and a synchronisation between replays, and every replay must
    equal the eager call bit for bit."""
    w = PRESETS["mlra4_b16_l32k"].replace(batch=3)
    lens = [5000, 1200, 3333]
    inp = make_inputs(w, seq_lens=lens)
    d = {k: v.to(DEV) for k, v in inp.items()}
    dc = w.latent_dim
    kv = d["kv"]
    lens_host = inp["seq_lens"].to(torch.int32).contiguous()
    out = torch.empty((w.batch, w.heads, w.head_dim), dtype=torch.bfloat16, device=DEV)

    def call():
        R.decode_noalloc(d["q_lat"], d["q_rope"], kv[..., :dc], kv[..., dc:], d["seq_lens"], d["w_v"],
                         sm_scale=w.sm_scale, alpha=w.alpha, out=out, seq_lens_host=lens_host)

    say("noalloc: eager reference, then capture")
    call()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(4):
        out.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=DEV).sum()     # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"noalloc graph replay {r}")
        assert torch.equal(out, ref), r
        assert bool(torch.isfinite(junk))
    assert row_rel_err(f64(out), oracle_decode(w, inp)) <= TOL_BF16
