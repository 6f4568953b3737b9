"""Shared helpers for the GPU parity tests: move seeded inputs to the device, run
the HIP library through the binding, and run the CPU oracle on the same values."""
from __future__ import annotations

import sys

import numpy as np
import torch

import rank_latent_kv_amd as R
from oracle import mlra_oracle as O

DEV = "cuda:0"


def say(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(inp: dict) -> dict:
    return {k: v.to(DEV) for k, v in inp.items()}


def gpu_decode(w, inp: dict, *, num_splits: int = 0, mla: bool = False, host_lens: bool = True,
               out_dtype=None, seq_lens_dev=None, error_flags=None, max_seq_len=None, workspace=None) -> torch.Tensor:
    d = to_dev(inp)
    dc = w.latent_dim
    lens_host = inp["seq_lens"].to(torch.int32).contiguous() if host_lens else None
    kw = dict(sm_scale=w.sm_scale, alpha=w.alpha, num_splits=num_splits, seq_lens_host=lens_host,
              out_dtype=out_dtype, error_flags=error_flags, workspace=workspace)
    seq_lens = d["seq_lens"] if seq_lens_dev is None else seq_lens_dev
    if w.paged:
        pool = d["pool"]
        kv_lat, kv_rope = pool[..., :dc], pool[..., dc:]
        kw.update(page_table=d["page_table"], page_size=w.page_size, num_pages=pool.shape[0],
                  row_stride=pool.shape[-1],
                  max_seq_len=max_seq_len or int(inp["seq_lens"].max()))
    else:
        kv = d["kv"]
        kv_lat, kv_rope = kv[..., :dc], kv[..., dc:]
        if max_seq_len is not None:
            kw["max_seq_len"] = max_seq_len
    fn = R.mla_decode if mla else R.decode
    y = fn(d["q_lat"], d["q_rope"], kv_lat, kv_rope, seq_lens, d["w_v"], **kw)
    torch.cuda.synchronize()
    return y


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def oracle_decode(w, inp: dict, seqs=None) -> np.ndarray:
    """Absorbed-form oracle on the same (bf16 / fp32) values, for the listed sequences."""
    lens = inp["seq_lens"].numpy()
    seqs = list(range(w.batch)) if seqs is None else list(seqs)
    dc = w.latent_dim
    q_lat = f64(inp["q_lat"][seqs])
    q_rope = f64(inp["q_rope"][seqs])
    w_v = f64(inp["w_v"])
    if w.paged:
        pool = f64(inp["pool"])
        pt = inp["page_table"].numpy()[seqs]
        return O.mlra_decode_paged(q_lat, q_rope, pool, pt, lens[seqs], w.page_size, dc, w_v, w.sm_scale, w.alpha)
    kv = inp["kv"][seqs]
    Lm = int(lens[seqs].max())
    kv = f64(kv[:, :Lm])
    return O.mlra_decode_absorbed(q_lat, q_rope, kv[:, :, :dc], kv[:, :, dc:], lens[seqs], w_v, w.sm_scale, w.alpha)


def row_rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    """max over output rows (sequence, head) of max_j |y - ref| / max_j |ref|."""
    num = np.max(np.abs(y - ref), axis=-1)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)
    return float(np.max(num / den))
