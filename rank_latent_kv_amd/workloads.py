"""Seeded synthetic inputs for MLRA / MLA decode attention.

This module draws random numbers and lays them out; it holds none of the
attention arithmetic. Both sides of every parity check (the HIP library and the
CPU oracle) receive exactly the tensors produced here.

Shapes follow a Qwen3-32B-shaped attention layer (64 query heads, head width
128, RoPE key width 32), the base model the MLRA page ("原生支持张量并行的
多分支低秩注意力MLRA", Table 1) uses for its KV-load comparison. The pages give
no decode inputs, so every value is drawn from a seeded generator:

* cache latents, RoPE keys and absorbed queries ~ N(0, 1) / sqrt(d) with
  d = branch width + RoPE width (the width of one branch score);
* W^V ~ N(0, 0.02**2);
* the tiny fp32 case draws everything from N(0, 1).

Every draw is float32 from ``numpy.random.Generator(PCG64(seed))`` and is then
rounded to the workload's storage type (bfloat16 round-to-nearest-even via
torch, or kept as float32).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Sequence

import numpy as np
import torch

BASE_SEED = 20260303


@dataclasses.dataclass(frozen=True)
class Workload:
    """One decode-attention configuration (one attention layer, one new token per sequence)."""

    name: str
    batch: int
    heads: int
    branches: int          # n_b: latent blocks (4 for MLRA-4, 1 for MLA)
    branch_dim: int        # d_b: width of one latent block
    rope_dim: int          # d_R: width of the shared RoPE key
    head_dim: int          # d_h: output width of W^V per head
    seq_len: Optional[int] = None                 # every sequence has this context length
    seq_len_range: Optional[tuple] = None         # or L ~ U{lo..hi} per sequence (inclusive)
    dtype: str = "bf16"                           # storage / MFMA input type: "bf16" or "f32"
    paged: bool = False
    page_size: int = 64
    sm_scale: float = 0.125
    alpha: float = 0.5
    value_std: Optional[float] = None             # std of cache and queries (None -> 1/sqrt(d_b + d_R))
    wv_std: float = 0.02
    seed_offset: int = 0

    @property
    def latent_dim(self) -> int:
        return self.branches * self.branch_dim

    @property
    def row_dim(self) -> int:
        return self.latent_dim + self.rope_dim

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def std(self) -> float:
        if self.value_std is not None:
            return self.value_std
        return 1.0 / math.sqrt(self.branch_dim + self.rope_dim)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


PRESETS: Dict[str, Workload] = {
    # tiny fp32 MLRA-4, small enough for brute force on the CPU
    "tiny_f32": Workload("tiny_f32", batch=1, heads=8, branches=4, branch_dim=16, rope_dim=16,
                         head_dim=64, seq_len=256, dtype="f32", sm_scale=1.0 / math.sqrt(32.0),
                         alpha=0.5, value_std=1.0, wv_std=1.0, seed_offset=0),
    # Qwen3-32B-shaped MLRA-4, contiguous cache (the headline decode workload)
    "mlra4_b16_l32k": Workload("mlra4_b16_l32k", batch=16, heads=64, branches=4, branch_dim=32,
                               rope_dim=32, head_dim=128, seq_len=32768, sm_scale=1.0 / 8.0,
                               alpha=0.5, seed_offset=1),
    # single-latent MLA at the same shapes (comparison path); same value law as MLRA-4
    "mla_b16_l32k": Workload("mla_b16_l32k", batch=16, heads=64, branches=1, branch_dim=128,
                             rope_dim=32, head_dim=128, seq_len=32768,
                             sm_scale=1.0 / math.sqrt(160.0), alpha=1.0,
                             value_std=1.0 / 8.0, seed_offset=2),
    # MLRA-2: the latent in two 64-wide branches, each head attending over both
    "mlra2_b16_l32k": Workload("mlra2_b16_l32k", batch=16, heads=64, branches=2, branch_dim=64,
                               rope_dim=32, head_dim=128, seq_len=32768,
                               sm_scale=1.0 / math.sqrt(96.0), alpha=1.0 / math.sqrt(2.0),
                               seed_offset=6),
    # long-context MLRA-4 through a scattered 64-token page table
    "mlra4_paged_b4_l64k_128k": Workload("mlra4_paged_b4_l64k_128k", batch=4, heads=64, branches=4,
                                         branch_dim=32, rope_dim=32, head_dim=128,
                                         seq_len_range=(65536, 131072), paged=True, page_size=64,
                                         sm_scale=1.0 / 8.0, alpha=0.5, seed_offset=3),
    # one tensor-parallel rank's share of MLRA-4: one branch, 16 local heads
    "mlra4_tp_shard_b64_l64k": Workload("mlra4_tp_shard_b64_l64k", batch=64, heads=16, branches=1,
                                        branch_dim=32, rope_dim=32, head_dim=128, seq_len=65536,
                                        sm_scale=1.0 / 8.0, alpha=0.5, seed_offset=4),
    # the MLA counterpart of that rank: MLA's single latent cannot be split across tensor-
    # parallel ranks, so a rank with 16 local heads still streams the whole 160-wide row
    "mla_tp_shard_b64_l64k": Workload("mla_tp_shard_b64_l64k", batch=64, heads=16, branches=1,
                                      branch_dim=128, rope_dim=32, head_dim=128, seq_len=65536,
                                      sm_scale=1.0 / math.sqrt(160.0), alpha=1.0,
                                      value_std=1.0 / 8.0, seed_offset=5),
    # the rank of the branch-sharded design: all 64 heads over the one 32-wide latent block it
    # holds, plus the replicated RoPE key (the rank runs the kernel with one branch and applies
    # alpha * W^V of its branch; the ranks' outputs are then summed)
    "mlra4_branch_shard_b64_l64k": Workload("mlra4_branch_shard_b64_l64k", batch=64, heads=64, branches=1,
                                            branch_dim=32, rope_dim=32, head_dim=128, seq_len=65536,
                                            sm_scale=1.0 / 8.0, alpha=0.5, seed_offset=7),
}


def _to_storage(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(f"unknown dtype {dtype}")


def draw_seq_lens(w: Workload, rng: np.random.Generator) -> np.ndarray:
    if w.seq_len is not None:
        return np.full(w.batch, w.seq_len, dtype=np.int32)
    lo, hi = w.seq_len_range
    return rng.integers(lo, hi + 1, size=w.batch, dtype=np.int64).astype(np.int32)


def default_seq_lens(w: Workload, seed: Optional[int] = None) -> np.ndarray:
    """The context lengths make_inputs(w, seed=seed) draws, without drawing the rest."""
    seed = BASE_SEED + w.seed_offset if seed is None else seed
    return draw_seq_lens(w, np.random.Generator(np.random.PCG64(seed)))


def _plant_peaks(rng, q_lat, q_rope, kv_lat, kv_rope, seq_lens, nb, db, gain):
    """Plant strongly aligned cache rows so that a few (head, token) logits dominate.

    Positions sit late in the context and right at both sides of common split
    boundaries (multiples of 512 / 1024 / 2048 tokens), each aligned with a
    randomly chosen head; this stresses the running-max rescaling and the
    cross-split merge.
    """
    B, h = q_lat.shape[0], q_lat.shape[1]
    for beta in range(B):
        L = int(seq_lens[beta])
        cand = {L - 1, L - 2, (3 * L) // 4 + 1, L // 2, L // 2 - 1}
        for m in (512, 1024, 2048):
            k = int(rng.integers(1, max(2, L // m + 1)))
            cand.update({k * m - 1, k * m})
        cand.add(int(rng.integers(0, L)))
        for s in sorted(p for p in cand if 0 <= p < L):
            i = int(rng.integers(0, h))
            kv_lat[beta, s, :] = gain * q_lat[beta, i].reshape(nb * db)
            kv_rope[beta, s, :] = gain * q_rope[beta, i]


def make_inputs(w: Workload, *, seed: Optional[int] = None, seq_lens: Optional[Sequence[int]] = None,
                seq_len: Optional[int] = None, peaked: bool = False, peak_gain: float = 4.0) -> dict:
    """Draw one decode batch for workload ``w``.

    Returns a dict of CPU torch tensors in the storage dtype:
      q_lat  [B, h, n_b, d_b], q_rope [B, h, d_R], w_v [h, d_h, n_b*d_b],
      seq_lens int32 [B];
    contiguous mode: kv [B, L_max, n_b*d_b + d_R] (latent columns first, RoPE key last);
    paged mode: pool [P, page_size, row], page_table int32 [B, max_pages] (-1 padded),
      where P = sum_b ceil(L_b / page_size) and the physical page order is a random
      permutation.
    ``peaked`` draws unscaled N(0, 1) values and plants dominant logits (see _plant_peaks).
    """
    seed = BASE_SEED + w.seed_offset if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    B, h, nb, db, dr, dh = w.batch, w.heads, w.branches, w.branch_dim, w.rope_dim, w.head_dim
    dc = nb * db
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int32)
        assert lens.shape == (B,)
    elif seq_len is not None:
        lens = np.full(B, seq_len, dtype=np.int32)
    else:
        lens = draw_seq_lens(w, rng)
    Lmax = int(lens.max())
    std = 1.0 if peaked else w.std
    f32 = np.float32
    q_lat = (rng.standard_normal((B, h, nb, db), dtype=f32) * f32(std))
    q_rope = (rng.standard_normal((B, h, dr), dtype=f32) * f32(std))
    w_v = rng.standard_normal((h, dh, dc), dtype=f32) * f32(w.wv_std)
    out = {"seq_lens": torch.from_numpy(lens.copy())}
    if not w.paged:
        kv = rng.standard_normal((B, Lmax, dc + dr), dtype=f32) * f32(std)
        if peaked:
            _plant_peaks(rng, q_lat, q_rope, kv[:, :, :dc], kv[:, :, dc:], lens, nb, db, peak_gain)
        out["kv"] = _to_storage(kv, w.dtype)
    else:
        ps = w.page_size
        npages = [(int(L) + ps - 1) // ps for L in lens]
        P = int(sum(npages))
        max_pages = max(npages)
        pool = rng.standard_normal((P, ps, dc + dr), dtype=f32) * f32(std)
        perm = rng.permutation(P).astype(np.int32)
        table = np.full((B, max_pages), -1, dtype=np.int32)
        off = 0
        for beta in range(B):
            table[beta, :npages[beta]] = perm[off:off + npages[beta]]
            off += npages[beta]
        if peaked:
            # plant through the page table so the logical rows carry the peaks
            for beta in range(B):
                ids = table[beta, :npages[beta]]
                flat = pool[ids].reshape(-1, dc + dr)  # fancy indexing copies
                _plant_peaks(rng, q_lat[beta:beta + 1], q_rope[beta:beta + 1],
                             flat[None, :, :dc], flat[None, :, dc:], lens[beta:beta + 1], nb, db, peak_gain)
                pool[ids] = flat.reshape(npages[beta], ps, dc + dr)
        out["pool"] = _to_storage(pool, w.dtype)
        out["page_table"] = torch.from_numpy(table)
    out["q_lat"] = _to_storage(q_lat, w.dtype)
    out["q_rope"] = _to_storage(q_rope, w.dtype)
    out["w_v"] = _to_storage(w_v, w.dtype)
    return out
