"""Work accounting for the decode step: the bytes and flops the method must
move or compute at least once, and MI355X's published peaks."""
from __future__ import annotations

from typing import Sequence

import numpy as np

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_DENSE_TFLOPS = 2500.0      # dense MFMA bf16
FP32_VECTOR_TFLOPS = 157.3


def algorithmic_bytes(w, seq_lens: Sequence[int]) -> dict:
    """Cache rows of every context token read once, plus the queries, W^V and the
    output (in the stored element type)."""
    eb = w.elem_bytes
    tokens = int(np.sum(np.asarray(seq_lens, dtype=np.int64)))
    cache = tokens * w.row_dim * eb
    q = w.batch * w.heads * (w.latent_dim + w.rope_dim) * eb
    wv = w.heads * w.head_dim * w.latent_dim * eb
    out = w.batch * w.heads * w.head_dim * eb
    return {"cache": cache, "queries": q, "w_v": wv, "out": out, "total": cache + q + wv + out,
            "attention_kernel": cache + q, "tokens": tokens}


def algorithmic_flops(w, seq_lens: Sequence[int]) -> dict:
    """Multiply-adds x 2 of the attention contractions per context token and
    sequence: branch scores n_b*h*d_b, the RoPE score h*d_R (shared by the
    branches), P.C n_b*h*d_b; plus the W^V up-projection per sequence."""
    tokens = int(np.sum(np.asarray(seq_lens, dtype=np.int64)))
    per_tok = 2 * (w.branches * w.heads * w.branch_dim + w.heads * w.rope_dim
                   + w.branches * w.heads * w.branch_dim)
    epi = 2 * w.batch * w.heads * w.latent_dim * w.head_dim
    return {"per_token": per_tok, "attention": per_tok * tokens, "epilogue": epi,
            "total": per_tok * tokens + epi, "softmax_elements": tokens * w.heads * w.branches}


def tp_per_device_load(head_dim: int, rope_dim: int, ways: int) -> dict:
    """Cache elements one device loads per token under ``ways``-way tensor
    parallelism: MLRA gives each device one latent block (head_dim / ways wide in
    the Qwen3-32B setting) plus the shared RoPE key; MLA's single latent cannot be
    split, so each device loads all of it (MLRA page "原生支持张量并行的多分支低秩
    注意力MLRA", §1.4 and §3.2)."""
    return {"mlra": rope_dim + head_dim // ways, "mla": rope_dim + head_dim}
