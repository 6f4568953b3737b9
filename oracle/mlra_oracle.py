"""Plain fp64 CPU oracle for the decode step of Multi-Head Low-Rank Attention
(MLRA) and of single-latent Multi-Head Latent Attention (MLA).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module. It shares no
code with the HIP library (no kernels, headers, helpers, tables or pre/post
processing) and imports nothing from it. Everything here is slow on purpose:
each function is the definition written out with numpy, so that it can be read
against the pages.

Pages cited (by title and section):
  [MLRA]   "原生支持张量并行的多分支低秩注意力MLRA：优化KV缓存，实现2.8倍解码加速"
           (yunpan.plus) — §1.3 MLA's three-step decode, §二 block decomposition of
           W^K, §三 moving the block sum after attention, §3.1 MLRA-4, §3.2 TP load,
           §3.3 output scaling.
  [MLA-LR] "Multi-Head Latent Attention：低秩近似优化Transformer计算效率"
           (jsqmd.com) — §2.2 K and V from one shared latent, §3.3 absorbed W_QK.
  [DS-MLA] DeepSeek MLA analysis (dlbhg.com), section "多頭潛在注意力（MLA）" —
           decoupled RoPE: extra per-head RoPE queries and one shared RoPE key.

Readings taken where the pages are silent or garbled (each is listed again in
the design notes):
  * The MLRA-4 equation did not survive extraction ([MLRA] §3.1 keeps only the
    sentence after it). Reading: for head i and branch b,
        z_s = tau * (q~_{i,b} . c_{s,b} + q^R_i . k^R_s)          (per token s)
        p   = softmax_s(z)      -- one independent softmax per (i, b)
        u_{i,b} = sum_s p_s c_{s,b}
        y_i = alpha * sum_b W^V_{i,b} u_{i,b}
    This is [MLRA] §三 (attention per block, then sum the block outputs) with
    §3.1's shared RoPE key and independent per-branch softmax.
  * Branch b owns latent columns [b*d_b, (b+1)*d_b) (contiguous blocks).
  * The RoPE query q^R_i is per head and shared by all branches of that head.
  * tau (softmax scale) and alpha (output scale, [MLRA] §3.3 gives no value) are
    plain arguments.
  * The query attends to exactly seq_lens[b] cached rows (no causal mask is
    needed for a single decode query); an empty context is rejected.
  * The pages name decoupled RoPE but print no rotation. Reading: the original
    rotary position embedding, consecutive pairs (x_2j, x_2j+1) turned by
    m * base^(-2j/d_R) at position m, base 10000; the cache stores RoPE keys
    already rotated to their own positions and the query is rotated to the new
    token's position.

Array layouts (float64 numpy; they mirror the library's boundary):
  q_lat   [B, h, n_b, d_b]   absorbed query of each head and branch
  q_rope  [B, h, d_R]        RoPE query of each head
  kv_lat  [B, L_max, d_c]    cached latents, d_c = n_b * d_b
  kv_rope [B, L_max, d_R]    cached shared RoPE keys (already rotated)
  seq_lens[B]                context length of each sequence
  w_v     [h, d_h, d_c]      W^V_{i,b} = w_v[i, :, b*d_b:(b+1)*d_b]  (d_h x d_b)
  result  y [B, h, d_h]
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np


def _softmax_rows(z: np.ndarray) -> np.ndarray:
    """Softmax along the last axis (textbook max-shifted form)."""
    zmax = z.max(axis=-1, keepdims=True)
    e = np.exp(z - zmax)
    return e / e.sum(axis=-1, keepdims=True)


def _check_lengths(seq_lens, L_max):
    for L in seq_lens:
        if not (1 <= int(L) <= L_max):
            raise ValueError(f"context length {int(L)} outside [1, {L_max}]")


def mlra_decode_absorbed(q_lat, q_rope, kv_lat, kv_rope, seq_lens, w_v, sm_scale, alpha):
    """MLRA decode with absorbed queries: one MQA-style attention per branch over
    that branch's latent block plus the shared RoPE key, an independent softmax per
    (head, branch), then W^V per branch and a scaled sum over branches.

    [MLRA] §1.3 (step 1 absorbed query, step 2 MQA-style attention over the cached
    latent, step 3 value up-projection), §三 and §3.1 (per-block attention with a
    shared RoPE key and independent softmax, block outputs summed), §3.3 (scaled
    sum). The RoPE score q^R_i . k^R_s is the same for every branch of head i.
    """
    q_lat = np.asarray(q_lat, dtype=np.float64)
    B, h, nb, db = q_lat.shape
    dh = w_v.shape[1]
    _check_lengths(seq_lens, kv_lat.shape[1])
    y = np.zeros((B, h, dh))
    for beta in range(B):
        L = int(seq_lens[beta])
        C = np.asarray(kv_lat[beta, :L], dtype=np.float64).reshape(L, nb, db)   # c_{s,b}
        KR = np.asarray(kv_rope[beta, :L], dtype=np.float64)                   # k^R_s
        rope_scores = np.asarray(q_rope[beta], dtype=np.float64) @ KR.T        # [h, L]
        for b in range(nb):
            z = sm_scale * (q_lat[beta, :, b, :] @ C[:, b, :].T + rope_scores)  # [h, L]
            p = _softmax_rows(z)
            u = p @ C[:, b, :]                                                  # [h, d_b]
            Wb = np.asarray(w_v[:, :, b * db:(b + 1) * db], dtype=np.float64)   # [h, d_h, d_b]
            y[beta] += np.einsum("inj,ij->in", Wb, u)
    return alpha * y


def mlra_decode_materialised(q_nope, w_k, q_rope, kv_lat, kv_rope, seq_lens, w_v, sm_scale, alpha,
                             num_branches, seqs=None, heads=None):
    """MLRA decode with per-branch keys and values materialised from the
    non-absorbed up-projections.

    [MLRA] §二: the per-head key up-projection W^K_i splits into blocks W^K_{i,b}
    (d_h x d_b) and the NoPE key is the sum of the block projections; §三 moves that
    sum after attention, so branch b attends with its own key
    k_{s,i,b} = W^K_{i,b} c_{s,b} and value v_{s,i,b} = W^V_{i,b} c_{s,b}
    (both width d_h), plus the shared RoPE key ([DS-MLA]).

      q_nope [B, h, d_h]   non-absorbed NoPE query of each head
      w_k    [h, d_h, d_c] W^K_{i,b} = w_k[i, :, b*d_b:(b+1)*d_b]
    Only the (sequence, head) pairs in ``seqs`` x ``heads`` are computed (others
    are left zero); the full product is expensive.
    """
    B, h, dh = q_nope.shape
    dc = w_k.shape[2]
    nb = num_branches
    db = dc // nb
    _check_lengths(seq_lens, kv_lat.shape[1])
    seqs = range(B) if seqs is None else seqs
    heads = range(h) if heads is None else heads
    y = np.zeros((B, h, w_v.shape[1]))
    for beta in seqs:
        L = int(seq_lens[beta])
        C = np.asarray(kv_lat[beta, :L], dtype=np.float64)
        KR = np.asarray(kv_rope[beta, :L], dtype=np.float64)
        for i in heads:
            qn = np.asarray(q_nope[beta, i], dtype=np.float64)
            qr = np.asarray(q_rope[beta, i], dtype=np.float64)
            for b in range(nb):
                Cb = C[:, b * db:(b + 1) * db]                                   # [L, d_b]
                K = Cb @ np.asarray(w_k[i, :, b * db:(b + 1) * db], dtype=np.float64).T  # [L, d_h]
                V = Cb @ np.asarray(w_v[i, :, b * db:(b + 1) * db], dtype=np.float64).T  # [L, d_h]
                z = sm_scale * (K @ qn + KR @ qr)
                p = _softmax_rows(z)
                y[beta, i] += p @ V
    return alpha * y


def mla_decode(q_lat, q_rope, kv_lat, kv_rope, seq_lens, w_v, sm_scale, alpha=1.0):
    """Single-latent MLA decode, [MLRA] §1.3: with the absorbed query (step 1)
    every head runs MQA-style attention (step 2) whose shared key is the cached row
    [c ; k^R] and whose shared value is the latent c; step 3 applies W^V_i.

      q_lat [B, h, d_c] (a [B, h, 1, d_c] array is accepted too), w_v [h, d_h, d_c].
    Written as one concatenated-key attention, independently of
    ``mlra_decode_absorbed``.
    """
    q_lat = np.asarray(q_lat, dtype=np.float64)
    if q_lat.ndim == 4:
        q_lat = q_lat.reshape(q_lat.shape[0], q_lat.shape[1], -1)
    B, h, dc = q_lat.shape
    _check_lengths(seq_lens, kv_lat.shape[1])
    y = np.zeros((B, h, w_v.shape[1]))
    for beta in range(B):
        L = int(seq_lens[beta])
        K = np.concatenate([np.asarray(kv_lat[beta, :L], dtype=np.float64),
                            np.asarray(kv_rope[beta, :L], dtype=np.float64)], axis=1)  # [L, d_c + d_R]
        Q = np.concatenate([q_lat[beta], np.asarray(q_rope[beta], dtype=np.float64)], axis=1)
        p = _softmax_rows(sm_scale * (Q @ K.T))                                         # [h, L]
        u = p @ K[:, :dc]                                                               # [h, d_c]
        y[beta] = np.einsum("inc,ic->in", np.asarray(w_v, dtype=np.float64), u)
    return alpha * y


def mlra_decode_bruteforce(q_lat, q_rope, kv_lat, kv_rope, seq_lens, w_v, sm_scale, alpha):
    """The same function as ``mlra_decode_absorbed`` with scalar Python loops,
    ``math.exp`` and ``math.fsum`` and no max shift. Tiny shapes only."""
    B, h, nb, db = np.shape(q_lat)
    dh = np.shape(w_v)[1]
    dr = np.shape(q_rope)[2]
    y = np.zeros((B, h, dh))
    for beta in range(B):
        L = int(seq_lens[beta])
        for i in range(h):
            for b in range(nb):
                w = []
                for s in range(L):
                    t = [float(q_lat[beta][i][b][j]) * float(kv_lat[beta][s][b * db + j]) for j in range(db)]
                    t += [float(q_rope[beta][i][r]) * float(kv_rope[beta][s][r]) for r in range(dr)]
                    w.append(math.exp(sm_scale * math.fsum(t)))
                tot = math.fsum(w)
                u = [math.fsum(w[s] * float(kv_lat[beta][s][b * db + j]) for s in range(L)) / tot
                     for j in range(db)]
                for n in range(dh):
                    y[beta][i][n] += math.fsum(float(w_v[i][n][b * db + j]) * u[j] for j in range(db))
            for n in range(dh):
                y[beta][i][n] *= alpha
    return y


def branch_partials(q_lat, q_rope, kv_lat, kv_rope, beta, start, stop, sm_scale):
    """Unnormalised attention state of one context chunk [start, stop) of sequence
    ``beta`` for every (head, branch): m = max logit, l = sum exp(z - m),
    o = sum exp(z - m) c_b. Natural-log units.

    Returns (o [h, n_b, d_b], m [h, n_b], l [h, n_b])."""
    q_lat = np.asarray(q_lat, dtype=np.float64)
    _, h, nb, db = q_lat.shape
    C = np.asarray(kv_lat[beta, start:stop], dtype=np.float64).reshape(stop - start, nb, db)
    KR = np.asarray(kv_rope[beta, start:stop], dtype=np.float64)
    rope_scores = np.asarray(q_rope[beta], dtype=np.float64) @ KR.T
    o = np.zeros((h, nb, db))
    m = np.zeros((h, nb))
    l = np.zeros((h, nb))
    for b in range(nb):
        z = sm_scale * (q_lat[beta, :, b, :] @ C[:, b, :].T + rope_scores)
        m[:, b] = z.max(axis=1)
        e = np.exp(z - m[:, b:b + 1])
        l[:, b] = e.sum(axis=1)
        o[:, b, :] = e @ C[:, b, :]
    return o, m, l


def merge_partials(parts: Sequence[Tuple[np.ndarray, np.ndarray, np.ndarray]]) -> np.ndarray:
    """Exact log-sum-exp merge of chunk states: with m* = max_k m_k and
    w_k = exp(m_k - m*), the attention output is sum_k w_k o_k / sum_k w_k l_k.
    Returns u [h, n_b, d_b]."""
    ms = np.stack([p[1] for p in parts])               # [K, h, n_b]
    mstar = ms.max(axis=0)
    w = np.exp(ms - mstar)
    num = sum(w[k][..., None] * parts[k][0] for k in range(len(parts)))
    den = sum(w[k] * parts[k][2] for k in range(len(parts)))
    return num / den[..., None]


def paged_gather(pool, page_table, seq_lens, page_size):
    """Logical cache rows of each sequence through its page table: row s of
    sequence b is pool[page_table[b][s // page_size]][s % page_size]. Rows past a
    sequence's length are zero. pool [P, page_size, R] -> rows [B, L_max, R]."""
    pool = np.asarray(pool)
    B = len(seq_lens)
    L_max = int(max(seq_lens))
    out = np.zeros((B, L_max, pool.shape[2]), dtype=pool.dtype)
    for beta in range(B):
        for s in range(int(seq_lens[beta])):
            out[beta, s] = pool[int(page_table[beta][s // page_size]), s % page_size]
    return out


def mlra_decode_paged(q_lat, q_rope, pool, page_table, seq_lens, page_size, latent_dim, w_v,
                      sm_scale, alpha):
    """MLRA decode over a paged cache: gather the logical rows (latent columns
    first, RoPE key after them), then the absorbed decode."""
    rows = paged_gather(pool, page_table, seq_lens, page_size)
    return mlra_decode_absorbed(q_lat, q_rope, rows[:, :, :latent_dim], rows[:, :, latent_dim:],
                                seq_lens, w_v, sm_scale, alpha)


def absorption_consistent_query(q_lat, head_dim, rng) -> Tuple[np.ndarray, np.ndarray]:
    """Build a non-absorbed NoPE query q^N and key up-projection W^K whose
    absorption reproduces ``q_lat`` ([MLA-LR] §3.3, [MLRA] §1.3 step 1:
    q~_{i,b} = W^K_{i,b}^T q^N_i).

    W^K_i (d_h x d_c) gets orthonormal columns (QR of a Gaussian, needs
    d_c <= d_h) and q^N_i = W^K_i q~_i, so W^K_i^T q^N_i = q~_i up to fp64
    rounding. Returns (q_nope [B, h, d_h], w_k [h, d_h, d_c])."""
    q_lat = np.asarray(q_lat, dtype=np.float64)
    B, h, nb, db = q_lat.shape
    dc = nb * db
    if dc > head_dim:
        raise ValueError("orthonormal columns need d_c <= d_h")
    w_k = np.empty((h, head_dim, dc))
    for i in range(h):
        qmat, _ = np.linalg.qr(rng.standard_normal((head_dim, dc)))
        w_k[i] = qmat[:, :dc]
    q_nope = np.einsum("inc,bic->bin", w_k, q_lat.reshape(B, h, dc))
    return q_nope, w_k


def rope_angles(positions, rope_dim: int, base: float = 10000.0) -> np.ndarray:
    """Rotary angles: pair j of a d_R-wide RoPE vector at position m turns by
    m * theta_j with theta_j = base^(-2j / d_R), j = 0 .. d_R/2 - 1 (the rotary
    position embedding behind [DS-MLA]'s decoupled RoPE; the pages do not print
    it, so the original rotary form is taken, see the readings). fp64, shape
    [len(positions), d_R / 2]."""
    if rope_dim % 2:
        raise ValueError("rope_dim must be even")
    pos = np.asarray(positions, dtype=np.float64).reshape(-1, 1)
    theta = base ** (-2.0 * np.arange(rope_dim // 2, dtype=np.float64) / rope_dim)
    return pos * theta[None, :]


def rope_rotate(x, positions, base: float = 10000.0) -> np.ndarray:
    """Rotate consecutive pairs (x_2j, x_2j+1) of the last axis by the angle of
    their row's position: (x_2j cos a - x_2j+1 sin a, x_2j sin a + x_2j+1 cos a).
    x has shape [B, ..., d_R] and positions [B] (one position per leading index)."""
    x = np.asarray(x, dtype=np.float64)
    B, dr = x.shape[0], x.shape[-1]
    ang = rope_angles(positions, dr, base)                       # [B, d_R/2]
    shape = (B,) + (1,) * (x.ndim - 2) + (dr // 2,)
    c, s = np.cos(ang).reshape(shape), np.sin(ang).reshape(shape)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


def absorb_query(q_nope, w_uk_t, num_branches: int) -> np.ndarray:
    """Absorbed query of [MLRA] §1.3 step 1 ([MLA-LR] §3.3): for head i,
    q~_i = W^UK_i^T q^N_i, so that q~_i . c = q^N_i . (W^UK_i c) for every latent
    c. w_uk_t [h, d_c, d_h] stores W^UK_i^T (row n is the d_h-vector whose dot
    with q^N_i gives q~_i[n]). Branch b takes q~_i[b*d_b:(b+1)*d_b] ([MLRA] §二).
    Returns q_lat [B, h, n_b, d_b]."""
    q_nope = np.asarray(q_nope, dtype=np.float64)
    w = np.asarray(w_uk_t, dtype=np.float64)
    B, h, dh = q_nope.shape
    dc = w.shape[1]
    q = np.einsum("ind,bid->bin", w, q_nope)                    # [B, h, d_c]
    return q.reshape(B, h, num_branches, dc // num_branches)


def prepare_decode(q_nope, q_pe, w_uk_t, num_branches, c_new, k_pe_new, positions, base=10000.0):
    """The step before the attention call, for one new token per sequence at
    position positions[b]: the absorbed query, the RoPE query rotated to that
    position, and the token's cache row (its latent, then its RoPE key rotated to
    the same position). Returns (q_lat, q_rope, row [B, d_c + d_R])."""
    q_lat = absorb_query(q_nope, w_uk_t, num_branches)
    q_rope = rope_rotate(q_pe, positions, base)
    k_rot = rope_rotate(np.asarray(k_pe_new, dtype=np.float64), positions, base)
    row = np.concatenate([np.asarray(c_new, dtype=np.float64), k_rot], axis=-1)
    return q_lat, q_rope, row


def shared_softmax_decode(q_lat, q_rope, kv_lat, kv_rope, seq_lens, w_v, sm_scale, alpha):
    """MLA over the same (blocked) cache: the branch queries are concatenated into
    one d_c-wide absorbed query and ONE softmax per head covers the summed score.
    This is what MLRA is not ([MLRA] §三): used to show the branches' softmaxes are
    independent."""
    B, h, nb, db = np.shape(q_lat)
    return mla_decode(np.asarray(q_lat).reshape(B, h, nb * db), q_rope, kv_lat, kv_rope, seq_lens,
                      w_v, sm_scale, alpha)
