"""Writes tests/golden/tiny_f32_y.npy: the CPU oracle's output on the tiny fp32
workload. Calls only the oracle and the seeded input generator."""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import mlra_oracle as O  # noqa: E402
from rank_latent_kv_amd.workloads import PRESETS, make_inputs  # noqa: E402


def main():
    w = PRESETS["tiny_f32"]
    inp = make_inputs(w)
    kv = inp["kv"].double().numpy()
    dc = w.latent_dim
    y = O.mlra_decode_absorbed(inp["q_lat"].double().numpy(), inp["q_rope"].double().numpy(), kv[:, :, :dc],
                               kv[:, :, dc:], inp["seq_lens"].numpy(), inp["w_v"].double().numpy(),
                               w.sm_scale, w.alpha)
    np.save(os.path.join(HERE, "tiny_f32_y.npy"), y)


if __name__ == "__main__":
    main()
