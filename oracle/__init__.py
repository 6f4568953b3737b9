"""CPU fp64 oracle for MLRA / MLA decode attention.

Test infrastructure only: imported by ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py``. The product path (the HIP library and
its Python binding) never imports, links or runs anything in this package.
"""
from .mlra_oracle import (  # noqa: F401
    mlra_decode_absorbed,
    mlra_decode_materialised,
    mla_decode,
    mlra_decode_bruteforce,
    branch_partials,
    merge_partials,
    paged_gather,
    mlra_decode_paged,
    shared_softmax_decode,
)
