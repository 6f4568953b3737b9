"""MI355X-native decode attention for Multi-Head Low-Rank Attention (MLRA) and
single-latent MLA. The compute lives in the HIP library ``libmlra.so`` (built
in-tree); this package is its thin ctypes binding plus input generators."""
