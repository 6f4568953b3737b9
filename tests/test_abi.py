"""CPU tests of the C ABI: the library loads and exports every symbol the header
declares, the ctypes struct matches the C struct, host validation returns the
documented status for bad arguments (it runs before any HIP call, so no GPU is
needed), and the host page allocator / page-table check behave as documented."""
import ctypes
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import rank_latent_kv_amd as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mlra.h")

pytestmark = pytest.mark.skipif(not os.path.exists(R.LIB_PATH), reason="libmlra.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(mlra_\w+|mla_\w+)\s*\(", text)
    return sorted(set(n for n in names if not n.startswith("mlra_status") and n != "mlra_decode_args"))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 14
    lib = R.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(R.EXPORTED_SYMBOLS)
    out = subprocess.run(["nm", "-D", "--defined-only", R.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}\b", out), n


def test_version_and_clean_error():
    assert "gfx950" in R.lib().mlra_version().decode()


def test_struct_layout_matches_header():
    fields = [f[0] for f in R.DecodeArgs._fields_]
    src = ["#include <stdio.h>", "#include <stddef.h>", '#include "mlra.h"', "int main(void) {",
           'printf("size %zu\\n", sizeof(mlra_decode_args));']
    src += [f'printf("{f} %zu\\n", offsetof(mlra_decode_args, {f}));' for f in fields]
    src += ["return 0; }"]
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(c, "w").write("\n".join(src))
        subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        got = dict(line.split() for line in subprocess.run([exe], capture_output=True, text=True).stdout.splitlines())
    assert int(got["size"]) == ctypes.sizeof(R.DecodeArgs)
    for f in fields:
        assert int(got[f]) == getattr(R.DecodeArgs, f).offset, f


# ---- host validation -----------------------------------------------------------------------

FAKE = 1 << 20   # 16-byte aligned stand-in device addresses; validation never dereferences them


def base_args(B=2, H=64, NB=4, DB=32, DR=32, DH=128, L=4096, dtype=R.MLRA_BF16, lens=None):
    a = R.DecodeArgs()
    a.batch, a.num_heads, a.num_branches, a.branch_dim, a.rope_dim, a.head_dim = B, H, NB, DB, DR, DH
    a.dtype = a.out_dtype = dtype
    a.sm_scale, a.alpha = 0.125, 0.5
    a.q_lat, a.q_rope, a.kv_lat = FAKE, FAKE * 2, FAKE * 4
    eb = 2 if dtype == R.MLRA_BF16 else 4
    a.kv_rope = FAKE * 4 + NB * DB * eb
    a.row_stride = NB * DB + DR
    a.seq_stride = L * a.row_stride
    a.seq_lens = FAKE * 8
    a.max_seq_len = L
    a.w_v, a.out = FAKE * 16, FAKE * 32
    if lens is not None:
        base_args.keep = (ctypes.c_int32 * B)(*lens)
        a.seq_lens_host = ctypes.cast(base_args.keep, ctypes.c_void_p).value
    return a


def with_workspace(a):
    n = R.workspace_size(a)
    a.workspace = FAKE * 64
    a.workspace_bytes = n
    return a


def test_valid_args_pass_validation():
    a = with_workspace(base_args(lens=[4096, 17]))
    assert R.validate(a) == R.MLRA_OK
    assert R.last_error() == ""


def test_workspace_size_formula():
    """One record per (sequence, split, head, branch): d_b outputs (fp16 for the MFMA kernel with
    several branches, as here) and an fp32 (m, l) pair, each array rounded up to 256 bytes."""
    a = base_args(B=16, L=32768)
    n = R.workspace_size(a)
    # MFMA path: 128-token stages, about one work-group per CU -> 16 splits of 2048 tokens
    recs = 16 * 16 * 64 * 4
    expect = -(-recs * 32 * 2 // 256) * 256 + -(-recs * 2 * 4 // 256) * 256
    assert n == expect
    a.num_splits = 7
    n7 = R.workspace_size(a)
    assert n7 == -(-16 * 7 * 64 * 4 * 32 * 2 // 256) * 256 + -(-16 * 7 * 64 * 4 * 2 * 4 // 256) * 256


def test_workspace_size_keeps_fp32_outputs_where_the_kernel_writes_them():
    """fp32 inputs (the generic kernel) and the MFMA shape whose waves write 2-row pieces (the
    16-head one-branch shard of eight phases) keep fp32 output records; the one-branch shapes
    of four phases (MLA at 64 heads, the 16-head MLA shard, the 64-head branch shard) write
    fp16 ones, like the multi-branch shapes."""
    f = base_args(B=2, L=4096, dtype=R.MLRA_F32)
    f.num_splits = 3
    recs = 2 * 3 * 64 * 4
    assert R.workspace_size(f) == -(-recs * 32 * 4 // 256) * 256 + -(-recs * 2 * 4 // 256) * 256
    for nb, db, h, eb in ((1, 128, 64, 2), (1, 128, 16, 2), (1, 32, 64, 2), (1, 32, 16, 4)):
        m = base_args(B=2, L=4096, NB=nb, DB=db, H=h)
        m.num_splits = 3
        recs = 2 * 3 * h * nb
        assert R.plan(m, cu_count=256)["kernel"] == "mfma"
        assert R.workspace_size(m) == -(-recs * db * eb // 256) * 256 + -(-recs * 2 * 4 // 256) * 256, (nb, db, h)


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, R.MLRA_ERR_INVALID_ARG),
    ("num_heads", 0, R.MLRA_ERR_INVALID_ARG),
    ("num_branches", 0, R.MLRA_ERR_INVALID_ARG),
    ("branch_dim", 0, R.MLRA_ERR_INVALID_ARG),
    ("head_dim", -1, R.MLRA_ERR_INVALID_ARG),
    ("rope_dim", -2, R.MLRA_ERR_INVALID_ARG),
    ("dtype", 7, R.MLRA_ERR_INVALID_ARG),
    ("out_dtype", 9, R.MLRA_ERR_INVALID_ARG),
    ("max_seq_len", 0, R.MLRA_ERR_INVALID_ARG),
    ("num_splits", -1, R.MLRA_ERR_INVALID_ARG),
    ("row_stride", 0, R.MLRA_ERR_INVALID_ARG),
    ("q_lat", None, R.MLRA_ERR_INVALID_ARG),
    ("kv_rope", None, R.MLRA_ERR_INVALID_ARG),
    ("seq_lens", None, R.MLRA_ERR_INVALID_ARG),
    ("w_v", None, R.MLRA_ERR_INVALID_ARG),
    ("out", None, R.MLRA_ERR_INVALID_ARG),
    ("sm_scale", float("nan"), R.MLRA_ERR_INVALID_ARG),
    ("sm_scale", 0.0, R.MLRA_ERR_INVALID_ARG),
    ("sm_scale", -0.5, R.MLRA_ERR_INVALID_ARG),
    ("alpha", float("inf"), R.MLRA_ERR_INVALID_ARG),
    ("seq_stride", 5, R.MLRA_ERR_INVALID_ARG),
])
def test_invalid_field(field, value, status):
    a = with_workspace(base_args())
    setattr(a, field, value)
    assert R.validate(a) == status
    assert R.last_error() != ""
    # the decode entry point reports the same error without launching anything
    assert R.lib().mlra_decode(ctypes.byref(a), None) == status


def test_empty_context_rejected():
    a = with_workspace_raw(base_args(lens=[4096, 0]))
    assert R.validate(a) == R.MLRA_ERR_INVALID_ARG
    assert "empty context" in R.last_error()
    assert R.lib().mlra_decode_workspace_size(ctypes.byref(a)) == 0
    a = with_workspace_raw(base_args(lens=[4097, 1]))
    assert R.validate(a) == R.MLRA_ERR_INVALID_ARG


def test_workspace_errors():
    a = base_args()
    n = R.workspace_size(a)
    a.workspace = None
    assert R.validate(a) == R.MLRA_ERR_WORKSPACE
    a.workspace, a.workspace_bytes = FAKE * 64, n - 1
    assert R.validate(a) == R.MLRA_ERR_WORKSPACE
    a.workspace, a.workspace_bytes = FAKE * 64 + 16, n
    assert R.validate(a) == R.MLRA_ERR_INVALID_ARG


def test_noalloc_refuses_on_the_host_first():
    """mlra_decode_noalloc checks its arguments and the size of the split state on the host
    before any device call: a NULL struct and invalid fields are refused, and so is a plan whose
    split state exceeds the library's device array (here without a GPU in the process)."""
    L = R.lib()
    assert L.mlra_decode_noalloc(None, None) == R.MLRA_ERR_INVALID_ARG
    a = base_args()
    a.num_heads = 0
    assert L.mlra_decode_noalloc(ctypes.byref(a), None) == R.MLRA_ERR_INVALID_ARG
    big = base_args(B=256, L=8192)
    big.num_splits = 64
    assert R.workspace_size(big) > R.NOALLOC_SCRATCH_BYTES
    assert L.mlra_decode_noalloc(ctypes.byref(big), None) == R.MLRA_ERR_WORKSPACE
    assert "device array" in R.last_error()


def test_noalloc_array_size_matches_the_header():
    text = open(os.path.join(ROOT, "include", "mlra.h")).read()
    m = re.search(r"#define MLRA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == R.NOALLOC_SCRATCH_BYTES


def test_overlapping_rope_rejected():
    a = with_workspace(base_args())
    a.kv_rope = a.kv_lat + 2 * 64
    assert R.validate(a) == R.MLRA_ERR_INVALID_ARG
    a = with_workspace(base_args())
    a.row_stride = 100
    a.seq_stride = 100 * 4096
    assert R.validate(a) == R.MLRA_ERR_INVALID_ARG


def test_mla_requires_one_branch():
    a = with_workspace(base_args())
    assert R.lib().mla_decode(ctypes.byref(a), None) == R.MLRA_ERR_INVALID_ARG
    assert "num_branches" in R.last_error()


def test_unsupported_shape():
    a = base_args(NB=32, DB=256)
    assert R.lib().mlra_decode_workspace_size(ctypes.byref(a)) == 0
    assert R.validate(with_workspace_raw(a)) in (R.MLRA_ERR_UNSUPPORTED,)


def with_workspace_raw(a):
    a.workspace, a.workspace_bytes = FAKE * 64, 1 << 40
    return a


def test_generic_path_shapes_validate():
    # shapes without an MFMA build still validate (generic kernel): 3 branches of 16, fp32
    a = with_workspace(base_args(NB=3, DB=16, DR=8, DH=24, dtype=R.MLRA_F32))
    assert R.validate(a) == R.MLRA_OK


def test_paged_validation():
    a = base_args()
    a.page_table = FAKE * 128
    a.page_size = 48
    a.max_pages, a.num_pages = 100, 100
    a.workspace, a.workspace_bytes = FAKE * 64, 1 << 40
    assert R.validate(a) == R.MLRA_ERR_INVALID_ARG          # page size not a power of two
    a.page_size = 64
    a.max_pages = 10                                          # 10 x 64 < 4096
    assert R.validate(a) == R.MLRA_ERR_INVALID_ARG
    a.max_pages = 64
    a.num_pages = 0
    assert R.validate(a) == R.MLRA_ERR_INVALID_ARG
    a.num_pages = 128
    assert R.validate(a) == R.MLRA_OK
    # a page of 2^24 rows x 160 bf16 elements is 5 GiB: beyond the 32-bit page offset
    a.page_size, a.max_pages = 1 << 24, 1
    assert R.validate(a) == R.MLRA_ERR_UNSUPPORTED
    assert "4 GiB" in R.last_error()


def test_paged_copy_validation():
    L = R.lib()
    vp = FAKE
    assert L.mlra_paged_append(None, 160, 160, 64, 4, vp, 4, vp, vp, 2, 0, None, None) == R.MLRA_ERR_INVALID_ARG
    assert L.mlra_paged_append(vp, 160, 160, 48, 4, vp, 4, vp, vp, 2, 0, None, None) == R.MLRA_ERR_INVALID_ARG
    assert L.mlra_paged_append(vp, 100, 160, 64, 4, vp, 4, vp, vp, 2, 0, None, None) == R.MLRA_ERR_INVALID_ARG
    assert L.mlra_paged_append(vp, 160, 160, 64, 4, vp, 4, vp, vp, 0, 0, None, None) == R.MLRA_ERR_INVALID_ARG
    assert L.mlra_paged_gather(vp, 160, 160, 64, 4, vp, 4, None, 64, 2, 0, vp, None, None) == R.MLRA_ERR_INVALID_ARG
    assert L.mlra_paged_gather(vp, 160, 160, 64, 4, vp, 4, vp, 0, 2, 0, vp, None, None) == R.MLRA_ERR_INVALID_ARG
    assert L.mlra_paged_gather(vp, 160, 160, 64, 4, vp, 4, vp, 64, 2, 3, vp, None, None) == R.MLRA_ERR_INVALID_ARG


# ---- host page allocator and page-table check -------------------------------------------------

def test_page_pool_lifo_and_exhaustion():
    p = R.PagePool(6)
    assert p.num_free == 6
    assert p.alloc(3) == [0, 1, 2]
    assert p.alloc(2) == [3, 4]
    with pytest.raises(R.MlraError) as e:
        p.alloc(2)
    assert e.value.status == R.MLRA_ERR_NO_PAGES
    assert p.num_free == 1                         # failed alloc changed nothing
    p.free([1, 3])
    assert p.alloc(2) == [3, 1]                    # LIFO: last freed first
    assert p.alloc(1) == [5]
    assert p.num_free == 0
    p.close()


def test_page_pool_free_errors():
    p = R.PagePool(4)
    ids = p.alloc(2)
    with pytest.raises(R.MlraError):
        p.free([2])                                # not allocated
    with pytest.raises(R.MlraError):
        p.free([0, 0])                             # repeated
    with pytest.raises(R.MlraError):
        p.free([7])                                # out of range
    assert p.num_free == 2                         # nothing changed
    p.free(ids)
    with pytest.raises(R.MlraError):
        p.free(ids)                                # double free
    assert p.num_free == 4
    with pytest.raises(R.MlraError):
        R.PagePool(0)


def test_page_pool_deterministic():
    a, b = R.PagePool(32), R.PagePool(32)
    rng = np.random.default_rng(0)
    held_a, held_b = [], []
    for _ in range(50):
        if held_a and rng.random() < 0.4:
            k = int(rng.integers(1, len(held_a) + 1))
            a.free(held_a[:k]); b.free(held_b[:k])
            held_a, held_b = held_a[k:], held_b[k:]
        else:
            n = int(rng.integers(0, 4))
            if n <= a.num_free:
                x, y = a.alloc(n), b.alloc(n)
                assert x == y
                held_a += x; held_b += y


def test_page_table_check():
    lens = torch.tensor([130, 64, 1], dtype=torch.int32)
    pt = torch.tensor([[4, 0, 7, -1], [2, -1, -1, -1], [5, -1, -1, -1]], dtype=torch.int32)
    R.page_table_check(pt, lens, 64, 8)
    bad = pt.clone(); bad[0, 2] = 8
    with pytest.raises(R.MlraError):
        R.page_table_check(bad, lens, 64, 8)       # out of range
    bad = pt.clone(); bad[1, 0] = 4
    with pytest.raises(R.MlraError):
        R.page_table_check(bad, lens, 64, 8)       # page shared by two slots
    with pytest.raises(R.MlraError):
        R.page_table_check(pt, torch.tensor([300, 64, 1], dtype=torch.int32), 64, 8)  # needs 5 pages > 4
    bad = pt.clone(); bad[2, 0] = -1
    with pytest.raises(R.MlraError):
        R.page_table_check(bad, lens, 64, 8)
    with pytest.raises(R.MlraError):
        R.page_table_check(pt, lens, 48, 8)


def test_split_limits_follow_the_merge_kernel():
    """The MFMA merge (bf16, 16-byte aligned W^V) has no per-split LDS, so the
    MLRA-4 shape takes up to 4096 one-stage splits; the vector-ALU merge (fp32
    W^V) keeps (m, l) of every split in LDS and refuses that many."""
    L = 4096 * 128
    a = base_args(B=1, L=L)
    a.num_splits = 4096
    n = R.workspace_size(a)
    assert n == 4096 * 64 * 4 * 32 * 2 + 4096 * 64 * 4 * 2 * 4   # fp16 outputs, fp32 (m, l)
    a.num_splits = 4097          # rounds up to 128-token splits again: still 4096 of them
    assert R.workspace_size(a) == n
    f = base_args(B=1, L=L, dtype=R.MLRA_F32)
    f.num_splits = 4096
    with pytest.raises(R.MlraError, match="LDS"):
        R.workspace_size(f)
    f.num_splits = 64
    assert R.workspace_size(f) > 0
    huge = base_args(B=1, L=8192 * 128)
    huge.num_splits = 8192
    with pytest.raises(R.MlraError, match="limit"):
        R.workspace_size(huge)


def test_auto_split_fits_one_pass_over_the_cus():
    """Ragged host lengths: the automatic split grows until the work-groups (the sum over
    sequences of ceil(L / split)) fit one per CU (256 on MI355X)."""
    lens = [84575, 128735, 91988, 118737]
    a = base_args(B=4, L=max(lens), lens=lens)
    n = R.workspace_size(a)
    recs_per_split = 4 * 64 * 4
    splits = n // (recs_per_split * 32 * 2 + recs_per_split * 2 * 4)   # fp16 outputs, fp32 (m, l)
    split_tokens = -(-max(lens) // splits)
    groups = sum(-(-L // (-(-split_tokens // 128) * 128)) for L in lens)
    assert splits == -(-max(lens) // 1792)
    assert groups <= 256


def _auto_split_tokens(lens):
    """The automatic split of an MLRA-4 headline-shaped launch, read back from the workspace
    size (one record of 32 fp16 outputs and an fp32 (m, l) pair per sequence, split, head,
    branch)."""
    a = base_args(B=len(lens), L=max(lens), lens=lens)
    recs_per_split = len(lens) * 64 * 4
    splits = R.workspace_size(a) // (recs_per_split * 32 * 2 + recs_per_split * 2 * 4)
    return splits, -(-max(lens) // splits)


def _working_groups_per_engine(lens, splits, split_tokens):
    """Work-groups that hold tokens on each shader engine, for the (splits, batch) grid placed
    as MI355X places it: linear id mod 8 picks the XCD, then (id / 8) mod 4 the engine."""
    split = -(-split_tokens // 128) * 128
    count = {}
    for b, L in enumerate(lens):
        s = 0
        while s * split < L:
            i = b * splits + s
            key = (i % 8, (i // 8) % 4)
            count[key] = count.get(key, 0) + 1
            s += 1
    return count


@pytest.mark.parametrize("lens,expect", [
    ([84575, 128735, 91988, 118737], 1792),        # the paged workload's lengths
    ([32768] * 16, 2048),                          # the headline: 256 groups, no empty ones
    ([16271, 41432, 23455, 72937, 107740, 66915, 69898, 93405, 57756, 111379, 35519, 20302], 4096),
    ([27772, 59750, 93319, 14328, 17494, 78239], 1280),
    ([12914, 19265, 64838, 62810], 768),
])
def test_auto_split_runs_one_pass_per_shader_engine(lens, expect):
    """The automatic split grows until no shader engine (8 CUs, one group each) gets a ninth
    group that holds tokens. On the last three batches a split chosen by the total group count
    alone (2944, 1152 and 640 tokens) puts nine on some engine, which measured 30% slower."""
    splits, split_tokens = _auto_split_tokens(lens)
    assert splits == -(-max(lens) // expect)
    count = _working_groups_per_engine(lens, splits, split_tokens)
    assert sum(count.values()) <= 256
    assert max(count.values()) <= 8


def _planner_by_linear_scan(lens, stage=128, cus=256):
    """The automatic split's rule, written as the plain scan it stands for: start at the mean
    tokens per CU and grow one stage at a time until the working groups fit one per CU and no
    shader engine gets a ninth (or the split covers the longest sequence)."""
    L = max(lens)
    split = max(-(-(-(-sum(lens) // cus)) // stage) * stage, stage)
    while split < L:
        ns = -(-L // split)
        if sum(-(-x // split) for x in lens) <= cus:
            count = {}
            for b, x in enumerate(lens):
                for s in range(-(-x // split)):
                    i = b * ns + s
                    count[(i % 8, (i // 8) % 4)] = count.get((i % 8, (i // 8) % 4), 0) + 1
            if max(count.values()) <= cus // 32:
                break
        split += stage
    return -(-L // min(split, L + stage))


@pytest.mark.parametrize("n_short", [199, 1023])
def test_auto_split_one_long_context_among_many_short(n_short):
    """One 2^20-token context beside many one-token ones: with 200 sequences one pass is still
    possible (the long one takes 57 of the 256 CUs); with 1024 every sequence gets one split.
    The planner bisects the group count, so the call stays cheap on the host (0.01 ms at 1024
    sequences, against 18 ms for growing the split one stage at a time)."""
    import time
    lens = [1] * n_short + [1 << 20]
    a = base_args(B=len(lens), L=max(lens), lens=lens)
    t0 = time.perf_counter()
    n = R.workspace_size(a)
    dt = time.perf_counter() - t0
    splits = n // (len(lens) * 64 * 4 * (32 * 2 + 2 * 4))
    assert splits == _planner_by_linear_scan(lens)
    if n_short == 1023:
        assert splits == 1
    assert dt < 0.005, dt   # a stage-by-stage scan took 18 ms here at 1024 sequences


# ---- the prepare step ------------------------------------------------------------------------

def test_prepare_struct_layout_matches_header():
    fields = [f[0] for f in R.PrepareArgs._fields_]
    src = ["#include <stdio.h>", "#include <stddef.h>", '#include "mlra.h"', "int main(void) {",
           'printf("size %zu\\n", sizeof(mlra_prepare_args));']
    src += [f'printf("{f} %zu\\n", offsetof(mlra_prepare_args, {f}));' for f in fields]
    src += ["return 0; }"]
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(c, "w").write("\n".join(src))
        subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        got = dict(line.split() for line in subprocess.run([exe], capture_output=True, text=True).stdout.splitlines())
    assert int(got["size"]) == ctypes.sizeof(R.PrepareArgs)
    for f in fields:
        assert int(got[f]) == getattr(R.PrepareArgs, f).offset, f


def prepare_args(**over):
    a = R.PrepareArgs()
    a.batch, a.num_heads, a.num_branches, a.branch_dim, a.rope_dim, a.head_dim = 2, 64, 4, 32, 32, 128
    a.dtype, a.rope_base = R.MLRA_BF16, 10000.0
    for name in ("q_nope", "q_pe", "w_uk", "c_new", "k_pe_new", "positions", "q_lat", "q_rope", "kv_lat"):
        setattr(a, name, FAKE)
    a.kv_rope = FAKE + 256
    a.row_stride, a.seq_stride, a.max_seq_len = 160, 160 * 100, 100
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value", [("rope_dim", 31), ("dtype", 5), ("rope_base", 0.0), ("batch", 0),
                                         ("q_nope", None), ("kv_lat", None), ("max_seq_len", 0), ("row_stride", 0)])
def test_prepare_rejects_bad_arguments(field, value):
    """Host validation fails before any HIP call (no GPU needed)."""
    a = prepare_args(**{field: value})
    assert R.lib().mlra_decode_prepare(ctypes.byref(a), None) == R.MLRA_ERR_INVALID_ARG
    assert R.last_error() != ""


def test_prepare_rejects_positions_outside_the_cache():
    pos = (ctypes.c_int32 * 2)(5, 100)
    a = prepare_args(positions_host=ctypes.cast(pos, ctypes.c_void_p).value)
    assert R.lib().mlra_decode_prepare(ctypes.byref(a), None) == R.MLRA_ERR_INVALID_ARG
    assert "outside the cache" in R.last_error()


@pytest.mark.parametrize("src,nbytes,out,words,msg", [
    (0, 4096, 256, 4096, "NULL"),
    (256, 4096, 0, 4096, "NULL"),
    (256, 0, 256, 4096, "multiple of 16"),
    (256, 4100, 256, 4096, "multiple of 16"),
    (264, 4096, 256, 4096, "aligned"),
    (256, 4096, 256, 7, "needs"),
])
def test_read_probe_validation(src, nbytes, out, words, msg):
    """Argument errors of the streaming-read probe come back before any HIP call (the
    pointers here are never dereferenced)."""
    L = R.lib()
    assert L.mlra_read_probe_words() >= 1
    st = L.mlra_read_probe(ctypes.c_void_p(src), nbytes, ctypes.c_void_p(out), words, None)
    assert st == R.MLRA_ERR_INVALID_ARG
    assert msg in R.last_error()


def test_arg_structs_keep_their_tensors_alive():
    """The ctypes structs hold raw pointers; they must keep the tensors behind them alive, or
    a caller that drops its own references leaves them pointing at freed memory."""
    import gc
    import weakref
    B, H, NB, DB, DR, DH, L = 2, 4, 4, 8, 8, 16, 8
    ws = torch.empty(64, dtype=torch.uint8)
    ref = weakref.ref(ws)
    a = R.make_args(torch.zeros(B, H, NB, DB), torch.zeros(B, H, DR), torch.zeros(B, L, NB * DB + DR)[..., :NB * DB],
                    torch.zeros(B, L, NB * DB + DR)[..., NB * DB:], torch.zeros(B, dtype=torch.int32),
                    torch.zeros(H, DH, NB * DB), sm_scale=1.0, alpha=1.0, workspace=ws)
    del ws
    gc.collect()
    assert ref() is not None and ref().data_ptr() == a.workspace
    qn = torch.zeros(B, H, DH)
    qref = weakref.ref(qn)
    pa = R.make_prepare_args(qn, torch.zeros(B, H, DR), torch.zeros(H, NB * DB, DH), torch.zeros(B, NB * DB),
                             torch.zeros(B, DR), torch.zeros(B, dtype=torch.int32), torch.zeros(B, L, NB * DB),
                             torch.zeros(B, L, DR), num_branches=NB, q_lat=torch.zeros(B, H, NB, DB),
                             q_rope=torch.zeros(B, H, DR))
    del qn
    gc.collect()
    assert qref() is not None and qref().data_ptr() == pa.q_nope
    del a, pa
    gc.collect()
    assert ref() is None and qref() is None


# ---- the binding refuses tensors whose raw pointers the library would misread ----------------

def _small_tensors(dtype=torch.bfloat16):
    B, H, NB, DB, DR, DH, L = 2, 4, 4, 8, 8, 16, 8
    kv = torch.zeros(B, L, NB * DB + DR, dtype=dtype)
    return dict(q_lat=torch.zeros(B, H, NB, DB, dtype=dtype), q_rope=torch.zeros(B, H, DR, dtype=dtype),
                kv_lat=kv[..., :NB * DB], kv_rope=kv[..., NB * DB:], seq_lens=torch.full((B,), L, dtype=torch.int32),
                w_v=torch.zeros(H, DH, NB * DB, dtype=dtype))


def _make(**over):
    t = _small_tensors()
    extra = {k: v for k, v in over.items() if k not in t}
    t.update({k: v for k, v in over.items() if k in t})
    return R.make_args(t["q_lat"], t["q_rope"], t["kv_lat"], t["kv_rope"], t["seq_lens"], t["w_v"], sm_scale=1.0,
                       alpha=1.0, **extra)


def test_binding_accepts_consistent_tensors():
    a = _make()
    assert a.batch == 2 and a.num_branches == 4 and a.dtype == R.MLRA_BF16


def test_binding_refuses_int64_lengths():
    # int64 [777, 1500] read as int32 would be [777, 0]: refused before any call
    with pytest.raises(TypeError, match="seq_lens"):
        _make(seq_lens=torch.tensor([777, 1500]))
    with pytest.raises(TypeError, match="seq_lens_host"):
        _make(seq_lens_host=torch.tensor([777, 1500]))


def test_binding_refuses_transposed_query():
    q = torch.zeros(2, 4, 8, 4, dtype=torch.bfloat16).transpose(2, 3)   # [B, h, n_b, d_b] view, not contiguous
    with pytest.raises(ValueError, match="q_lat must be contiguous"):
        _make(q_lat=q)


def test_binding_refuses_mixed_dtypes():
    with pytest.raises(TypeError, match="w_v"):
        _make(w_v=torch.zeros(4, 16, 32, dtype=torch.float32))
    with pytest.raises(TypeError, match="q_rope"):
        _make(q_rope=torch.zeros(2, 4, 8, dtype=torch.float32))
    with pytest.raises(TypeError, match="page_table"):
        _make(page_table=torch.zeros(2, 4, dtype=torch.int64))
    with pytest.raises(TypeError, match="error_flags"):
        _make(error_flags=torch.zeros(1, dtype=torch.int64))


def test_binding_refuses_bad_shapes():
    with pytest.raises(ValueError, match="w_v must be"):
        _make(w_v=torch.zeros(4, 16, 31, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="seq_lens holds"):
        _make(seq_lens=torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="unit stride"):
        kv = torch.zeros(2, 8, 40, dtype=torch.bfloat16)
        _make(kv_lat=kv[..., 0:32:2][..., :16].expand(2, 8, 16))


def test_decode_refuses_host_tensors():
    t = _small_tensors()
    with pytest.raises(ValueError, match="GPU"):
        R.decode(t["q_lat"], t["q_rope"], t["kv_lat"], t["kv_rope"], t["seq_lens"], t["w_v"], sm_scale=1.0, alpha=1.0)
    pool = torch.zeros(4, 64, 40, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        R.paged_append(pool, torch.zeros(2, 2, dtype=torch.int32), torch.zeros(2, dtype=torch.int32),
                       torch.zeros(2, 40, dtype=torch.bfloat16), page_size=64)


# ---- planning for the device's topology, and the kernel-choice report ----------------------

def test_plan_reports_the_mfma_path_at_the_headline_shape():
    lens = np.full(16, 32768, dtype=np.int32)
    a = base_args(B=16, L=32768)
    a.seq_lens_host = lens.ctypes.data
    p = R.plan(a, cu_count=256)
    assert p["kernel"] == "mfma" and p["generic_reasons"] == []
    assert p["num_splits"] == 16 and p["work_groups"] == 256 and p["cu_count"] == 256
    assert p["workspace_bytes"] == R.lib().mlra_decode_workspace_size(ctypes.byref(a))
    # without a GPU the current-device plan falls back to the largest gfx950 part
    assert R.plan(a)["cu_count"] in (256, p["cu_count"]) or torch.cuda.is_available()


@pytest.mark.parametrize("cus", [32, 64, 128, 200, 256])
def test_plan_fits_one_group_per_cu_of_a_mocked_device(cus):
    """A partitioned or smaller device gets fewer, longer splits: the groups that hold tokens fit
    one per CU, and the workspace the plan needs never exceeds the size the library reports."""
    rng = np.random.default_rng(cus)
    lens = rng.integers(1000, 40000, size=12).astype(np.int32)
    a = base_args(B=12, L=int(lens.max()))
    a.seq_lens_host = lens.ctypes.data
    p = R.plan(a, cu_count=cus)
    assert p["kernel"] == "mfma" and p["cu_count"] == cus
    assert p["work_groups"] <= cus or p["num_splits"] == 1
    # the workspace size and the call plan for the current device (here the fallback, 256 CUs)
    assert R.plan(a)["workspace_bytes"] == R.lib().mlra_decode_workspace_size(ctypes.byref(a)) or torch.cuda.is_available()


def test_plan_reports_the_generic_kernel_and_why():
    a = base_args(dtype=R.MLRA_F32)
    p = R.plan(a, cu_count=256)
    assert p["kernel"] == "generic" and p["generic_reasons"] == ["dtype"]
    a = base_args(H=32)            # 32 heads: no matrix-core build of this shape
    p = R.plan(a, cu_count=256)
    assert p["kernel"] == "generic" and p["generic_reasons"] == ["shape"]
    a = base_args()
    a.kv_lat += 2                 # misaligned latent rows
    a.kv_rope += 2
    p = R.plan(a, cu_count=256)
    assert p["kernel"] == "generic" and p["generic_reasons"] == ["alignment"]
    assert p["work_groups"] == p["num_splits"] * 2 * 64   # one group per (split, sequence, head)
    a = base_args()
    a.page_table, a.max_pages, a.num_pages = FAKE * 64, 4096 // 8, 4096 // 8 * 2
    a.page_size = 8               # MLRA-4's paged kernel moves 16-token blocks per wave from one page
    p = R.plan(a, cu_count=256)
    assert p["kernel"] == "generic" and p["generic_reasons"] == ["page_size"]
    a.page_size, a.max_pages = 16, 4096 // 16
    assert R.plan(a, cu_count=256)["kernel"] == "mfma"


def test_paged_split_spans_at_most_the_page_id_cache():
    """One long paged context on few CUs: the MLRA-4 split is capped so that it spans at most
    the 64 page ids its kernel keeps in one register (a split may start mid-page)."""
    lens = np.array([1 << 20], dtype=np.int32)
    for ps in (16, 64, 1024):
        a = base_args(B=1, L=1 << 20)
        a.seq_lens_host = lens.ctypes.data
        a.page_table, a.page_size = FAKE * 64, ps
        a.max_pages = a.num_pages = (1 << 20) // ps
        p = R.plan(a, cu_count=32)
        assert p["kernel"] == "mfma"
        assert -(-p["split_tokens"] // ps) + 1 <= 64


def test_plan_rejects_bad_arguments():
    a = base_args()
    info = R.PlanInfo()
    assert R.lib().mlra_decode_plan(ctypes.byref(a), -1, ctypes.byref(info)) == R.MLRA_ERR_INVALID_ARG
    assert R.lib().mlra_decode_plan(ctypes.byref(a), 256, None) == R.MLRA_ERR_INVALID_ARG
    a.batch = 0
    assert R.lib().mlra_decode_plan(ctypes.byref(a), 256, ctypes.byref(info)) == R.MLRA_ERR_INVALID_ARG
