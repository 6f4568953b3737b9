"""Decode-attention benchmark for MLRA-4 (and the MLA / paged / TP-shard workloads).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one full decode call of the library, the attention kernel over
context splits plus the split merge with the W^V epilogue, over one batch of
synthetic input already resident in HBM. Steps rotate among enough identical
copies of the cache (>= 512 MiB in total) that the 256 MiB Infinity Cache cannot
serve them. W untimed steps, then exactly K steps timed by the wall clock with a
device synchronisation on both sides give `value` (decoded tokens/s) and
`ms_per_step`; no timing event sits inside that region.

After it, a separate pass measures the attention kernel alone for the roofline: a
warm-up of back-to-back calls (so that the kernel is timed in the steady state of a
long run, not in the first calls after a synchronisation), then calls that alternate
with and without HIP events recorded by the library around that kernel on its own
stream. The events are created with hipEventDisableSystemFence, so that recording them adds
no system-scope cache write-back and invalidate around the kernel (default events read 4-9%
above rocprofv3's kernel averages, these 1-3%). `roofline.achieved` is the kernel's
algorithmic bytes over the mean event duration; the sample count, median and p10/p90 are
reported with it. The CPU oracle
is timed on a bounded sample on this host (all affinity cores, then one thread), with
the materialised form on a few (sequence, head) rows reported beside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import rank_latent_kv_amd as R  # noqa: E402
from rank_latent_kv_amd.roofline import HBM_PEAK_GBPS, algorithmic_bytes, algorithmic_flops  # noqa: E402
from rank_latent_kv_amd.workloads import PRESETS, make_inputs  # noqa: E402

METRIC = "MLRA-4 decode tokens/s + achieved HBM TB/s (% peak), h=64 L=32k bf16"
DEFAULT_WORKLOAD = "mlra4_b16_l32k"
ROTATE_BYTES = 512 << 20
CALIBRATION_BYTES = 256 << 20
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "rank_latent_kv_amd", "csrc", f) for f in ("attn_mfma.hip", "mlra_api.cpp")]


def code_tokens(text: str) -> str:
    """C++ source without its comments and with whitespace collapsed: what the compiler sees,
    so that a comment edit does not void the stored counter figures. String literals are kept
    whole (a "//" inside one is not a comment)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"' or c == "'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the attention kernel's and the planner's code (comments and whitespace ignored)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, encoding="utf-8") as fh:
            h.update(code_tokens(fh.read()).encode())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, launches_bytes: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    if there is none for this workload or the kernel sources changed since."""
    try:
        with open(PMC_SUMMARY) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    e = d.get(workload)
    if not e or e.get("kernel_source_hash") != kernel_source_hash():
        return None
    return e.get("hbm_bytes_per_launch")


def setup(w, inp, dev, copies):
    d = {k: v.to(dev) for k, v in inp.items() if k not in ("kv", "pool")}
    big = inp["pool"] if w.paged else inp["kv"]
    caches = [big.to(dev)]
    for _ in range(copies - 1):
        caches.append(caches[0].clone())
    return d, caches


def make_step_args(w, d, cache, out, ws, lens_host, events=None):
    dc = w.latent_dim
    kv_lat, kv_rope = cache[..., :dc], cache[..., dc:]
    kw = dict(sm_scale=w.sm_scale, alpha=w.alpha, out=out, workspace=ws, seq_lens_host=lens_host, events=events)
    if w.paged:
        kw.update(page_table=d["page_table"], page_size=w.page_size, num_pages=cache.shape[0],
                  row_stride=cache.shape[-1], max_seq_len=int(lens_host.max()))
    return R.make_args(d["q_lat"], d["q_rope"], kv_lat, kv_rope, d["seq_lens"], d["w_v"], **kw)


def _oracle_rows(w, inp, beta):
    """Sequence beta's cached rows as fp64 [1, L, row] (gathered through the page table when paged)."""
    L = int(inp["seq_lens"][beta])
    if w.paged:
        pool = inp["pool"]
        n = -(-L // w.page_size)
        ids = torch.from_numpy(inp["page_table"].numpy()[beta, :n]).long()
        rows = pool[ids].reshape(1, -1, pool.shape[-1])[:, :L]
    else:
        rows = inp["kv"][beta:beta + 1, :L]
    return rows.double().numpy()


def _oracle_pass(w, inp, budget_s: float, max_seqs: int = 10 ** 6):
    """Whole sequences of the batch through the absorbed-form oracle, pass after pass, until
    the budget is spent (at least one). Returns (sequences, seconds, y of the first pass)."""
    from oracle import mlra_oracle as O
    lens = inp["seq_lens"].numpy()
    dc = w.latent_dim
    w_v = inp["w_v"].double().numpy()
    done, ys = 0, []
    t0 = time.perf_counter()
    for step in range(max_seqs):
        beta = step % w.batch
        rows = _oracle_rows(w, inp, beta)
        y = O.mlra_decode_absorbed(inp["q_lat"][beta:beta + 1].double().numpy(),
                                   inp["q_rope"][beta:beta + 1].double().numpy(), rows[:, :, :dc], rows[:, :, dc:],
                                   lens[beta:beta + 1], w_v, w.sm_scale, w.alpha)
        if step < w.batch:
            ys.append(y[0])
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    return done, time.perf_counter() - t0, ys


def cpu_baseline(w, inp, budget_s: float):
    """The CPU oracle as it stands, timed on this host. Returns (cpu_baseline dict, y of the
    sequences the first pass covered).

    - value: the absorbed-form fp64 oracle over whole sequences, pass after pass for about
      budget_s, with the BLAS pool allowed every core of this process's affinity set;
    - single_thread: the same on one thread, over one sequence;
    - materialised_subset: the materialised form (per-branch keys and values built from the
      non-absorbed up-projections) on sequence 0 and a seeded set of 4 heads, with its largest
      relative difference from the absorbed form on those rows."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import mlra_oracle as O
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        done, dt, ys = _oracle_pass(w, inp, budget_s)
    with threadpool_limits(limits=1):
        done1, dt1, _ = _oracle_pass(w, inp, 0.0, max_seqs=1)
        rng = np.random.Generator(np.random.PCG64(11))
        heads = sorted(rng.choice(w.heads, size=min(4, w.heads), replace=False).tolist())
        rows = _oracle_rows(w, inp, 0)
        q_lat = inp["q_lat"][0:1].double().numpy()
        q_nope, w_k = O.absorption_consistent_query(q_lat, max(w.head_dim, w.latent_dim), rng)
        t0 = time.perf_counter()
        ym = O.mlra_decode_materialised(q_nope, w_k, inp["q_rope"][0:1].double().numpy(), rows[:, :, :w.latent_dim],
                                        rows[:, :, w.latent_dim:], inp["seq_lens"].numpy()[0:1],
                                        inp["w_v"].double().numpy(), w.sm_scale, w.alpha, w.branches,
                                        seqs=[0], heads=heads)
        dtm = time.perf_counter() - t0
    ya = ys[0][heads]
    mat_err = float(np.max(np.abs(ym[0, heads] - ya)) / max(float(np.max(np.abs(ya))), 1e-300))
    L0 = int(inp["seq_lens"][0])
    out = {"value": done / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": f"{done} whole-context sequences (passes over the {w.batch}-sequence batch), fp64 numpy "
                     f"absorbed-form oracle, {dt:.1f} s, BLAS threads {blas_threads} of {cores} affinity cores",
           "blas_threads": blas_threads,
           "single_thread": {"value": done1 / dt1, "unit": "tokens/s", "seconds": dt1,
                             "sample": f"{done1} sequence(s) on one thread"},
           "materialised_subset": {"seconds": dtm, "rows": f"sequence 0 (L={L0}) x heads {heads}",
                                   "max_rel_diff_vs_absorbed": mat_err}}
    return out, np.stack(ys)


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence (hip_runtime_api.h)


class TimingEvents:
    """Pairs of HIP events for timing only, made through the HIP runtime that torch has already
    loaded (the same soname, so no second copy): torch's events take no creation flags."""

    def __init__(self, n: int):
        import ctypes
        self._c = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pairs = [(self._create(), self._create()) for _ in range(n)]

    def _create(self) -> int:
        e = self._c.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self._c.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed with HIP error {rc}")
        return e.value

    def elapsed_ms(self) -> list:
        out = []
        for e0, e1 in self.pairs:
            ms = self._c.c_float()
            rc = self.hip.hipEventElapsedTime(self._c.byref(ms), e0, e1)
            if rc != 0:
                raise RuntimeError(f"hipEventElapsedTime failed with HIP error {rc}")
            out.append(ms.value)
        return out

    def destroy(self) -> None:
        for pair in self.pairs:
            for e in pair:
                self.hip.hipEventDestroy(e)
        self.pairs = []


def event_pass(fn, args_list, ev_args, stream, warm: int, samples: int):
    """Time the attention kernel alone: `warm` back-to-back calls, then 2 * samples calls
    alternating an event-bracketed call with a plain one. Returns the event durations in us."""
    import ctypes
    n = len(args_list)
    for k in range(warm):
        fn(ctypes.byref(args_list[k % n]), stream)
    for j in range(samples):
        fn(ctypes.byref(ev_args[j]), stream)
        fn(ctypes.byref(args_list[j % n]), stream)
    return ev_args


def reduce_pmc(workload: str, fetch_csv: str, write_csv: str, command: str) -> str:
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE,
    both with --calibration-copy) into HBM bytes per attention launch.

    Both counters are in KiB per dispatch. Each is scaled by the factor that makes
    it read CALIBRATION_BYTES for the first three large plain device copies of the
    run (the calibration copies; a copy reads and writes that many bytes).
    Records the result, keyed by workload and the attention kernel's source hash,
    in profiles/pmc_traffic.json and returns a Markdown summary."""
    import csv
    from rank_latent_kv_amd.workloads import default_seq_lens

    def load(path, counter):
        out = []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        return sorted(out)

    def calibration(rows):
        big = [v for _, k, v in rows if "copyBuffer" in k and v * 1024 > CALIBRATION_BYTES / 8][:3]
        if len(big) < 3:
            raise SystemExit("no calibration copies in the counter file: run bench.py with --calibration-copy")
        return CALIBRATION_BYTES / (1024.0 * float(np.mean(big))), big

    def kernel_mean(rows, name):
        v = [x for _, k, x in rows if name in k]
        return float(np.mean(v)) if v else float("nan"), len(v)

    fetch, write = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
    ff, fbig = calibration(fetch)
    wf, wbig = calibration(write)
    w = PRESETS[workload]
    ab = algorithmic_bytes(w, default_seq_lens(w).tolist())
    lines = [f"# HBM traffic per launch, {workload}", "",
             "Made by (two passes, FETCH_SIZE then WRITE_SIZE):", "", "```", command, "```", "",
             f"Calibration: {CALIBRATION_BYTES >> 20} MiB device copies read FETCH_SIZE "
             f"{', '.join('%.0f' % v for v in fbig)} KiB (factor {ff:.3f}) and WRITE_SIZE "
             f"{', '.join('%.0f' % v for v in wbig)} KiB (factor {wf:.3f}).", "",
             "| kernel | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled HBM bytes | algorithmic bytes | ratio |",
             "|---|---|---|---|---|---|---|"]
    entry = None
    for kname, alg in (("attn_mfma_kernel", ab["attention_kernel"]), ("attn_generic_kernel", ab["attention_kernel"]),
                       ("merge_mfma_kernel", None), ("merge_kernel", None)):
        fm, n = kernel_mean(fetch, kname)
        wm, _ = kernel_mean(write, kname)
        if n == 0:
            continue
        hbm = fm * 1024 * ff + wm * 1024 * wf
        lines.append(f"| {kname} | {n} | {fm:.0f} | {wm:.0f} | {hbm:.4g} | "
                     f"{'%.4g' % alg if alg else '-'} | {'%.3f' % (hbm / alg) if alg else '-'} |")
        if alg and entry is None:
            entry = {"kernel": kname, "kernel_source_hash": kernel_source_hash(), "hbm_bytes_per_launch": hbm,
                     "fetch_kib_per_launch": fm, "write_kib_per_launch": wm, "fetch_factor": ff,
                     "write_factor": wf, "algorithmic_bytes_per_launch": alg, "command": command}
    try:
        with open(PMC_SUMMARY) as f:
            d = json.load(f)
    except (OSError, ValueError):
        d = {}
    if entry is not None:
        d[workload] = entry
        with open(PMC_SUMMARY, "w") as f:
            json.dump(d, f, indent=1, sort_keys=True)
            f.write("\n")
    return "\n".join(lines) + "\n"


def read_probe(sizes=(167_772_160, 536_870_912), calls=400, warmup=2000):
    """The box's practical streaming-read rate: the library's read probe (one coalesced
    stream of 16-byte nontemporal loads) over buffers of the headline and TP-shard cache
    sizes, rotating enough copies (>= 512 MiB) that the Infinity Cache cannot serve them,
    timed with events around all calls after a warm-up as long as the decode bench's."""
    dev = torch.device("cuda:0")
    res = []
    for nbytes in sizes:
        copies = max(1, math.ceil(ROTATE_BYTES / nbytes))
        bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(copies)]
        out = torch.empty(int(R.lib().mlra_read_probe_words()), dtype=torch.int32, device=dev)
        for k in range(warmup):
            R.read_probe(bufs[k % copies], out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for k in range(calls):
            R.read_probe(bufs[k % copies], out)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / calls
        res.append({"bytes": nbytes, "us_per_read": us, "tbps": nbytes / us / 1e6, "copies": copies})
        del bufs
        torch.cuda.empty_cache()
    return {"read_probe": res, "peak_tbps": HBM_PEAK_GBPS / 1e3, "op": "mlra_read_probe"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=2000,
                    help="untimed steps first: under back-to-back decode calls the GPU takes some 25-30 ms "
                         "(about 500 headline calls) to settle its clocks, and shorter warm-ups time that ramp")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(PRESETS))
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--batch", type=int, default=0, help="override the workload's batch (reported in config)")
    ap.add_argument("--seq-len", type=int, default=0, help="override every sequence's length (reported in config)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--event-samples", type=int, default=40,
                    help="event-bracketed attention-kernel launches in the roofline pass after the timed region")
    ap.add_argument("--event-warmup", type=int, default=1000,
                    help="back-to-back calls before the roofline samples, so that they see the steady state")
    ap.add_argument("--prepare", action="store_true",
                    help="time the prepare step (query absorption, RoPE, new cache row) before each decode call")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="first run a plain 256 MiB device-to-device copy (reference for HBM byte counters)")
    ap.add_argument("--pmc-reduce", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: reduce two rocprofv3 counter files of --workload into profiles/")
    ap.add_argument("--pmc-command", default="", help="with --pmc-reduce: the command that made the files")
    ap.add_argument("--read-probe", action="store_true",
                    help="only measure this GPU's streaming-read rate (the library's read probe over rotated "
                         "buffers of the headline and TP-shard cache sizes) and print it as one JSON line")
    args = ap.parse_args()

    if args.pmc_reduce:
        text = reduce_pmc(args.workload, args.pmc_reduce[0], args.pmc_reduce[1], args.pmc_command)
        out = os.path.join(ROOT, "profiles", f"attn_mfma_kernel_{args.workload}_hbm_traffic.md")
        with open(out, "w") as f:
            f.write(text)
        print(text)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "bench.py measures one GPU: the decode kernel runs on one GPU's share of "
                                   "the work; sharding across GPUs is described but not implemented"}))
        sys.exit(2)
    if args.read_probe:
        print(json.dumps(read_probe()))
        return

    w = PRESETS[args.workload]
    if args.batch:
        w = w.replace(batch=args.batch)
    if args.seq_len:
        w = w.replace(seq_len=args.seq_len, seq_len_range=None)
    dev = torch.device("cuda:0")
    if args.calibration_copy:
        # before any other device copy, so the counter summary can find these three
        src = torch.empty(CALIBRATION_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    inp = make_inputs(w)
    lens = inp["seq_lens"]
    lens_host = lens.to(torch.int32).contiguous()
    ab = algorithmic_bytes(w, lens.tolist())
    af = algorithmic_flops(w, lens.tolist())
    cache_bytes = (inp["pool"] if w.paged else inp["kv"]).numel() * w.elem_bytes
    copies = max(1, math.ceil(ROTATE_BYTES / cache_bytes))
    d, caches = setup(w, inp, dev, copies)
    outs = [torch.empty((w.batch, w.heads, w.head_dim), dtype=torch.bfloat16, device=dev) for _ in range(copies)]
    a0 = make_step_args(w, d, caches[0], outs[0], None, lens_host)
    a0.num_splits = args.num_splits
    ws = torch.empty(R.workspace_size(a0), dtype=torch.uint8, device=dev)
    K, W = args.steps, args.warmup
    step_args = []
    for k in range(K):
        c = k % copies
        a = make_step_args(w, d, caches[c], outs[c], ws, lens_host)
        a.num_splits = args.num_splits
        step_args.append(a)
    # the roofline pass: HIP events recorded by the library around the attention kernel alone
    n_ev = max(20, args.event_samples)
    tev = TimingEvents(n_ev)
    ev_args = []
    for j, (e0, e1) in enumerate(tev.pairs):
        a = make_step_args(w, d, caches[(j + 1) % copies], outs[(j + 1) % copies], ws, lens_host,
                           events=(e0, e1))
        a.num_splits = args.num_splits
        ev_args.append(a)
    warm_args = []
    for k in range(W):
        a = make_step_args(w, d, caches[k % copies], outs[k % copies], ws, lens_host)
        a.num_splits = args.num_splits
        warm_args.append(a)
    stream = torch.cuda.current_stream().cuda_stream
    L = R.lib()
    import ctypes
    fn = L.mlra_decode
    prep_args = {}
    if args.prepare:
        # one new token per sequence at the last position: its absorbed query and rotated RoPE query feed
        # the decode (written into the same q_lat / q_rope buffers), its row goes into the cache copy
        g = torch.Generator().manual_seed(7)
        bf = lambda *shape, s=1.0: (torch.randn(shape, generator=g) * s).to(torch.bfloat16).to(dev)
        q_nope, q_pe = bf(w.batch, w.heads, w.head_dim), bf(w.batch, w.heads, w.rope_dim, s=w.std)
        w_uk_t = bf(w.heads, w.latent_dim, w.head_dim, s=w.head_dim ** -0.5)
        c_new, k_pe_new = bf(w.batch, w.latent_dim, s=w.std), bf(w.batch, w.rope_dim, s=w.std)
        positions = (lens - 1).to(torch.int32)
        pos_d = positions.to(dev)
        kw = {}
        if w.paged:
            kw = dict(page_table=d["page_table"], page_size=w.page_size, num_pages=caches[0].shape[0])
        for c in range(copies):
            cc = caches[c].view(-1, caches[c].shape[-1])[None] if w.paged else caches[c]
            prep_args[c] = R.make_prepare_args(q_nope, q_pe, w_uk_t, c_new, k_pe_new, pos_d,
                                               cc[..., :w.latent_dim], cc[..., w.latent_dim:],
                                               num_branches=w.branches, q_lat=d["q_lat"], q_rope=d["q_rope"],
                                               positions_host=positions, **kw)
    fprep = L.mlra_decode_prepare

    torch.cuda.synchronize()
    for k, a in enumerate(warm_args):
        if prep_args:
            st = fprep(ctypes.byref(prep_args[k % copies]), stream)
            if st != 0:
                raise R.MlraError(st, R.last_error())
        st = fn(ctypes.byref(a), stream)
        if st != 0:
            raise R.MlraError(st, R.last_error())
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if prep_args:
        for k, a in enumerate(step_args):
            fprep(ctypes.byref(prep_args[k % copies]), stream)
            fn(ctypes.byref(a), stream)
    else:
        for a in step_args:
            fn(ctypes.byref(a), stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if R.last_error():
        raise RuntimeError(R.last_error())
    step_s = (t1 - t0) / K
    y_last = outs[(K - 1) % copies].float().cpu().double().numpy()

    # roofline pass, after the timed region: its warm-up and events do not touch ms_per_step
    event_pass(fn, step_args, ev_args, stream, args.event_warmup, n_ev)
    torch.cuda.synchronize()
    if R.last_error():
        raise RuntimeError(R.last_error())
    attn_ms = np.array(tev.elapsed_ms())
    tev.destroy()
    attn_s = float(np.mean(attn_ms)) * 1e-3

    tokens_per_s = w.batch / step_s
    achieved_gbps = ab["attention_kernel"] / attn_s / 1e9
    step_gbps = ab["total"] / step_s / 1e9
    traffic = stored_traffic(w.name, ab["attention_kernel"])

    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1)/sqrt(d_b+d_R) cache and queries, N(0,0.02) W^V)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "branches": w.branches,
                   "branch_dim": w.branch_dim, "rope_dim": w.rope_dim, "head_dim": w.head_dim,
                   "seq_lens": "all %d" % w.seq_len if w.seq_len else "U[%d,%d]: %s" % (
                       w.seq_len_range[0], w.seq_len_range[1], lens.tolist()),
                   "paged": w.paged, "cache_copies_rotated": copies, "num_splits": args.num_splits or "auto",
                   "step": "prepare + decode" if args.prepare else "decode"},
        "hbm_tbps_step": step_gbps / 1e3,
        "pct_hbm_peak_step": 100.0 * step_gbps / HBM_PEAK_GBPS,
        "roofline": {"bound": "hbm", "achieved": achieved_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic,
                     "kernel": "attn_mfma_kernel", "algorithmic_bytes_per_launch": ab["attention_kernel"],
                     "avg_launch_us": attn_s * 1e6, "median_us": float(np.median(attn_ms)) * 1e3,
                     "p10_us": float(np.percentile(attn_ms, 10)) * 1e3,
                     "p90_us": float(np.percentile(attn_ms, 90)) * 1e3,
                     "event_samples": len(attn_ms), "event_pass": f"after the timed region: {args.event_warmup} "
                     f"back-to-back calls, then {n_ev} event-bracketed calls each followed by a plain one; "
                     "events without the system-scope fence",
                     "mfma_tflops": af["attention"] / attn_s / 1e12},
    }

    # parity of this exact launch configuration against the oracle on the sampled sequences
    if not args.no_cpu_baseline:
        cb, yref = cpu_baseline(w, inp, args.cpu_budget)
        yg = y_last[:len(yref)]
        num = np.max(np.abs(yg - yref), axis=-1)
        den = np.maximum(np.max(np.abs(yref), axis=-1), 1e-30)
        result["cpu_baseline"] = cb
        # with --prepare the decode ran on the prepared queries and cache row, not on these inputs
        result["parity_max_row_rel_err"] = None if args.prepare else float(np.max(num / den))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
