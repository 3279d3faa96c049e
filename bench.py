"""Benchmark of the DSA sparse-attention step on one MI355X.

A step is one pass of the whole hot path over one batch: indexer scoring,
head weighting, Top-K selection and sparse attention (``dsa_fused_decode``).
Inputs are seeded synthetic tensors already resident in HBM; the caches are
replicated R times (different addresses, same content) and the steps rotate
over the replicas so the 256 MB Infinity Cache cannot hold the working set.

Prints ONE JSON line (rank 0).  ``roofline`` is for the dominant stage; its
duration is measured with HIP events recorded on the stream the library
launches on.  ``cpu_baseline`` times the CPU oracle on the host cores on a
bounded sample of the same workload and checks the GPU result against it.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from lightning_indexer_top_02_amd import dsa, inputs  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp8": 5000.0}  # dense, MI355X
VALU_F32_PEAK_TFLOPS = 157.3  # fp32 routes run on the vector ALUs
METRIC = "DSA decode tokens/s + HBM GB/s (% peak) at 32K ctx; prefill indexer MFMA util"

WORKLOADS = {
    "decode_32k": dict(
        make=lambda dev, batch=1: inputs.decode_32k(batch=batch, device=dev),
        desc="DSA decode step: batch {batch}, 1 query token, context 32768 in 512 shuffled 64-token "
             "pages; indexer 64 heads x 128 bf16, Top-K 2048; sparse attention 128 heads x "
             "(512+64) bf16 latent, bf16 out, fp32 accumulation"),
    "decode_32k_kv8": dict(
        make=lambda dev, batch=1: inputs.decode_32k(batch=batch, device=dev, sfa_dtype="fp8",
                                                    name=f"decode_32k_kv8_b{batch}"),
        desc="DSA decode step: batch {batch}, 1 query token, context 32768 in 512 shuffled 64-token "
             "pages; indexer 64 heads x 128 bf16, Top-K 2048; sparse attention 128 heads over an fp8 "
             "latent cache (512 e4m3 + 16-byte block of E8M0 tile exponents + 64 bf16 rope = 656 bytes a "
             "row), bf16 q "
             "and out, fp32 accumulation"),
    "batched_fp8_narrow_kv8": dict(
        make=lambda dev, batch=64: inputs.batched_decode_fp8(device=dev, batch=batch, sfa_dtype="fp8",
                                                             name="batched_fp8_narrow_kv8"),
        desc="DSA decode step: batch {batch}, contexts U[4096,131072], fp8 indexer 4 x 64, Top-K 2048, "
             "sparse attention 16 heads over an fp8 latent cache (656-byte rows), bf16 q and out"),
    "tiny_decode": dict(
        make=lambda dev, batch=1: inputs.tiny_decode(device=dev),
        desc="DSA decode step: batch 1, context 4096, fp32 indexer 4 x 64, Top-K 256, fp32 "
             "sparse attention 16 heads"),
    "batched_fp8_narrow": dict(
        make=lambda dev, batch=64: inputs.batched_decode_fp8(device=dev, batch=batch),
        desc="DSA decode step: batch {batch}, contexts U[4096,131072], fp8 indexer 4 x 64, Top-K 2048, "
             "bf16 sparse attention 16 heads"),
    "batched_fp8_wide": dict(
        make=lambda dev, batch=64: inputs.batched_decode_fp8(device=dev, batch=batch, wide=True),
        desc="DSA decode step: batch {batch}, contexts U[4096,131072], fp8 indexer 64 x 128, Top-K "
             "2048, bf16 sparse attention 128 heads"),
    "chunked_prefill": dict(
        make=lambda dev, batch=1, sfa=True: inputs.chunked_prefill(device=dev, **({} if sfa else
                                                                                 {"sfa_dtype": None})),
        desc="DSA chunked-prefill step: 4096 query tokens appended to a 61440-token prefix (65536 "
             "positions, causal), indexer 64 heads x 128 bf16, Top-K 2048 per row, sparse attention "
             "128 heads x (512+64) bf16"),
    "batched_mxfp8_wide": dict(
        make=lambda dev, batch=64: inputs.batched_decode_fp8(device=dev, batch=batch, wide=True, idx_dtype="mxfp8",
                                                             name="batched_mxfp8_wide"),
        desc="DSA decode step: batch {batch}, contexts U[4096,131072], MXFP8 indexer 64 x 128 (e4m3 with one "
             "E8M0 scale per 32 elements of q and k), Top-K 2048, bf16 sparse attention 128 heads"),
    "chunked_prefill_mxfp8": dict(
        make=lambda dev, batch=1, sfa=True: inputs.chunked_prefill(
            device=dev, idx_dtype="mxfp8", name="prefill_61440+4096_mxfp8", **({} if sfa else {"sfa_dtype": None})),
        desc="DSA chunked-prefill step: 4096 query tokens appended to a 61440-token prefix (65536 "
             "positions, causal), MXFP8 indexer 64 heads x 128 (one E8M0 scale per 32 elements), Top-K "
             "2048 per row, sparse attention 128 heads x (512+64) bf16"),
    "scratch_prefill": dict(
        make=lambda dev, batch=1, sfa=True: inputs.chunked_prefill(
            device=dev, prefix=0, new=16384, name="prefill_0+16384_bf16", **({} if sfa else {"sfa_dtype": None})),
        desc="DSA prefill from scratch: one request of 16384 tokens, every one a causal query row (row i "
             "sees i + 1 positions), indexer 64 heads x 128 bf16, Top-K 2048 per row, sparse attention "
             "128 heads x (512+64) bf16"),
    "spec_verify": dict(
        make=lambda dev, batch=16: inputs.spec_verify(device=dev, batch=batch),
        desc="DSA speculative-verify step: {batch} requests x 4 causal query tokens at context "
             "262144, fp8 indexer 64 x 128, Top-K 2048, bf16 sparse attention 128 heads"),
}


def elem_bytes(dtype):
    return {"f32": 4, "bf16": 2, "fp8": 1, "mxfp8": 1}[dtype]


def scale_bytes(dtype, dim):
    """Scale bytes per indexer vector (a q (row, head) or a key)."""
    return {"fp8": 4, "mxfp8": dim // 32}.get(dtype, 0)


def visible_per_row(case: inputs.Case):
    """Positions each query row sees (its request's length minus the rows after it)."""
    qo = case.q_offsets.cpu().tolist()
    lens = case.ctx_lens.cpu().tolist()
    return [lens[b] - (qo[b + 1] - qo[b]) + j + 1 for b in range(len(lens)) for j in range(qo[b + 1] - qo[b])]


def algorithmic_bytes(case: inputs.Case):
    """Bytes (and flops) the method itself needs per step, per stage.

    indexer: every visible key once per request (head dim x element size,
             plus its scale bytes: fp8 4, MXFP8 one per 32 elements), q, w
             (and q scales), the block
             table, and the Top-K indices written; flops = 2 H_I D_I per
             visible (row, position) pair (the logits).
    sparse attention: the indices read, the latent rows gathered (each cached
             row of a request at most once: min(sum over its rows of the
             rows each selects, its length)), q and the output; flops =
             2 H_q (576 + 512) per selected (query row, cached row) pair.
    """
    lens = case.ctx_lens.cpu().tolist()
    qo = case.q_offsets.cpu().tolist()
    T, K = case.num_tokens, case.topk
    eK = elem_bytes(case.idx_dtype)
    sb = scale_bytes(case.idx_dtype, case.head_dim_idx)
    key_row = case.head_dim_idx * eK + sb
    H = case.n_heads_idx
    idx_bytes = (sum(lens) * key_row + T * H * case.head_dim_idx * eK + T * H * (4 + sb)
                 + sum((L + 63) // 64 for L in lens) * 4 + T * K * 4)
    eS = elem_bytes(case.sfa_dtype) if case.sfa_dtype != "none" else 0
    # latent row bytes; the fp8 latent route has bf16 q and out
    row_bytes = (case.v_dim + 16 + 2 * (case.qk_dim - case.v_dim) if case.sfa_dtype == "fp8"
                 else case.qk_dim * eS)
    eIO = 2 if case.sfa_dtype == "fp8" else eS
    vis = visible_per_row(case)
    sel = sum(min(v, K) for v in vis)
    rows_read = sum(min(sum(min(v, K) for v in vis[qo[b]:qo[b + 1]]), lens[b]) for b in range(len(lens)))
    sfa_bytes = (T * K * 4 + rows_read * row_bytes + T * case.n_heads_sfa * (case.qk_dim + case.v_dim) * eIO)
    idx_flops = 2 * sum(vis) * H * case.head_dim_idx
    sfa_flops = 2 * sel * case.n_heads_sfa * (case.qk_dim + case.v_dim)
    return {"indexer": idx_bytes, "sparse_attn": sfa_bytes, "total": idx_bytes + sfa_bytes,
            "indexer_flops": idx_flops, "sparse_attn_flops": sfa_flops}


def compute_peak(dtype: str) -> float:
    return MFMA_PEAK_TFLOPS.get(dtype, VALU_F32_PEAK_TFLOPS)


def roofline_entry(kernel: str, workload: str, nbytes: float, flops: float, ms: float, peak_tflops: float):
    """Roofline of one kernel (or call): the bound is whichever of HBM bytes
    at 8 TB/s and flops at the compute peak takes longer; achieved is the
    algorithmic figure over the measured duration."""
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_cmp = flops / (peak_tflops * 1e12)
    sec = ms * 1e-3
    if t_cmp > t_hbm:
        ach = flops / sec / 1e12
        return {"kernel": kernel, "bound": "mfma" if peak_tflops != VALU_F32_PEAK_TFLOPS else "alu",
                "achieved": ach, "peak": peak_tflops, "unit": "TFLOP/s", "frac": ach / peak_tflops,
                "traffic": measured_traffic(kernel, workload), "algorithmic_flops": flops,
                "algorithmic_bytes": nbytes, "kernel_ms": ms}
    ach = nbytes / sec / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": ach / HBM_PEAK_GBS, "traffic": measured_traffic(kernel, workload),
            "algorithmic_bytes": nbytes, "algorithmic_flops": flops, "kernel_ms": ms}


class Step:
    """Preallocated buffers for one workload and R cache replicas."""

    def __init__(self, case: inputs.Case, replicas: int):
        self.case = case
        self.R = replicas
        self.k = [case.k_cache] + [case.k_cache.clone() for _ in range(replicas - 1)]
        self.ks = ([case.k_scale] + [case.k_scale.clone() for _ in range(replicas - 1)]
                   if case.k_scale is not None else [None] * replicas)
        self.kv = ([case.kv_cache] + [case.kv_cache.clone() for _ in range(replicas - 1)]
                   if case.kv_cache is not None else [None] * replicas)
        dev = case.q_idx.device
        T, K = case.num_tokens, case.topk
        self.idx = torch.empty((T, K), dtype=torch.int32, device=dev)
        if case.sfa_dtype != "none":
            odt = torch.float32 if case.sfa_dtype == "f32" else torch.int16
            self.out = torch.empty((T, case.n_heads_sfa, case.v_dim), dtype=odt, device=dev)
            self.lse = torch.empty((T, case.n_heads_sfa), dtype=torch.float32, device=dev)
        self.paged = dsa.make_paged(case.q_offsets, case.ctx_lens, case.block_table, case.num_pages,
                                    max_q_per_req=case.max_q_per_req, max_ctx_len=case.max_ctx,
                                    num_q_tokens=T)
        self.indexers = [dsa.make_indexer(case.q_idx, case.weights, self.k[r], K, case.idx_dtype,
                                          q_scale=case.q_scale, k_scale=self.ks[r]) for r in range(replicas)]
        self.scores = None
        if case.sfa_dtype == "none":  # scoring only
            self.sfas = None
            return
        self.sfas = [dsa.make_sfa(case.q_sfa, self.kv[r], self.out, case.scale, case.sfa_dtype, lse=self.lse,
                                  v_dim=case.v_dim) for r in range(replicas)]
        n_fused = dsa.fused_decode_workspace_size(self.paged, self.indexers[0], self.sfas[0])
        n_idx = dsa.indexer_topk_workspace_size(self.paged, self.indexers[0])
        n_sfa = dsa.sparse_attn_workspace_size(self.paged, self.sfas[0], K)
        self.ws = dsa.new_workspace(max(n_fused, n_idx, n_sfa), dev)
        self.ws2 = dsa.new_workspace(n_sfa, dev)

    def fused(self, s: int, stream):
        r = s % self.R
        dsa.fused_decode(self.paged, self.indexers[r], self.sfas[r], topk_idx=self.idx, workspace=self.ws,
                         stream=stream)

    def indexer(self, s: int, stream):
        dsa.indexer_topk(self.paged, self.indexers[s % self.R], self.idx, workspace=self.ws, stream=stream)

    def sparse_attn(self, s: int, stream):
        dsa.sparse_attn(self.paged, self.sfas[s % self.R], self.idx, workspace=self.ws2, stream=stream)

    def scores_only(self, s: int, stream):
        """The indexer's scoring kernel alone (dsa_indexer_scores)."""
        if self.scores is None:
            self.scores = torch.empty((self.case.num_tokens, self.case.max_ctx), dtype=torch.float32,
                                      device=self.case.q_idx.device)
        dsa.indexer_scores(self.paged, self.indexers[s % self.R], self.scores, stream=stream)


def strip_comments(src: str) -> str:
    """C++ source without its comments and blank-line or trailing-space
    differences (the sources hold no string literal with // or /*)."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(line.rstrip() for line in src.splitlines() if line.strip())


def kernel_source_hash() -> str:
    """Hash of the HIP sources' code (comments left out): counter data taken
    on other kernel code is stale."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "lightning_indexer_top_02_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode() + b"\0")
        h.update(strip_comments(open(f, encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE scaled by the copy-kernel factor), or
    None when no summary exists for the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_hash") != kernel_source_hash():
        return None
    return d["bytes_per_launch"]


# HBM byte counters: bytes moved = FETCH_SIZE KiB x FETCH_SCALE + WRITE_SIZE KiB
# x WRITE_SCALE (x 1024), the factors a plain 256 MiB device copy of known
# traffic gives (`--calibrate-copy 256` under rocprofv3 --pmc).
FETCH_SCALE, WRITE_SCALE = 1.999817388043494, 1.0

# The kernels of one call of each measured stage, by name.
KERNEL_GROUPS = {
    "indexer_topk": ("li_fused", "li_score", "li_prefill", "li_seg_gather", "li_seg_resolve", "li_seg_write"),
    "indexer_scores": ("li_prefill",),
    "sparse_attn": ("sfa_bf16", "sfa_f32", "sfa_combine"),
}


def traffic_summary(label: str, fetch_csv: str, write_csv: str, bench_args: str, out_dir: str = "") -> str:
    """Per-launch HBM bytes of each stage from two rocprofv3 counter runs
    (FETCH_SIZE, then WRITE_SIZE, one row per dispatch): the median over
    dispatches of each kernel, summed over the kernels of one call, scaled by
    the copy factors.  Writes profiles/traffic_<stage>_<label>.json (with the
    kernel-source hash they hold for) and returns a markdown summary."""
    per = {}
    for path, ctr in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == ctr:
                    per.setdefault(r["Kernel_Name"], {}).setdefault(ctr, []).append(float(r["Counter_Value"]))

    def median(v):
        v = sorted(v)
        return v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])

    def moved(k):
        return (median(per[k]["FETCH_SIZE"]) * FETCH_SCALE + median(per[k]["WRITE_SIZE"]) * WRITE_SCALE) * 1024

    kern = [k for k in per if "FETCH_SIZE" in per[k] and "WRITE_SIZE" in per[k]]
    cmds = [f"timeout -s KILL 150 rocprofv3 --pmc {c} --output-format csv -d gpurun_out/pmc_{label}_{c} -o run "
            f"-- python3 bench.py {bench_args}" for c in ("FETCH_SIZE", "WRITE_SIZE")]
    lines = [f"# HBM traffic per launch: {label}", "", "Commands (one counter per run, from the repository root;"
             " TMPDIR=/tmp), then `python3 bench.py --traffic-summary` on the two counter files:", "", "```",
             *cmds, "```", "",
             f"Scale factors (256 MiB device copy): FETCH x {FETCH_SCALE:.4f}, WRITE x {WRITE_SCALE:.4f}. "
             f"Kernel sources: hash {kernel_source_hash()}.", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | bytes moved (MB) |", "|---|---|---|---|---|"]
    for k in sorted(kern, key=lambda k: -moved(k)):
        if "dsa::" not in k:
            continue
        lines.append(f"| `{k}` | {len(per[k]['FETCH_SIZE'])} | {median(per[k]['FETCH_SIZE']):.1f} | "
                     f"{median(per[k]['WRITE_SIZE']):.1f} | {moved(k) / 1e6:.2f} |")
    lines.append("")
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    for group, names in KERNEL_GROUPS.items():
        ks = [k for k in kern if any(f"dsa::{n}<" in k or f"dsa::{n}(" in k for n in names)]
        if not ks:
            continue
        nbytes = sum(moved(k) for k in ks)
        rec = {"kernel": group, "workload": label, "source_hash": kernel_source_hash(), "bytes_per_launch": nbytes,
               "launches": ks, "fetch_kib": sum(median(per[k]["FETCH_SIZE"]) for k in ks),
               "write_kib": sum(median(per[k]["WRITE_SIZE"]) for k in ks), "fetch_scale": FETCH_SCALE,
               "write_scale": WRITE_SCALE, "commands": cmds}
        with open(os.path.join(out_dir, f"traffic_{group}_{label}.json"), "w") as f:
            json.dump(rec, f, indent=1)
        lines.append(f"- `{group}` = {' + '.join(f'`{k}`' for k in ks)}: {nbytes / 1e6:.2f} MB per call.")
    return "\n".join(lines) + "\n"


def calibrate_copy(mb: int, reps: int):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    n = mb * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "reps": reps}), flush=True)


def time_steps(fn, steps, stream):
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for s in range(steps):
        fn(s, stream)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_graph(fn, steps, warmup, repeats=5):
    """Capture `steps` calls of fn into one HIP graph (on a side stream) and
    time `repeats` replays with events on the replay stream; the host issues a
    single launch per replay.  Returns the median replay's ms per step."""
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        for s in range(max(1, warmup)):
            fn(s, cs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        for s in range(steps):
            fn(s, cs)
    torch.cuda.synchronize()
    g.replay()  # untimed first replay
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(repeats):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        g.replay()
        end.record(stream)
        torch.cuda.synchronize()
        times.append(start.elapsed_time(end) / steps)
    del g
    return sorted(times)[len(times) // 2]


def stage_breakdown(step: Step, steps, stream):
    """Average duration of each stage, from HIP events around each call."""
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        evs[s][0].record(stream)
        step.indexer(s, stream)
        evs[s][1].record(stream)
        step.sparse_attn(s, stream)
        evs[s][2].record(stream)
    torch.cuda.synchronize()
    idx = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    sfa = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    return idx, sfa


def cache_append_timing(case: inputs.Case, steps: int, stream):
    """dsa_indexer_cache_append of the step's new keys (one per query token,
    fp32 in) into a copy of the K pool in the workload's indexer dtype: the
    producer step before the indexer, `steps` calls replayed as one HIP graph
    and timed with HIP events on the replay stream.  Algorithmic bytes: the fp32 keys read, the stored keys and their
    scales written, and the paging entries read."""
    T, D = case.num_tokens, case.head_dim_idx
    g = torch.Generator(device=case.q_idx.device)
    g.manual_seed(7)
    k_new = torch.randn((T, D), generator=g, device=case.q_idx.device)
    kc = case.k_cache.clone()
    ks = None if case.k_scale is None else case.k_scale.clone()
    paged = dsa.make_paged(case.q_offsets, case.ctx_lens, case.block_table, case.num_pages,
                           max_q_per_req=case.max_q_per_req, max_ctx_len=case.max_ctx, num_q_tokens=T)
    ap = dsa.make_cache_append(k_new, "f32", kc, case.idx_dtype, k_scale=ks)
    fn = lambda s, st: dsa.cache_append(paged, ap, stream=st)  # noqa: E731
    ms = time_graph(fn, steps, 3)  # one graph replay: no host launch gaps
    nbytes = T * D * 4 + T * (D * elem_bytes(case.idx_dtype) + scale_bytes(case.idx_dtype, D)) + T * 4 \
        + case.batch * 12
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {"kernel": "li_cache_append", "keys": T, "dtype": f"f32->{case.idx_dtype}", "ms": ms,
           "algorithmic_bytes": nbytes, "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": gbs / HBM_PEAK_GBS}
    del kc, ks, k_new
    return out


def prefill_scoring(steps: int, warmup: int, stream):
    """MFMA utilisation of the indexer's scoring kernel on the chunked-prefill
    shape (4096 rows x 64 heads x 128 bf16 against 65536 positions, causal):
    useful flops (2 H_I D_I per visible pair) over the kernel's average
    duration from HIP events on the launch stream."""
    case = WORKLOADS["chunked_prefill"]["make"](torch.device("cuda:0"), sfa=False)
    step = Step(case, 1)
    for s in range(warmup):
        step.scores_only(s, stream)
    ms = time_steps(step.scores_only, steps, stream)
    flops = algorithmic_bytes(case)["indexer_flops"]
    tflops = flops / (ms * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[case.idx_dtype]
    out = {"kernel": "indexer scores, row-tiled MFMA (li_prefill)", "workload": WORKLOADS["chunked_prefill"]["desc"],
           "bound": "mfma", "ms": ms, "achieved": tflops, "peak": peak, "unit": "TFLOP/s", "frac": tflops / peak,
           "useful_flops": flops, "traffic": measured_traffic("indexer_scores", "chunked_prefill"),
           "steps": steps, "warmup": warmup}
    del step, case
    torch.cuda.empty_cache()
    return out


def cpu_baseline(case: inputs.Case, step: Step, budget_s: float):
    """The CPU oracle on a bounded sample of the workload (whole steps, or a
    subset of query rows), on this host's cores; also checks the GPU result of
    replica 0 on the same sample."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    import parity

    oracle.build(force=False)
    threads = len(os.sched_getaffinity(0))
    T = case.num_tokens
    rows = list(range(T)) if T <= 4 else sorted({0, T - 1, T // 2, T // 3})
    sub = parity.rows_subcase(case, rows)
    # GPU result of the same rows (replica 0)
    stream = torch.cuda.current_stream()
    step.fused(0, stream)
    torch.cuda.synchronize()
    g_idx = step.idx.clone()
    g_out = step.out.clone()
    t0 = time.perf_counter()
    n = 0
    while True:
        o_idx, o_sc = parity.oracle_indexer(sub, nthreads=threads)
        o_out, _ = parity.oracle_sfa(sub, o_idx, nthreads=threads)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 1000:
            break
    rows_per_s = n * len(rows) / el
    status = "ok"
    try:
        parity.check_rows(case, g_idx, g_out, rows, nthreads=threads)
    except AssertionError as e:
        status = f"MISMATCH: {e}"
    return {"value": rows_per_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} of {T} query rows of the same workload (indexer over the full context, "
                      f"Top-K, sparse attention), repeated {n} times in {el:.1f} s with OpenMP over "
                      f"{threads} host threads",
            "parity_vs_gpu": status}


def replicas_for(case: inputs.Case) -> int:
    """Cache replicas so that the rotated state is at least three times the
    256 MB Infinity Cache (at most 32): each step then reads its caches from
    HBM, as each layer of a model reads its own caches."""
    state = sum(x.numel() * x.element_size() for x in (case.k_cache, case.kv_cache, case.k_scale) if x is not None)
    return max(1, min(32, math.ceil(768e6 / state)))


def measure(name: str, case: inputs.Case, steps: int, warmup: int, eager: bool = False, R: int = 0):
    """One workload's step (dsa_fused_decode) and its two stages, timed as
    the median of 5 graph replays of `steps` steps (or eagerly), with the
    dominant stage's roofline."""
    R = R or replicas_for(case)
    step = Step(case, R)
    ab = algorithmic_bytes(case)
    stream = torch.cuda.current_stream()
    for s in range(warmup):
        step.fused(s, stream)
    torch.cuda.synchronize()
    ms_eager = time_steps(step.fused, steps, stream)
    if eager:
        ms = ms_eager
        t_idx, t_sfa = stage_breakdown(step, steps, stream)
    else:
        # the whole timed region as one HIP graph: no host launch gaps between steps
        ms = time_graph(step.fused, steps, warmup)
        t_idx = time_graph(step.indexer, steps, 1)
        t_sfa = time_graph(step.sparse_attn, steps, 1)
    T = case.num_tokens
    dom = "indexer" if t_idx >= t_sfa else "sparse_attn"
    rows_route = case.max_q_per_req > 4 and T >= 1024 and case.idx_dtype in MFMA_PEAK_TFLOPS
    kernels_ms = {}
    if rows_route:
        # the indexer call is two launches: the scoring GEMM, then per-row selection
        kernels_ms["indexer_scores"] = time_steps(step.scores_only, steps, stream)
    if dom == "indexer" and rows_route:
        roofline = roofline_entry("indexer_scores", name, ab["indexer"], ab["indexer_flops"],
                                  kernels_ms["indexer_scores"], compute_peak(case.idx_dtype))
    elif dom == "indexer":
        roofline = roofline_entry("indexer_topk", name, ab["indexer"], ab["indexer_flops"], t_idx,
                                  compute_peak(case.idx_dtype))
    else:
        roofline = roofline_entry("sparse_attn", name, ab["sparse_attn"], ab["sparse_attn_flops"], t_sfa,
                                  compute_peak("bf16" if case.sfa_dtype == "fp8" else case.sfa_dtype))  # fp8 latent: bf16 MFMAs
    out = {"ms_per_step": ms, "ms_per_step_eager": ms_eager, "tokens_per_s": T / (ms * 1e-3),
           "algorithmic_bytes": ab["total"], "hbm_gbs_step": ab["total"] / (ms * 1e-3) / 1e9,
           "hbm_frac_step": ab["total"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "stages_ms": {"indexer_topk": t_idx, "sparse_attn": t_sfa, **kernels_ms},
           "roofline": roofline, "cache_replicas": R, "steps": steps,
           "timing": "eager launches" if eager else f"median of 5 HIP-graph replays of {steps} steps"}
    return step, out


# The grid of workloads measured beside the headline (the batch x sequence-length
# baselines of the decode and prefill routes): name -> (maker, steps).
GRID = {
    "decode_32k_b2": (lambda dev: inputs.decode_32k(batch=2, device=dev), 100),
    "decode_32k_b4": (lambda dev: inputs.decode_32k(batch=4, device=dev), 100),
    "decode_32k_b8": (lambda dev: inputs.decode_32k(batch=8, device=dev), 50),
    "decode_32k_b32": (lambda dev: inputs.decode_32k(batch=32, device=dev), 20),
    "decode_32k_b64": (lambda dev: inputs.decode_32k(batch=64, device=dev), 20),
    "decode_32k_b128": (lambda dev: inputs.decode_32k(batch=128, device=dev), 10),
    "batched_fp8_narrow": (lambda dev: inputs.batched_decode_fp8(device=dev), 20),
    "batched_fp8_wide": (lambda dev: inputs.batched_decode_fp8(device=dev, wide=True), 20),
    "spec_verify": (lambda dev: inputs.spec_verify(device=dev), 10),
    "chunked_prefill": (lambda dev: inputs.chunked_prefill(device=dev), 5),
}


def grid(dev):
    """Every grid workload: step time, tokens/s, algorithmic GB/s and its
    fraction of 8 TB/s, stage times and the dominant stage's roofline."""
    res = {}
    for name, (make, steps) in GRID.items():
        case = make(dev)
        step, m = measure(name, case, steps, 3)
        m["workload"] = {"name": case.name, "batch": case.batch, "query_tokens": case.num_tokens,
                         "max_context": case.max_ctx, "sum_context": int(case.ctx_lens.sum().item()),
                         "indexer": f"{case.n_heads_idx}x{case.head_dim_idx} {case.idx_dtype}",
                         "sparse_attn": f"{case.n_heads_sfa} heads {case.sfa_dtype}", "topk": case.topk}
        res[name] = m
        print(f"# grid {name}: {m['ms_per_step'] * 1e3:.1f} us/step, {m['tokens_per_s']:.0f} tokens/s", file=sys.stderr,
              flush=True)
        del step, case
        torch.cuda.empty_cache()
    return res


def prolog_overlap(dev, steps: int = 20):
    """The step's two producers before the indexer: the indexer-key append and
    the latent-row append (independent: different pools), either on one
    stream one after the other, or on two same-priority streams at once,
    joined by events before the fused decode.  Two sizes: a 64-request 32K
    decode batch (one new token each) and the chunked prefill (4096 new
    tokens).  Each variant is timed eagerly and as one captured HIP graph
    (the two streams become two graph branches), median of 5 runs of `steps`
    steps."""
    res = {}
    for label, case in (("decode_32k_b64", inputs.decode_32k(batch=64, device=dev)),
                        ("chunked_prefill", inputs.chunked_prefill(device=dev))):
        T = case.num_tokens
        g = torch.Generator(device=dev)
        g.manual_seed(11)
        k_new = torch.randn((T, case.head_dim_idx), generator=g, device=dev)
        x_new = torch.randn((T, 576), generator=g, device=dev) * 0.5
        step = Step(case, 1)
        ak = dsa.make_cache_append(k_new, "f32", step.k[0], case.idx_dtype, k_scale=step.ks[0])
        al = dsa.make_latent_append(x_new, "f32", step.kv[0], case.sfa_dtype)
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()

        def appends(main, two):
            if not two:
                dsa.cache_append(step.paged, ak, stream=main)
                dsa.latent_append(step.paged, al, stream=main)
                return
            s1.wait_stream(main)
            s2.wait_stream(main)
            dsa.cache_append(step.paged, ak, stream=s1)
            dsa.latent_append(step.paged, al, stream=s2)
            main.wait_stream(s1)
            main.wait_stream(s2)

        def run(main, two, with_step):
            appends(main, two)
            if with_step:
                step.fused(0, main)

        def eager(two, with_step):
            main = torch.cuda.current_stream()
            for _ in range(3):
                run(main, two, with_step)
            torch.cuda.synchronize()
            ts = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(main)
                for _ in range(steps):
                    run(main, two, with_step)
                e1.record(main)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) / steps)
            return sorted(ts)[2]

        def graph(two, with_step):
            return time_graph(lambda s_, cs: run(cs, two, with_step), steps, 2)

        r = {"new_tokens": T}
        for with_step in (False, True):
            key = "appends_then_step" if with_step else "appends"
            r[key] = {"one_stream_eager_ms": eager(False, with_step), "two_streams_eager_ms": eager(True, with_step),
                      "one_stream_graph_ms": graph(False, with_step), "two_streams_graph_ms": graph(True, with_step)}
        res[label] = r
        del step, case, k_new, x_new
        torch.cuda.empty_cache()
    res["note"] = ("appends: dsa_indexer_cache_append (fp32 keys -> bf16 pool) and dsa_latent_cache_append "
                   "(fp32 rows -> bf16 latent pool); step: dsa_fused_decode after them")
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_32k", choices=sorted(WORKLOADS))
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--replicas", type=int, default=0,
                    help="cache replicas (0 = enough to exceed three times the 256 MB Infinity Cache)")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle time")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-grid", action="store_true", help="skip the grid of other workloads")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step from the host instead of replaying a captured HIP graph")
    ap.add_argument("--prefill-steps", type=int, default=20,
                    help="steps of the chunked-prefill scoring measurement (0 = skip)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MB",
                    help="only run a plain MB-sized device copy (counter calibration)")
    ap.add_argument("--prolog-only", action="store_true",
                    help="only measure the two cache appends on one stream against two streams")
    ap.add_argument("--traffic-summary", nargs=3, metavar=("LABEL", "FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn two rocprofv3 counter files (FETCH_SIZE, WRITE_SIZE) of a run of "
                         "this script into profiles/traffic_<stage>_LABEL.json and print a summary")
    ap.add_argument("--traffic-bench-args", default="",
                    help="the bench.py arguments of the profiled run (recorded with the summary)")
    args = ap.parse_args()
    if args.traffic_summary:
        print(traffic_summary(*args.traffic_summary, args.traffic_bench_args), end="")
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, 10)
        return
    if args.prolog_only:
        print(json.dumps({"prolog_overlap": prolog_overlap(dev, args.steps)}), flush=True)
        return

    w = WORKLOADS[args.workload]
    kw = {} if args.batch is None else {"batch": args.batch}
    case = w["make"](dev, **kw)
    stream = torch.cuda.current_stream()
    step, m = measure(args.workload, case, args.steps, args.warmup, args.eager, args.replicas)
    T = case.num_tokens
    result = {
        "metric": METRIC,
        "value": m["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.idx_dtype if case.idx_dtype == case.sfa_dtype else f"{case.idx_dtype}+{case.sfa_dtype}",
        "data": "synthetic",
        "config": {"workload": w["desc"].format(batch=case.batch), "name": case.name, "batch": case.batch,
                   "query_tokens": T, "max_context": case.max_ctx, "topk": case.topk,
                   "cache_replicas": m["cache_replicas"], "parallelism": "single GPU",
                   "launch": "eager" if args.eager else "hip_graph", "timing": m["timing"]},
        "ms_per_step_eager": m["ms_per_step_eager"],
        "hbm_gbs_step": m["hbm_gbs_step"],
        "hbm_frac_step": m["hbm_frac_step"],
        "stages_ms": m["stages_ms"],
        "roofline": m["roofline"],
        "cache_append": cache_append_timing(case, args.steps, stream),
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu:
        # the correctness gate first, on the headline workload's own result
        result["cpu_baseline"] = cpu_baseline(case, step, args.cpu_budget)
        if result["cpu_baseline"]["parity_vs_gpu"] != "ok":
            # a result that fails the correctness gate yields no throughput figure
            result["value"] = None
            print(json.dumps(result), flush=True)
            sys.exit(1)
    del step, case
    torch.cuda.empty_cache()
    if args.prefill_steps and args.workload != "chunked_prefill":
        result["prefill_indexer_mfma"] = prefill_scoring(args.prefill_steps, max(2, args.prefill_steps // 10), stream)
    if not args.no_grid and args.workload == "decode_32k" and args.batch is None:
        result["prolog_overlap"] = prolog_overlap(dev)
        result["grid"] = grid(dev)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
