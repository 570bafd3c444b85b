#!/usr/bin/env python3
"""Benchmark of the chunked-prefill causal attention path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input:

  1. a 131072-token prompt split into 8 chunks of 16384 tokens (64 query
     heads over 8 KV heads, head dim 128, bf16, paged KV of 64-token blocks):
     chunk k attends to the cache of chunks 0..k (VPP technical review,
     English edition, §2.3; the per-chunk latency growth of its §3 / §4.1);
  2. one mixed batch: a 2048-token prefill chunk at offset 65536 plus 256
     single-token decode requests with contexts uniform on [1024, 32768]
     (32 / 8 heads, head dim 128), which exercises the split-KV decode
     kernel, its merge and the varlen dispatch.

``value`` is the causal-effective TFLOP/s of the whole step: the sum over
every query row of (visible keys) x 2 x (d_qk + d_v), divided by the step
time.  Inputs are resident in HBM before timing starts.  Per-chunk latency,
the split into prefill and decode parts, the prefill kernel's roofline
fraction (bf16 matrix-core peak) and the decode part's HBM fraction are
reported beside it, with the fp64 CPU oracle timed on a bounded sample of the
same workload and its outputs compared with the GPU's.  Beside the step, and
outside it, the MLA latent paths are timed on their own workloads: 256 latent
decodes and a 131072-token prompt in 8192-token chunks over the shared
576/512 latent record (GLM5.3 PP-split deployment notes §1, §4), each from a
bf16 and an fp8 latent cache.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 matrix peak: 256 CUs x 4096 flop/clk x 2.4 GHz (published 2.5 PF)
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
METRIC = "causal-effective attn TFLOP/s & per-chunk latency vs chunk index (1 MI355X)"
DOMINANT = "prefill_paged_kernel<bf16 out, d 128, d_v 128> (chunk loop launches)"
DOMINANT_NAMES = ("prefill_paged_kernel<unsigned short, 128, 128, false, false>",   # rocprofv3, demangled
                  "prefill_paged_kernelItLi128ELi128ELb0ELb0E")              # mangled
KERNEL_SOURCES = ["chunked_prefill_causal_amd/csrc/prefill_paged.hip",
                  "chunked_prefill_causal_amd/csrc/device_common.h", "chunked_prefill_causal_amd/csrc/launch.h"]
TRAFFIC_SUMMARY = "profiles/prefill_paged_gqa128k_traffic.md"
CALIB_BYTES = 1 << 30                                             # the calibration copy: reads and writes 1 GiB


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def causal_pairs(past: int, c: int) -> int:
    """Visible (query, key) pairs of one head for a chunk of c tokens at offset past."""
    return c * past + c * (c + 1) // 2


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--cpu-rows", type=int, default=6144, help="oracle rows sampled per chunk for the CPU baseline (about 10 s on 16 host cores)")
    p.add_argument("--curve-reps", type=int, default=3,
                   help="repetitions per chunk for the 32K and 512K MLA-shaped prompt curves")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--reps", type=int, default=10, help="repetitions for the decode-only / prefill-only timings")
    p.add_argument("--copy-calibration", action="store_true",
                   help="after the timed region, copy 1 GiB device to device (a known-size kernel for counter scaling)")
    p.add_argument("--alp-only", action="store_true",
                   help="time only the latency-predictor grid on the 128K prompt's cache (prints its JSON object)")
    p.add_argument("--mla-only", action="store_true",
                   help="time only the MLA latent decode batches and prompt (prints their JSON object)")
    p.add_argument("--chunk-reps", type=int, default=20, help="repetitions per chunk for the latency distribution")
    p.add_argument("--summarize-mla-profile", nargs=2, metavar="DIR",
                   help="TRACE_DIR MFMA_DIR: summarize rocprofv3 output of --mla-only for the latent prefill "
                        "kernel (no GPU needed)")
    p.add_argument("--summarize-profile", nargs="+", metavar="DIR",
                   help="TRACE_DIR FETCH_DIR WRITE_DIR [MFMA_DIR]: write the profile summary from rocprofv3 "
                        "output of this script (no GPU needed)")
    return p.parse_args()


def strip_comments(src: str) -> str:
    """C++ source without its comments, whitespace runs collapsed: what the compiler reads, so that editing
    a comment leaves the hash (and a counter summary taken on the code) valid.  The kernel sources hold no
    string literal with // or /* in it."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM-side bytes per chunk-loop launch from the committed counter summary, or None (with the reason)
    when there is no summary or the kernel sources changed since its counters were taken."""
    try:
        with open(os.path.join(ROOT, TRAFFIC_SUMMARY)) as f:
            text = f.read()
    except OSError:
        return None, "no counter summary"
    m = re.search(r"<!-- traffic (\{.*?\}) -->", text)
    if not m:
        return None, "counter summary has no traffic record"
    rec = json.loads(m.group(1))
    if rec.get("kernel_sha256") != kernel_source_hash():
        return None, "kernel sources changed since the counters were taken"
    return rec, None


def _csv_rows(directory, suffix):
    for root, _, files in os.walk(directory):
        for name in files:
            if name.endswith(suffix):
                with open(os.path.join(root, name), newline="") as f:
                    return list(csv.DictReader(f))
    raise FileNotFoundError(f"no *{suffix} under {directory}")


def _counter_per_dispatch(directory, counter, reduce=sum):
    """Per dispatch: the counter reduced over its instances, the kernel name and the grid size."""
    parts, names, grids = {}, {}, {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        parts.setdefault(d, []).append(float(r["Counter_Value"]))
        names[d] = r["Kernel_Name"]
        grids[d] = int(r["Grid_Size"])
    return {d: reduce(v) for d, v in parts.items()}, names, grids


def mixed_decode_kv_lens(inputs):
    w = inputs.WORKLOADS["mixed"]
    return inputs.context_lengths(w.decode_requests, w.decode_ctx[0], w.decode_ctx[1], w.seed + 7).tolist()


def gqa_decode_bytes(kv_lens, heads, kv_heads, d, dv):
    """Least bytes a GQA decode batch moves: K and V of every cached token once per KV head, plus q and out."""
    return sum(kv * kv_heads * (d + dv) * 2 for kv in kv_lens) + len(kv_lens) * heads * (d + dv) * 2


def mla_decode_read_bytes(inputs, bytes_per_token):
    """Bytes an MLA decode batch must read: every cached record once, the queries, the block-table entries."""
    w = inputs.WORKLOADS["mla_decode"]
    kv = inputs.context_lengths(w.decode_requests, w.decode_ctx[0], w.decode_ctx[1], w.seed)
    return (int(kv.sum()) * bytes_per_token + w.decode_requests * w.heads * w.head_dim * 2
            + sum(math.ceil(int(k) / 64) for k in kv) * 4)


def summarize_profile(trace_dir, fetch_dir, write_dir, mfma_dir=None):
    """Markdown summary of the bench command's kernel trace and its FETCH_SIZE / WRITE_SIZE passes."""
    stats = _csv_rows(trace_dir, "kernel_stats.csv")
    trace = _csv_rows(trace_dir, "kernel_trace.csv")
    lines = ["## --stats summary (kernels of the library)", "",
             "| Kernel | Calls | Average (ms) | Min (ms) | Max (ms) |", "|---|---|---|---|---|"]
    for r in stats:
        if "chunkattn" not in r["Name"]:
            continue
        short = re.sub(r"\(.*", "", r["Name"]).replace("void ", "")
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.4f} | "
                     f"{float(r['MinNs']) / 1e6:.4f} | {float(r['MaxNs']) / 1e6:.4f} |")
    durs = [(int(r["Dispatch_Id"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6) for r in trace
            if any(n in r["Kernel_Name"] for n in DOMINANT_NAMES)]
    durs = [t for _, t in sorted(durs)]
    # the trace run is the default command: 2 warmup steps, then the 5 timed steps' chunk loops (8 launches each)
    timed = durs[2 * 8: 7 * 8]
    lines += ["", f"Dominant kernel `{DOMINANT}`: {len(durs)} dispatches in the trace, average "
              f"{sum(durs) / len(durs):.4f} ms over all of them; the {len(timed)} launches of the 5 timed steps "
              f"(after the 2 warmup steps) average {sum(timed) / len(timed):.4f} ms."]
    out = {"kernel_sha256": kernel_source_hash()}
    for counter, directory in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals, names, _ = _counter_per_dispatch(directory, counter)
        # the runtime's device-to-device copy (16-byte lanes, like every kernel here); torch's elementwise
        # copy kernels count differently per byte and are not used
        calib = [d for d in vals if "copyBuffer" in names[d]]
        if not calib:
            raise SystemExit(f"{directory}: no __amd_rocclr_copyBuffer dispatch (run with --copy-calibration)")
        cal = max(calib, key=lambda d: vals[d])
        factor = CALIB_BYTES / (vals[cal] * 1024)
        # the counter passes run one warmup step and one timed step: the timed chunk loop is launches 9-16
        # (the first loop of a process runs its first chunks several times slower)
        dom = sorted(d for d in vals if any(n in names[d] for n in DOMINANT_NAMES))[8:16]
        per = [vals[d] * 1024 * factor for d in dom]
        out[counter] = {"calibration_kib": vals[cal], "factor": round(factor, 4), "dispatches": len(dom),
                        "bytes_per_launch": sum(per) / len(per), "bytes_by_chunk": [round(x) for x in per]}
        lines += ["", f"{counter}: the 1 GiB calibration copy (`{re.sub(r'[(<].*', '', names[cal])}`) counts "
                  f"{vals[cal]:.0f} KiB, so bytes = KiB x 1024 x {factor:.4f}.  Dominant kernel, by launch: "
                  + ", ".join(f"{x / 1e9:.2f} GB" for x in per) + f" (mean {sum(per) / len(per) / 1e9:.3f} GB)."]
    out["bytes_per_launch"] = out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"]
    lines += decode_fetch_check(fetch_dir, out["FETCH_SIZE"]["factor"])
    if mfma_dir:
        lines += mfma_counter_summary(mfma_dir)
    lines += ["", f"<!-- traffic {json.dumps(out)} -->"]
    return "\n".join(lines) + "\n"


def decode_fetch_check(fetch_dir, factor):
    """HBM-side reads of the decode kernels against the byte model (FETCH_SIZE, same calibration)."""
    sys.path.insert(0, ROOT)
    from chunked_prefill_causal_amd import inputs

    vals, names, grids = _counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    w = inputs.WORKLOADS["mixed"]
    checks = [("decode_kernel<128, 128>", "GQA decode, 256 requests (decode-only batch)",
               gqa_decode_bytes(mixed_decode_kv_lens(inputs), w.heads, w.kv_heads, w.head_dim, w.head_dim_v)),
              ("mla_decode_kernel<false>", "MLA decode, bf16 latent cache", mla_decode_read_bytes(inputs, 1152)),
              ("mla_decode_kernel<true>", "MLA decode, fp8 latent cache", mla_decode_read_bytes(inputs, 656))]
    lines = ["", "Decode kernels, FETCH_SIZE (same calibration) against the bytes the batch must read:", "",
             "| Kernel | Batch | Dispatches | Counted GB | Model GB | Counted / model |", "|---|---|---|---|---|---|"]
    for kname, label, model in checks:
        ds = [d for d in vals if kname in names[d]]
        if not ds:
            continue
        if kname.startswith("decode_kernel"):     # the decode-only batch: the most frequent grid
            common = max(set(grids[d] for d in ds), key=lambda g: sum(grids[d] == g for d in ds))
            ds = [d for d in ds if grids[d] == common]
        got = sum(vals[d] for d in ds) / len(ds) * 1024 * factor
        lines.append(f"| `{kname}` | {label} | {len(ds)} | {got / 1e9:.3f} | {model / 1e9:.3f} | {got / model:.3f} |")
    return lines


def mfma_counter_summary(mfma_dir):
    """Executed bf16 MFMA flops and matrix-pipe busy cycles of the chunk-loop launches (one counter pass)."""
    sys.path.insert(0, ROOT)
    from chunked_prefill_causal_amd import inputs

    mops, names, _ = _counter_per_dispatch(mfma_dir, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    busy, _, _ = _counter_per_dispatch(mfma_dir, "SQ_VALU_MFMA_BUSY_CYCLES")
    dur = {}
    for r in _csv_rows(mfma_dir, "counter_collection.csv"):
        dur[int(r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    dom = sorted(d for d in mops if any(n in names[d] for n in DOMINANT_NAMES))[8:16]
    w = inputs.WORKLOADS["gqa_128k"]
    simds, clock = 1024, 2.4e9
    lines = ["", "Chunk-loop launches, one pass of SQ_INSTS_VALU_MFMA_MOPS_BF16 and SQ_VALU_MFMA_BUSY_CYCLES. Executed "
             "flops = MOPS x 512. The busy counter is the matrix-pipe cycles summed over the 1024 SIMDs (16 per "
             "16x16x32 bf16 MFMA); busy % = busy cycles per SIMD / (launch duration under counting x 2.4 GHz), the "
             "same nominal clock as the 2516.6 TFLOP/s peak.", "",
             "| Chunk | Executed MFMA TFLOP | Causal-effective TFLOP | Executed / effective | Duration (ms) | "
             "Busy cycles per SIMD (M) | Busy % at 2.4 GHz |", "|---|---|---|---|---|---|---|"]
    for k, d in enumerate(dom):
        eff = w.heads * causal_pairs(k * w.chunk_len, w.chunk_len) * 2 * (w.head_dim + w.head_dim_v)
        ex = mops[d] * 512
        per_simd = busy.get(d, 0.0) / simds
        lines.append(f"| {k} | {ex / 1e12:.2f} | {eff / 1e12:.2f} | {ex / eff:.3f} | {dur[d] * 1e3:.3f} | "
                     f"{per_simd / 1e6:.2f} | {100 * per_simd / (dur[d] * clock):.1f} |")
    return lines


def summarize_mla_prefill_profile(trace_dir, mfma_dir):
    """Markdown summary of `--mla-only` under a kernel trace and under one matrix-counter pass: the latent
    prefill kernel per cache format and chunk.  Each format runs every chunk once warm, then `reps` times
    timed (bf16 first, then fp8), so a format's launches are its first 16 plus 16 x reps."""
    sys.path.insert(0, ROOT)
    from chunked_prefill_causal_amd import inputs

    w = inputs.WORKLOADS["mla_prefill"]
    n = w.n_chunks
    eff = [w.heads * causal_pairs(k * w.chunk_len, w.chunk_len) * 2 * (w.head_dim + w.head_dim_v)
           for k in range(n)]

    def split(ds):
        ds = sorted(ds)
        half = len(ds) // 2
        return {"bf16": ds[n:half], "fp8": ds[half + n:]}     # the timed launches of each format

    trace = {int(r["Dispatch_Id"]): (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6
             for r in _csv_rows(trace_dir, "kernel_trace.csv") if "mla_prefill_kernel" in r["Kernel_Name"]}
    deq = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6
           for r in _csv_rows(trace_dir, "kernel_trace.csv") if "mla_dequant_kernel" in r["Kernel_Name"]]
    mops, _, _ = _counter_per_dispatch(mfma_dir, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    busy, names, _ = _counter_per_dispatch(mfma_dir, "SQ_VALU_MFMA_BUSY_CYCLES")
    dur = {int(r["Dispatch_Id"]): (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
           for r in _csv_rows(mfma_dir, "counter_collection.csv")}
    mla = split(d for d in mops if "mla_prefill_kernel" in names[d])
    tr = split(trace)
    lines = ["## Kernel trace", "",
             f"`mla_prefill_kernel` launches in the trace: {len(trace)}; the widening pass `mla_dequant_kernel` "
             f"(fp8 cache): {len(deq)} launches, average {sum(deq) / max(1, len(deq)):.4f} ms.", "",
             "| Cache | Timed launches | Chunk-loop sum of per-chunk means (ms) | Average launch (ms) | "
             "Causal-effective TFLOP/s | of 2516.6 |", "|---|---|---|---|---|---|"]
    for fmt, ds in tr.items():
        per = [sum(trace[d] for d in ds[k::n]) / len(ds[k::n]) for k in range(n)]
        tf = sum(eff) / (sum(per) / 1e3) / 1e12
        lines.append(f"| {fmt} | {len(ds)} | {sum(per):.3f} | {sum(per) / n:.4f} | {tf:.1f} | "
                     f"{100 * tf / PEAK_BF16_TFLOPS:.1f} % |")
    lines += ["", "## Matrix-core counters (SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES)", "",
              "Timed launch of each chunk.  Executed flops = MOPS x 512; busy % = matrix-pipe busy cycles per "
              "SIMD (1024 SIMDs) / (launch duration under counting x 2.4 GHz).", "",
              "| Chunk | Executed TFLOP | Causal-effective TFLOP | Executed / effective | bf16 cache: ms, busy % | "
              "fp8 cache: ms, busy % |", "|---|---|---|---|---|---|"]
    for k in range(n):
        cells = []
        for fmt in ("bf16", "fp8"):
            d = mla[fmt][k]
            cells.append(f"{dur[d] * 1e3:.3f}, {100 * busy[d] / 1024 / (dur[d] * 2.4e9):.1f}")
        ex = mops[mla["bf16"][k]] * 512
        lines.append(f"| {k} | {ex / 1e12:.3f} | {eff[k] / 1e12:.3f} | {ex / eff[k]:.3f} | {cells[0]} | {cells[1]} |")
    return "\n".join(lines) + "\n"


class PrefillLoop:
    """A chunked prompt: paged pool, block table, every chunk's queries, one output buffer."""

    def __init__(self, L, inputs, torch, name="gqa_128k", keep_logical=True):
        w = inputs.WORKLOADS[name]
        self.w = w
        n, hkv, d, dv = w.seq_len, w.kv_heads, w.head_dim, w.head_dim_v
        needed = math.ceil(n / 64)
        self.table = torch.from_numpy(inputs.block_table(needed, w.seed + 3)).cuda()
        self.k, self.v = L.paged_pool(inputs.pool_size(needed), hkv, d, dv, torch.bfloat16)
        self.k.fill_(float("nan"))
        self.v.fill_(float("nan"))
        kk = inputs.normal_device((n, hkv, d), w.seed + 1, "bf16")
        vv = inputs.normal_device((n, hkv, dv), w.seed + 2, "bf16")
        L.chunkattn_kv_append(kk, vv, 0, self.table, self.k, self.v)
        if keep_logical:
            self.k_logical, self.v_logical = kk, vv    # kept for the oracle sample
        del kk, vv
        self.q = [inputs.normal_device((w.chunk_len, w.heads, d), inputs.chunk_seeds(w, c), "bf16")
                  for c in range(w.n_chunks)]
        self.out = torch.empty((w.chunk_len, w.heads, dv), dtype=torch.bfloat16, device="cuda")
        self.flops = [w.heads * causal_pairs(c * w.chunk_len, w.chunk_len) * 2 * (d + dv)
                      for c in range(w.n_chunks)]

    def run_chunk(self, L, c, out=None):
        w = self.w
        return L.chunk_prefill_attn(self.q[c], self.k, self.v, c * w.chunk_len, w.scale, kv_layout="paged",
                                    block_table=self.table, out=self.out if out is None else out, num_splits=0)


class MixedBatch:
    """One prefill chunk + 256 decode requests in one shared paged pool."""

    def __init__(self, L, inputs, torch, decode_only=False, prefill_only=False, parent=None):
        w = inputs.WORKLOADS["mixed"]
        self.w = w
        hq, hkv, d, dv = w.heads, w.kv_heads, w.head_dim, w.head_dim_v
        if parent is None:
            dec = inputs.context_lengths(w.decode_requests, w.decode_ctx[0], w.decode_ctx[1], w.seed + 7)
            q_lens = [w.chunk_len] + [1] * w.decode_requests
            kv_lens = [w.prefill_past + w.chunk_len] + dec.tolist()
            needed = [math.ceil(x / 64) for x in kv_lens]
            pool_blocks = inputs.pool_size(sum(needed))
            perm = inputs.block_table(sum(needed), w.seed + 8, pool_blocks)
            max_blocks = max(needed)
            tables = torch.zeros((len(kv_lens), max_blocks), dtype=torch.int32)
            off = 0
            for s, nb in enumerate(needed):
                tables[s, :nb] = torch.from_numpy(perm[off: off + nb])
                off += nb
            self.tables = tables.cuda()
            self.k, self.v = L.paged_pool(pool_blocks, hkv, d, dv, torch.bfloat16)
            self.k.fill_(float("nan"))
            self.v.fill_(float("nan"))
            for s, n in enumerate(kv_lens):
                kk = inputs.normal_device((n, hkv, d), w.seed + 100 + 2 * s, "bf16")
                vv = inputs.normal_device((n, hkv, dv), w.seed + 101 + 2 * s, "bf16")
                L.chunkattn_kv_append(kk, vv, 0, self.tables[s], self.k, self.v)
            self.q_all = inputs.normal_device((sum(q_lens), hq, d), w.seed + 9, "bf16")
            self.q_lens, self.kv_lens = q_lens, kv_lens
        else:
            self.k, self.v = parent.k, parent.v
            sel = list(range(1, len(parent.kv_lens))) if decode_only else [0]
            self.tables = parent.tables[sel].contiguous()
            self.q_lens = [parent.q_lens[s] for s in sel]
            self.kv_lens = [parent.kv_lens[s] for s in sel]
            first = parent.q_lens[0]
            self.q_all = (parent.q_all[first:] if decode_only else parent.q_all[:first]).contiguous()
        cu = [0]
        for x in self.q_lens:
            cu.append(cu[-1] + x)
        self.cu = cu
        self.cu_dev = torch.tensor(cu, dtype=torch.int32, device="cuda")
        self.kv_dev = torch.tensor(self.kv_lens, dtype=torch.int32, device="cuda")
        need = L.chunkattn_varlen_workspace_size(cu, self.kv_lens, hq, hkv, dv)
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        self.out = torch.empty((cu[-1], hq, dv), dtype=torch.bfloat16, device="cuda")
        pref = [(kv - ql, ql) for ql, kv in zip(self.q_lens, self.kv_lens) if ql * (hq // hkv) > 32]
        decs = [kv for ql, kv in zip(self.q_lens, self.kv_lens) if 0 < ql * (hq // hkv) <= 32]
        self.prefill_flops = sum(hq * causal_pairs(p, c) * 2 * (d + dv) for p, c in pref)
        self.decode_flops = sum(hq * kv * 2 * (d + dv) for kv in decs)
        # bytes the decode part must move: K and V of every cached token once per KV head, plus q and out
        self.decode_bytes = gqa_decode_bytes(decs, hq, hkv, d, dv)
        self.flops = self.prefill_flops + self.decode_flops

    def run(self, L):
        return L.chunk_attn_varlen(self.q_all, self.k, self.v, self.tables, self.cu, self.kv_lens, self.w.scale,
                                   out=self.out, workspace=self.ws, cu_seqlens_q_dev=self.cu_dev,
                                   kv_lens_dev=self.kv_dev)


class MlaDecode:
    """256 absorbed MLA decodes over a paged latent cache of one format (bf16 or fp8).

    Records are written by the library's cache-write kernel (fp8: quantised
    there); the pool is poisoned with 0xFF first.  ``bytes`` is what the
    decode must move at least: every cached record once (1152 B bf16, 656 B
    fp8 per token), the queries and outputs, and the block-table entries.
    """

    def __init__(self, L, inputs, torch, fmt):
        w = inputs.WORKLOADS["mla_decode"]
        self.w, self.fmt = w, fmt
        kv = inputs.context_lengths(w.decode_requests, w.decode_ctx[0], w.decode_ctx[1], w.seed)
        tables, pool_blocks = inputs.batch_block_tables(kv, w.seed + 1)
        self.tables = torch.from_numpy(tables).cuda()
        self.pool = L.mla_pool(pool_blocks, fmt)
        self.pool.fill_(0xFF)
        gen = torch.Generator(device="cuda")
        for s, n in enumerate(kv.tolist()):
            gen.manual_seed(inputs.mla_record_seed(w, s))
            lat = torch.randn((n, L.MLA_LATENT), generator=gen, device="cuda").to(torch.bfloat16)
            rope = torch.randn((n, L.MLA_ROPE), generator=gen, device="cuda").to(torch.bfloat16)
            L.chunkattn_mla_kv_append(lat, rope, 0, self.tables[s], self.pool, fmt)
        self.q = inputs.normal_device((w.decode_requests, w.heads, w.head_dim), w.seed + 2, "bf16")
        self.kv_host = torch.from_numpy(kv)
        self.kv_dev = self.kv_host.cuda()
        self.out = torch.empty((w.decode_requests, w.heads, w.head_dim_v), dtype=torch.bfloat16, device="cuda")
        need = L.chunkattn_mla_decode_workspace_size(kv, w.heads, fmt)
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        self.tokens = int(kv.sum())
        self.bytes_per_token = L.chunkattn_mla_block_bytes(fmt) // 64
        self.bytes = (self.tokens * self.bytes_per_token + (self.q.numel() + self.out.numel()) * 2
                      + sum(math.ceil(int(k) / 64) for k in kv) * 4)

    def run(self, L):
        return L.chunk_mla_decode(self.q, self.pool, self.fmt, self.tables, self.kv_host, self.w.scale,
                                  out=self.out, workspace=self.ws, kv_lens_dev=self.kv_dev)


class MlaPrefill:
    """The 128K-token latent prompt (16 chunks of 8192, 16 heads) over a paged latent cache of one format.

    The whole prompt's records are written first (0xFF-poisoned pool, fp8 quantised by the write kernel);
    chunk k then attends to records 0 .. its positions, as after appending it.  Matrix work per chunk:
    2 * (576 + 512) flops per visible (query, key) pair and head; the fp8 path includes its widening pass.
    """

    def __init__(self, L, inputs, torch, fmt):
        w = inputs.WORKLOADS["mla_prefill"]
        self.w, self.fmt = w, fmt
        needed = math.ceil(w.seq_len / 64)
        self.table = torch.from_numpy(inputs.block_table(needed, w.seed + 3)).cuda()
        self.pool = L.mla_pool(inputs.pool_size(needed), fmt)
        self.pool.fill_(0xFF)
        gen = torch.Generator(device="cuda")
        gen.manual_seed(inputs.mla_record_seed(w, 0))
        lat = torch.randn((w.seq_len, L.MLA_LATENT), generator=gen, device="cuda").to(torch.bfloat16)
        rope = torch.randn((w.seq_len, L.MLA_ROPE), generator=gen, device="cuda").to(torch.bfloat16)
        L.chunkattn_mla_kv_append(lat, rope, 0, self.table, self.pool, fmt)
        del lat, rope
        self.q = [inputs.normal_device((w.chunk_len, w.heads, w.head_dim), inputs.chunk_seeds(w, k), "bf16")
                  for k in range(w.n_chunks)]
        self.out = torch.empty((w.chunk_len, w.heads, w.head_dim_v), dtype=torch.bfloat16, device="cuda")
        need = L.chunkattn_mla_prefill_workspace_size(0, w.seq_len, fmt)
        self.ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
        self.flops = [w.heads * 2 * (w.head_dim + w.head_dim_v) * causal_pairs(k * w.chunk_len, w.chunk_len)
                      for k in range(w.n_chunks)]

    def run_chunk(self, L, k):
        return L.chunk_mla_prefill(self.q[k], self.pool, self.fmt, self.table, k * self.w.chunk_len, self.w.scale,
                                   out=self.out, workspace=self.ws)


def mla_prefill_summary(L, inputs, torch, reps):
    """Both latent formats of the 128K MLA prompt: per-chunk latency (median of `reps`), the chunk loop's
    matrix TFLOP/s against the dense bf16 peak."""
    res = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for name, fmt in (("bf16", L.CA_MLA_BF16), ("fp8", L.CA_MLA_FP8)):
        m = MlaPrefill(L, inputs, torch, fmt)
        for k in range(m.w.n_chunks):
            m.run_chunk(L, k)
        per = []
        for k in range(m.w.n_chunks):
            ts = []
            for _ in range(reps):
                e0.record()
                m.run_chunk(L, k)
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            per.append(median(ts))
        a, b, r2 = fit_line(list(range(m.w.n_chunks)), per)
        tflops = sum(m.flops) / (sum(per) / 1e3) / 1e12
        res[name] = {"loop_ms": round(sum(per), 3), "per_chunk_ms": [round(x, 4) for x in per],
                     "fit": {"a_ms": round(a, 4), "b_ms_per_chunk": round(b, 4), "r2": round(r2, 5)},
                     "tokens_per_s": round(m.w.seq_len / (sum(per) / 1e3), 1),
                     "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                                  "avg_launch_ms": round(sum(per) / m.w.n_chunks, 4),
                                  "avg_flops_per_launch": sum(m.flops) / m.w.n_chunks}}
        log(f"MLA prefill {name}: loop {sum(per):.2f} ms, {tflops:.1f} TFLOP/s "
            f"({tflops / PEAK_BF16_TFLOPS:.1%} of dense bf16 peak)")
        del m
        torch.cuda.empty_cache()
    w = inputs.WORKLOADS["mla_prefill"]
    res["workload"] = (f"{w.seq_len}-token prompt as {w.n_chunks} chunks of {w.chunk_len}, {w.heads} q heads over "
                       "one shared 512+64 latent record per token (d_qk 576, d_v 512), paged KV (64); fp8 includes "
                       "its widening pass; inputs resident in HBM")
    return res


def mla_decode_summary(L, inputs, torch, timed, reps, warmup):
    """Both latent formats of the MLA decode batch: op time, HBM fraction, requests/s."""
    res = {}
    for name, fmt in (("bf16", L.CA_MLA_BF16), ("fp8", L.CA_MLA_FP8)):
        m = MlaDecode(L, inputs, torch, fmt)
        for _ in range(max(1, warmup)):
            m.run(L)
        torch.cuda.synchronize()
        ms = timed(lambda: m.run(L), reps)
        gbps = m.bytes / (ms / 1e3) / 1e9
        res[name] = {"ms": round(ms, 4), "requests_per_s": round(m.w.decode_requests / (ms / 1e3), 1),
                     "cached_tokens": m.tokens, "bytes_per_token": m.bytes_per_token,
                     "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                                  "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4),
                                  "algorithmic_bytes": m.bytes}}
        log(f"MLA decode {name}: {ms:.3f} ms, {gbps:.0f} GB/s ({gbps / PEAK_HBM_GBPS:.1%} of HBM)")
        del m
        torch.cuda.empty_cache()
    res["fp8_speedup"] = round(res["bf16"]["ms"] / res["fp8"]["ms"], 3)
    res["workload"] = ("256 decodes, ctx U[1024,32768], 16 q heads over one shared 576-value latent record per "
                       "token, paged KV (64); decode + split merge, inputs resident in HBM")
    return res


def contiguous_cache_summary(L, loop, torch, timed, reps):
    """Chunks 3 and 7 read from a bf16 contiguous [tokens, kv_heads, d] cache holding the same logical K/V
    as the paged pool.  With workspace room the library re-lays the prefix for the paged kernel; that copy
    is inside the timed call.  With no workspace it reads the cache in place (the 8-wave kernel on
    token-major tiles).  The paged pool's time for the same chunk is measured beside both."""
    w = loop.w
    last = w.n_chunks - 1
    ws = torch.empty(L.chunkattn_prefill_contiguous_workspace_size(last * w.chunk_len, w.chunk_len, w.heads,
                                                                   w.kv_heads, w.head_dim, w.head_dim_v, 0),
                     dtype=torch.uint8, device="cuda")
    res = {"chunks": [], "ms": [], "tflops": [], "in_place_ms": [], "in_place_tflops": [], "paged_ms": []}
    for c in (3, last):
        past = c * w.chunk_len
        kc, vc = loop.k_logical[: past + w.chunk_len], loop.v_logical[: past + w.chunk_len]
        f = lambda: L.chunk_prefill_attn(loop.q[c], kc, vc, past, w.scale, out=loop.out, workspace=ws)
        f()
        torch.cuda.synchronize()
        t = timed(f, reps)
        g = lambda: L.chunk_prefill_attn(loop.q[c], kc, vc, past, w.scale, out=loop.out, relayout=False)
        g()
        torch.cuda.synchronize()
        ti = timed(g, reps)
        tp = timed(lambda: loop.run_chunk(L, c), reps)
        res["chunks"].append(c)
        res["ms"].append(round(t, 3))
        res["tflops"].append(round(loop.flops[c] / (t / 1e3) / 1e12, 1))
        res["in_place_ms"].append(round(ti, 3))
        res["in_place_tflops"].append(round(loop.flops[c] / (ti / 1e3) / 1e12, 1))
        res["paged_ms"].append(round(tp, 3))
    res["note"] = ("ms: bf16 contiguous cache re-laid into the workspace (identity block table) and read by the "
                   "paged kernel, the copy timed; in_place_ms: no workspace, the 8-wave kernel reads the cache in "
                   "place (token-major tiles, V transposed once per workgroup in LDS)")
    return res


def chunk_latency_stats(L, loop, torch, reps):
    """Each chunk `reps` times (median, p10, p90); then each once cold, after a 512 MiB write evicts the
    caches."""
    n = loop.w.n_chunks
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    warm = []
    for c in range(n):
        ts = []
        for _ in range(reps):
            e0.record()
            loop.run_chunk(L, c)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ts.sort()
        at = lambda q: ts[min(len(ts) - 1, int(round(q * (len(ts) - 1))))]
        warm.append((median(ts), at(0.1), at(0.9)))
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = []
    for c in range(n):
        flush.fill_(c & 0xFF)
        torch.cuda.synchronize()
        e0.record()
        loop.run_chunk(L, c)
        e1.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    del flush
    return {"reps": reps, "median_ms": [round(x[0], 3) for x in warm], "p10_ms": [round(x[1], 3) for x in warm],
            "p90_ms": [round(x[2], 3) for x in warm], "cold_ms": [round(x, 3) for x in cold],
            "cold_note": "one call per chunk right after writing a 512 MiB buffer (L2 and MALL evicted)"}


def prompt_curve(L, inputs, torch, name, reps):
    """Per-chunk latency of a whole prompt (every chunk `reps` times, median), its linear fit and the
    chunk loop's causal-effective TFLOP/s against the dense bf16 peak."""
    loop = PrefillLoop(L, inputs, torch, name, keep_logical=False)
    w = loop.w
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for c in range(w.n_chunks):
        loop.run_chunk(L, c)
    per = []
    for c in range(w.n_chunks):
        ts = []
        for _ in range(reps):
            e0.record()
            loop.run_chunk(L, c)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        per.append(median(ts))
    a, b, r2 = fit_line(list(range(w.n_chunks)), per)
    tflops = sum(loop.flops) / (sum(per) / 1e3) / 1e12
    out = {"workload": f"{w.seq_len}-token prompt as {w.n_chunks} chunks of {w.chunk_len}, {w.heads} q / "
                       f"{w.kv_heads} KV heads, d {w.head_dim}/{w.head_dim_v}, bf16, paged KV block 64",
           "reps": reps, "per_chunk_ms": [round(x, 4) for x in per],
           "per_chunk_tflops": [round(f / (t / 1e3) / 1e12, 1) for f, t in zip(loop.flops, per)],
           "fit": {"a_ms": round(a, 4), "b_ms_per_chunk": round(b, 4), "r2": round(r2, 5),
                   "b_over_a": round(b / a, 3) if a else None},
           "loop_ms": round(sum(per), 3), "tflops": round(tflops, 1),
           "frac": round(tflops / PEAK_BF16_TFLOPS, 4)}
    del loop
    torch.cuda.empty_cache()
    return out


def copy_bandwidth(torch, nbytes=1 << 30, reps=5):
    """A plain device copy and a plain reduction over 1 GiB (torch kernels): what the memory system gives
    these access patterns, as a sanity figure beside the decode rooflines."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def t(fn):
        fn()
        ts = []
        for _ in range(reps):
            torch.cuda.synchronize()
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return median(ts)

    copy_ms = t(lambda: dst.copy_(src))
    read_ms = t(lambda: src.sum())
    del src, dst
    return {"bytes": nbytes, "copy_gbps": round(2 * nbytes / (copy_ms / 1e3) / 1e9, 1),
            "read_gbps": round(nbytes / (read_ms / 1e3) / 1e9, 1),
            "note": "copy counts bytes read + written; read is a sum over the buffer; peak 8000 GB/s"}


class GpuMonitor:
    """Samples the GPU's shader (GFX) clock and socket power with amdsmi, read-only, from a thread while
    a region runs; every figure is None where the interface is not available."""

    def __init__(self, period_s=0.025):
        import threading
        self.period, self.samples, self._stop = period_s, [], threading.Event()
        self.handle, self.cap_w = None, None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self.amdsmi = amdsmi
            self.handle = amdsmi.amdsmi_get_processor_handles()[0]
            cap = amdsmi.amdsmi_get_power_cap_info(self.handle)
            self.cap_w = cap.get("power_cap", None)
            if self.cap_w is not None and self.cap_w > 10000:
                self.cap_w = self.cap_w / 1e6            # reported in microwatts on some versions
        except Exception:
            self.handle = None
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        clk = self.amdsmi.amdsmi_get_clock_info(self.handle, self.amdsmi.AmdSmiClkType.GFX)
        pwr = self.amdsmi.amdsmi_get_power_info(self.handle)
        mhz = clk.get("clk", clk.get("cur_clk"))
        watts = pwr.get("current_socket_power", "N/A")
        if not isinstance(watts, (int, float)):
            watts = pwr.get("average_socket_power", None)
        return mhz, watts if isinstance(watts, (int, float)) else None

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._read())
            except Exception:
                return
            self._stop.wait(self.period)

    def __enter__(self):
        if self.handle is not None:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.handle is not None:
            self._thread.join()

    def summary(self):
        clk = [c for c, _ in self.samples if isinstance(c, (int, float))]
        pw = [p for _, p in self.samples if isinstance(p, (int, float))]
        if not clk:
            return {"gfx_clock_mhz": None, "note": "amdsmi not available"}
        return {"samples": len(self.samples), "gfx_clock_mhz_median": median(clk), "gfx_clock_mhz_min": min(clk),
                "gfx_clock_mhz_max": max(clk), "socket_power_w_median": median(pw) if pw else None,
                "power_cap_w": self.cap_w,
                "note": "amdsmi GFX clock and socket power sampled every 25 ms during the timed steps"}


def median(xs):
    s = sorted(xs)
    return s[len(s) // 2] if len(s) % 2 else 0.5 * (s[len(s) // 2 - 1] + s[len(s) // 2])


def fit_line(ks, ts):
    n = len(ks)
    mk, mt = sum(ks) / n, sum(ts) / n
    sxx = sum((k - mk) ** 2 for k in ks)
    b = sum((k - mk) * (t - mt) for k, t in zip(ks, ts)) / sxx
    a = mt - b * mk
    ss_res = sum((t - (a + b * k)) ** 2 for k, t in zip(ks, ts))
    ss_tot = sum((t - mt) ** 2 for t in ts)
    return a, b, 1 - ss_res / ss_tot if ss_tot else 1.0


def schedule_summary(L, tau):
    """Two-rank CPP / VPP / VPP-Async schedules (VPP review §4.2-§4.5) driven by the measured per-chunk
    latencies: one request, and two back-to-back requests with and without Alg. 2 packing."""
    out = {"tau_ms": [round(x, 4) for x in tau], "comm_ms": 0.0}
    names = {L.CA_SCHED_CPP: "cpp", L.CA_SCHED_VPP: "vpp", L.CA_SCHED_VPP_ASYNC: "vpp_async"}
    for kind, name in names.items():
        one = L.chunkattn_sched_simulate(kind, tau)
        two = {p: L.chunkattn_sched_simulate(kind, list(tau) * 2, request=[0] * len(tau) + [1] * len(tau), pack=p)
               for p in (False, True)}
        bubble = lambda r: 1.0 - float(r["busy"].sum()) / (2 * r["makespan"])
        out[name] = {"makespan_ms": round(one["makespan"], 3), "bubble_frac": round(bubble(one), 4),
                     "two_requests_ms": round(two[False]["makespan"], 3),
                     "two_requests_packed_ms": round(two[True]["makespan"], 3)}
    return out


def latency_predictor(L, loop, torch, reps=3):
    """ALP-style attention-latency predictor (FastPP notes §2.3) fitted to this kernel's own timings.

    Batches on the 128K prompt's cache (64 q / 8 KV heads, d 128): single prefill chunks over a grid of
    (past, chunk) sizes, decode-only batches and mixed batches, all through the varlen entry.  A seeded
    half trains the library's recursive least-squares fit, the other half is held out; the token-count-only
    model (constant + total new tokens) is fitted the same way for comparison."""
    import numpy as np

    w = loop.w
    rng = np.random.default_rng(w.seed + 17)
    cases = []
    for c in (512, 1024, 2048, 4096, 8192, 16384):
        for past in (0, 8192, 24576, 49152, 81920, 114688):
            if past + c <= w.seq_len:
                cases.append(([c], [past + c]))
    for m in (16, 64, 128, 256):
        cases.append(([1] * m, rng.integers(1024, w.seq_len + 1, m).tolist()))
        for c in (1024, 4096):
            past = int(rng.integers(0, w.seq_len - c + 1))
            cases.append(([c] + [1] * m, [past + c] + rng.integers(1024, w.seq_len + 1, m).tolist()))
    max_q = max(sum(q) for q, _ in cases)
    max_s = max(len(q) for q, _ in cases)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 18)
    q_buf = torch.randn((max_q, w.heads, w.head_dim), generator=gen, device="cuda").to(torch.bfloat16)
    out_buf = torch.empty((max_q, w.heads, w.head_dim_v), dtype=torch.bfloat16, device="cuda")
    tables = loop.table.unsqueeze(0).expand(max_s, -1).contiguous()
    times = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for q_lens, kv_lens in cases:
        n, tq = len(q_lens), sum(q_lens)
        cu = [0]
        for x in q_lens:
            cu.append(cu[-1] + x)
        ws = torch.empty(max(L.chunkattn_varlen_workspace_size(cu, kv_lens, w.heads, w.kv_heads, w.head_dim_v), 1),
                         dtype=torch.uint8, device="cuda")
        cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda")
        kv_d = torch.tensor(kv_lens, dtype=torch.int32, device="cuda")
        run = lambda: L.chunk_attn_varlen(q_buf[:tq], loop.k, loop.v, tables[:n], cu, kv_lens, w.scale,
                                          out=out_buf[:tq], workspace=ws, cu_seqlens_q_dev=cu_d, kv_lens_dev=kv_d)
        run()
        ts = []
        for _ in range(reps):
            e0.record()
            run()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        times.append(median(ts))
    order = rng.permutation(len(cases))
    train, test = order[: len(cases) // 2], order[len(cases) // 2:]
    fits = {}
    # The times span three orders of magnitude and the score is relative, so each observation is
    # weighted by 1/T^2: the fit sees x / T with target 1 (relative least squares).
    H, G = w.heads, w.kv_heads
    for name, feat in (("token_count_only", lambda q, kv: [1.0, sum(q) / 1e3, 0.0, 0.0, 0.0]),
                       ("alp_features", lambda q, kv: list(L.chunkattn_alp_features(q, kv, H, G)[:4]) + [0.0]),
                       ("alp_plus_fill", lambda q, kv: list(L.chunkattn_alp_features(q, kv, H, G)))):
        model = L.AlpPredictor(1.0, 1e6)
        for i in train:
            model.update([v / times[i] for v in feat(*cases[i])], 1.0)
        err = [abs(model.predict(feat(*cases[i])) - times[i]) / times[i] for i in test]
        fits[name] = {"mape_holdout": round(float(np.mean(err)), 4), "max_ape": round(float(np.max(err)), 4),
                      "theta": [round(t, 6) for t in model.theta]}
    samples = [[sum(q), len(q)] + [round(v, 6) for v in L.chunkattn_alp_features(q, kv, H, G)[1:]] + [round(t, 5)]
               for (q, kv), t in zip(cases, times)]
    return {"cases": len(cases), "train": len(train), "holdout": len(test), "unit": "ms",
            "features": "[1, sum(L_past*L_pre)/1e6, sum(L_pre^2)/1e6, sum(L_dec)/1e3, fill]; alp_features fits the "
                        "first four (the pages' model), alp_plus_fill all five (fill: idle fraction of the prefill "
                        "launch's last round x its causal pairs / 1e6)",
            "fit": "recursive least squares on x/T -> 1 (relative error), lambda 1, delta 1e6", **fits,
            "samples": {"columns": ["new_tokens", "sequences", "past_x_pre_M", "pre_sq_M", "dec_ctx_K", "fill_M", "ms"],
                        "rows": samples}}


def cpu_baseline(args, loop, torch):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload (host cores)."""
    import numpy as np

    import oracle
    from chunked_prefill_causal_amd import _lib as L
    from chunked_prefill_causal_amd import inputs

    w = loop.w
    cores = len(os.sched_getaffinity(0))
    k_host = inputs.to_oracle(loop.k_logical)
    v_host = inputs.to_oracle(loop.v_logical)
    total_flops, total_s, worst, rows = 0, 0.0, 0.0, 0
    for c in range(w.n_chunks):
        tok, head = inputs.sample_rows(w.chunk_len, w.heads, args.cpu_rows, w.seed * 7 + c)
        q_host = inputs.to_oracle(loop.q[c])
        past = c * w.chunk_len
        kv_len = past + w.chunk_len
        t0 = time.perf_counter()
        ref, _ = oracle.attend_rows(q_host, k_host[:kv_len], v_host[:kv_len], past, w.scale, tok, head,
                                    threads=cores)
        total_s += time.perf_counter() - t0
        total_flops += int(sum(past + t + 1 for t in tok.tolist())) * 2 * (w.head_dim + w.head_dim_v)
        out = loop.run_chunk(L, c, out=torch.empty_like(loop.out))
        got = out[torch.from_numpy(tok).cuda(), torch.from_numpy(head.astype(np.int64)).cuda()]
        worst = max(worst, float(np.max(np.abs(got.float().cpu().numpy() - ref))))
        rows += len(tok)
        log(f"oracle chunk {c}: {len(tok)} rows, running max |gpu - oracle| = {worst:.3e}")
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    rate = total_flops / total_s
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "rows": rows, "seconds": round(total_s, 2), "rows_per_s": round(rows / total_s, 1),
            "fp64_gflops": round(rate / 1e9, 2),
            "extrapolated_full_chunk_loop_s": round(sum(loop.flops) / rate, 1),
            "sample": f"{args.cpu_rows} seeded (token, head) rows per chunk of the 131072-token prompt, all 8 "
                      f"chunks ({rows} rows, {total_flops:.3e} causal-effective flops in fp64, "
                      f"{total_s:.1f} s); CPU {cpu_model}",
            "parity_max_abs_err_on_sample": worst}


def main():
    args = parse()
    if args.summarize_mla_profile:
        sys.stdout.write(summarize_mla_prefill_profile(*args.summarize_mla_profile))
        return
    if args.summarize_profile:
        if len(args.summarize_profile) not in (3, 4):
            sys.exit("--summarize-profile takes TRACE_DIR FETCH_DIR WRITE_DIR [MFMA_DIR]")
        sys.stdout.write(summarize_profile(*args.summarize_profile))
        return
    if args.gpus != 1:
        print(f"bench.py measures a single GPU; --gpus {args.gpus} is not supported: the attention path here "
              "runs on one MI355X and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    import torch

    from chunked_prefill_causal_amd import _lib as L
    from chunked_prefill_causal_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    L.lib()
    torch.cuda.set_device(0)

    def timed(fn, reps):
        """GPU time of one call, median of `reps`.  Each timed call is enqueued right behind an untimed call of
        the same work, so the host's argument checks and launches for it overlap the GPU's run of the one
        before (as in a serving loop that runs ahead of the GPU) instead of showing as idle GPU time."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for _ in range(reps):
            fn()
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return median(ts)

    if args.mla_only:
        print(json.dumps({"mla_decode": mla_decode_summary(L, inputs, torch, timed, args.reps, args.warmup),
                          "mla_prefill": mla_prefill_summary(L, inputs, torch, args.curve_reps)}), flush=True)
        return
    log("generating inputs in HBM")
    loop = PrefillLoop(L, inputs, torch)
    if args.alp_only:
        print(json.dumps({"latency_predictor": latency_predictor(L, loop, torch)}), flush=True)
        return
    mixed = MixedBatch(L, inputs, torch)
    dec_only = MixedBatch(L, inputs, torch, decode_only=True, parent=mixed)
    pre_only = MixedBatch(L, inputs, torch, prefill_only=True, parent=mixed)
    torch.cuda.synchronize()
    n_chunks = loop.w.n_chunks
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_chunks + 1)]

    def step(record):
        for c in range(n_chunks):
            if record:
                ev[c][0].record()
            loop.run_chunk(L, c)
            if record:
                ev[c][1].record()
        if record:
            ev[n_chunks][0].record()
        mixed.run(L)
        if record:
            ev[n_chunks][1].record()

    log(f"warmup {args.warmup} step(s)")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"timing {args.steps} step(s)")
    chunk_ms = [[] for _ in range(n_chunks)]
    mixed_ms = []
    monitor = GpuMonitor()
    torch.cuda.synchronize()
    with monitor:
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(True)
            torch.cuda.synchronize()
            for c in range(n_chunks):
                chunk_ms[c].append(ev[c][0].elapsed_time(ev[c][1]))
            mixed_ms.append(ev[n_chunks][0].elapsed_time(ev[n_chunks][1]))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    step_flops = sum(loop.flops) + mixed.flops
    value = step_flops / (ms_per_step / 1e3) / 1e12

    per_chunk = [median(x) for x in chunk_ms]
    a, b, r2 = fit_line(list(range(n_chunks)), per_chunk)
    prefill_tflops = sum(loop.flops) / (sum(per_chunk) / 1e3) / 1e12
    log(f"step {ms_per_step:.2f} ms, {value:.1f} TFLOP/s; chunk loop {sum(per_chunk):.2f} ms "
        f"({prefill_tflops:.1f} TFLOP/s); mixed {median(mixed_ms):.3f} ms")
    log(f"per-chunk latency distribution ({args.chunk_reps} repetitions each) and a cold pass")
    chunk_stats = chunk_latency_stats(L, loop, torch, args.chunk_reps)

    # the two halves of the mixed batch on their own (for the decode HBM roofline)
    dec_ms = timed(lambda: dec_only.run(L), args.reps)
    pre_ms = timed(lambda: pre_only.run(L), args.reps)
    dec_gbps = dec_only.decode_bytes / (dec_ms / 1e3) / 1e9
    log(f"decode-only {dec_ms:.3f} ms = {dec_gbps:.0f} GB/s; mixed prefill-only {pre_ms:.3f} ms")
    contig = contiguous_cache_summary(L, loop, torch, timed, args.reps)
    log(f"contiguous cache, chunks {contig['chunks']}: re-laid {contig['ms']} ms ({contig['tflops']} TFLOP/s), "
        f"in place {contig['in_place_ms']} ms ({contig['in_place_tflops']} TFLOP/s); paged pool {contig['paged_ms']} ms")
    log("copy-bandwidth sanity figure")
    bw = copy_bandwidth(torch)
    log(f"1 GiB copy {bw['copy_gbps']} GB/s, read {bw['read_gbps']} GB/s")
    curves = {}
    for name in ("gqa_32k", "mla_512k"):
        log(f"per-chunk latency curve of {name}")
        curves[name] = prompt_curve(L, inputs, torch, name, args.curve_reps)
        log(f"{name}: chunk loop {curves[name]['loop_ms']} ms = {curves[name]['tflops']} TFLOP/s "
            f"({100 * curves[name]['frac']:.1f}% of bf16 peak)")

    if args.copy_calibration:
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("calibration copy of 1 GiB done")

    log("timing the MLA latent decode batches")
    del dec_only, pre_only
    mla = mla_decode_summary(L, inputs, torch, timed, args.reps, args.warmup)
    log("timing the MLA latent prompt (both cache formats)")
    mla_pre = mla_prefill_summary(L, inputs, torch, args.curve_reps)

    log("timing the latency-predictor grid")
    alp = latency_predictor(L, loop, torch)
    log(f"latency predictor held-out MAPE: token count only {alp['token_count_only']['mape_holdout']:.3f}, "
        f"ALP features {alp['alp_features']['mape_holdout']:.3f}, with the fill term "
        f"{alp['alp_plus_fill']['mape_holdout']:.3f} (worst {alp['alp_plus_fill']['max_ape']:.3f})")
    sched = schedule_summary(L, per_chunk)
    log(f"schedules on the measured chunk latencies: CPP {sched['cpp']['makespan_ms']} ms, "
        f"VPP {sched['vpp']['makespan_ms']} ms, VPP-Async {sched['vpp_async']['makespan_ms']} ms")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a bounded sample")
        cpu = cpu_baseline(args, loop, torch)
        cpu["gpu_over_cpu_chunk_loop"] = round(prefill_tflops / cpu["value"], 1)

    w = loop.w
    traffic, traffic_note = recorded_traffic()
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded iid N(0,1) bf16 inputs; random paged block tables)",
        "config": {
            "workload": "131072-token prompt as 8 chunks of 16384 (64 q / 8 KV heads, d 128, bf16, paged KV "
                        "block 64) + mixed batch (2048-token chunk at past 65536 + 256 decodes, ctx U[1024,32768], "
                        "32 q / 8 KV heads, d 128)",
            "seq_len": w.seq_len, "chunk_len": w.chunk_len, "n_chunks": n_chunks, "heads": w.heads,
            "kv_heads": w.kv_heads, "head_dim": w.head_dim, "kv_block": 64,
            "decode_requests": mixed.w.decode_requests, "step_causal_flops": step_flops,
        },
        "per_chunk_ms": [round(x, 3) for x in per_chunk],
        "per_chunk_latency": chunk_stats,
        "per_chunk_fit": {"a_ms": round(a, 4), "b_ms_per_chunk": round(b, 4), "r2": round(r2, 5),
                          "b_over_a": round(b / a, 3) if a else None},
        "prefill_chunk_loop": {"ms": round(sum(per_chunk), 3), "tflops": round(prefill_tflops, 1)},
        "roofline": {
            "bound": "mfma",
            "kernel": DOMINANT,
            "achieved": round(prefill_tflops, 1),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(prefill_tflops / PEAK_BF16_TFLOPS, 4),
            "avg_launch_ms": round(sum(per_chunk) / n_chunks, 4),
            "avg_causal_flops_per_launch": sum(loop.flops) / n_chunks,
            "traffic": round(traffic["bytes_per_launch"]) if traffic else None,
            "traffic_note": ("HBM-side bytes per launch (L2 misses to the fabric, MALL hits included) from "
                             f"rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a 1 GiB copy; {TRAFFIC_SUMMARY}"
                             if traffic else traffic_note),
        },
        "mixed_batch": {
            "ms": round(median(mixed_ms), 4),
            "prefill_only_ms": round(pre_ms, 4),
            "decode_only_ms": round(dec_ms, 4),
            "prefill_tflops": round(mixed.prefill_flops / (pre_ms / 1e3) / 1e12, 1),
            "serial_sum_ms": round(pre_ms + dec_ms, 4),
            "ideal_overlap_ms": round(1e3 * max(mixed.prefill_flops / (PEAK_BF16_TFLOPS * 1e12),
                                                mixed.decode_bytes / (PEAK_HBM_GBPS * 1e9)), 4),
            "vs_serial": round(median(mixed_ms) / (pre_ms + dec_ms), 4),
            "note": ("one chunk_attn_varlen call; the library runs the prefill and decode parts at once on "
                     "two CU-masked halves of the GPU. serial_sum_ms = prefill-only + decode-only calls; "
                     "ideal_overlap_ms = max(prefill flops / dense bf16 peak, decode bytes / HBM peak)"),
            "roofline_decode": {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": PEAK_HBM_GBPS,
                                "unit": "GB/s", "frac": round(dec_gbps / PEAK_HBM_GBPS, 4),
                                "algorithmic_bytes": mixed.decode_bytes},
        },
        "gpu_clock_power": monitor.summary(),
        "copy_bandwidth": bw,
        "other_prompts": curves,
        "contiguous_cache": contig,
        "mla_decode": mla,
        "mla_prefill": mla_pre,
        "schedule_sim": sched,
        "latency_predictor": alp,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
