"""Measured HBM traffic of the layer's kernels from rocprofv3 counter passes.

Two steps, both run on the GPU host:

    # 1. a plain device copy of known size, for the counters' scale
    rocprofv3 --pmc FETCH_SIZE -f csv -d OUT/copy_fetch -o p -- \
        python3 -m mixture_memories_recurrence_amd.pmc_traffic copy --mib 1024
    rocprofv3 --pmc WRITE_SIZE -f csv -d OUT/copy_write -o p -- (same command)
    # 2. the bench steps on one stream (each stage one launch per step, as the
    #    roofline pass times it), without the decode and gradient parts
    rocprofv3 --pmc FETCH_SIZE -f csv -d OUT/fetch -o p -- python3 bench.py --steps 2 --warmup 1 \
        --no-decode --no-cpu-baseline --no-gla --no-single --no-bwd --serial
    rocprofv3 --pmc WRITE_SIZE -f csv -d OUT/write -o p -- (same command)
    python3 -m mixture_memories_recurrence_amd.pmc_traffic summarize --dir OUT --copy-mib 1024 \
        --workload l380m --out profiles/traffic_l380m.json

FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch.  Each is scaled by
the ratio of the copy's known bytes (read = written = the copy size) to what the
same counter reads for the copy, so that the figures are bytes of HBM traffic
per call of each entry point (the sum over the kernels it launches).  The JSON
also records a hash of each stage's kernel sources: bench.py reports the
traffic only while those sources are unchanged.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys

_PKG = os.path.dirname(os.path.abspath(__file__))
_CSRC = os.path.join(_PKG, "csrc")

# kernels launched by each entry point, and the sources they are built from
STAGES = {
    "route": (("k_route",), ("route.hip",)),
    "dispatch": (("k_count", "k_scan", "k_scatter"), ("dispatch.hip",)),
    "project": (("k_project",), ("project.hip",)),
    "chunk": (("k_gdn_prep", "k_gdn_chain", "k_gdn_chunk_valu"),
              ("gdn_chunk_mfma.hip", "chunk_mfma.h", "gdn_chunk_valu.hip")),
    "combine": (("k_combine",), ("combine.hip",)),
}


def stage_kernels(stage: str, dtype: str = "bf16"):
    """Kernels the stage launches for the given storage type ("bf16" or "f32")."""
    if stage == "chunk":
        return ("k_gdn_prep", "k_gdn_chain") if dtype == "bf16" else ("k_gdn_chunk_valu",)
    return STAGES[stage][0]


def source_hash(stage: str) -> str:
    h = hashlib.sha256()
    for f in STAGES[stage][1] + ("common.h",):
        with open(os.path.join(_CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _rows(d):
    f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not f:
        raise SystemExit("no counter_collection.csv under %s" % d)
    return list(csv.DictReader(open(f[0])))


def _per_kernel(d, counter):
    """Average counter value (KiB) per dispatch, by kernel name."""
    tot, n = collections.defaultdict(float), collections.Counter()
    for r in _rows(d):
        if r["Counter_Name"] != counter:
            continue
        tot[r["Kernel_Name"]] += float(r["Counter_Value"])
        n[r["Kernel_Name"]] += 1
    return {k: tot[k] / n[k] for k in tot}


def _copy_kib(d, counter):
    """Counter value of the largest dispatch of the copy run (KiB)."""
    vals = [float(r["Counter_Value"]) for r in _rows(d) if r["Counter_Name"] == counter]
    return max(vals)


def cmd_copy(a):
    import torch
    n = a.mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(a.reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print("copied %d MiB x %d" % (a.mib, a.reps), flush=True)


def cmd_summarize(a):
    known = a.copy_mib * (1 << 20)
    f_scale = known / (_copy_kib(os.path.join(a.dir, "copy_fetch"), "FETCH_SIZE") * 1024)
    w_scale = known / (_copy_kib(os.path.join(a.dir, "copy_write"), "WRITE_SIZE") * 1024)
    fetch = _per_kernel(os.path.join(a.dir, "fetch"), "FETCH_SIZE")
    write = _per_kernel(os.path.join(a.dir, "write"), "WRITE_SIZE")
    out = {"workload": a.workload, "copy_mib": a.copy_mib, "fetch_scale": round(f_scale, 4),
           "write_scale": round(w_scale, 4), "stages": {}}
    for st, (prefixes, _) in STAGES.items():
        ks = sorted(k for k in fetch if any(p in k for p in prefixes) and "_bwd" not in k)
        if not ks:
            continue
        rd = sum(fetch[k] for k in ks) * 1024 * f_scale
        wr = sum(write.get(k, 0.0) for k in ks) * 1024 * w_scale
        out["stages"][st] = {"kernels": ks, "read_bytes": round(rd), "write_bytes": round(wr),
                             "bytes_per_launch": round(rd + wr), "source_hash": source_hash(st)}
    with open(a.out, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def load_traffic(path: str, stage: str, workload: str):
    """bytes_per_launch of `stage` from a summary file, or None when the file
    is missing, is for another workload, or the stage's sources changed."""
    if not path or not os.path.exists(path):
        return None
    tr = json.load(open(path))
    s = tr.get("stages", {}).get(stage)
    if tr.get("workload") != workload or not s or s.get("source_hash") != source_hash(stage):
        return None
    return s["bytes_per_launch"]


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=3)
    s = sub.add_parser("summarize")
    s.add_argument("--dir", required=True)
    s.add_argument("--copy-mib", type=int, default=1024)
    s.add_argument("--workload", default="l380m")
    s.add_argument("--out", required=True)
    a = p.parse_args(argv)
    {"copy": cmd_copy, "summarize": cmd_summarize}[a.cmd](a)


if __name__ == "__main__":
    main(sys.argv[1:])
