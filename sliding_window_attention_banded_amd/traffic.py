"""HBM traffic of the forward kernel from rocprofv3 counters.

Two modes:

``run``: the program that rocprofv3 observes. It runs an elementwise kernel
over a buffer of known size (the calibration: FETCH_SIZE and WRITE_SIZE of
a plain streaming kernel must read that size) and then a few forwards of
one workload::

    rocprofv3 --pmc FETCH_SIZE -d OUT_F -o t -- \\
        python -m sliding_window_attention_banded_amd.traffic run --workload W
    rocprofv3 --pmc WRITE_SIZE -d OUT_W -o t -- \\
        python -m sliding_window_attention_banded_amd.traffic run --workload W

``summarize``: reads the two rocprofv3 databases, scales the forward
kernel's counters by copy_bytes / copy_counter, and writes (or updates) the
JSON record that ``bench.py`` reports as ``roofline.traffic``::

    python -m sliding_window_attention_banded_amd.traffic summarize \\
        OUT_F OUT_W --workload W --out profiles/attn_fwd_traffic.json

The record carries a hash of the kernel source; ``bench.py`` ignores it
once the kernels have changed.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sqlite3
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SRC = os.path.join(HERE, "csrc", "kernels.hpp")
COPY_BYTES = 256 * 2 ** 20
FWD_KERNEL = "attn_fwd"


def kernel_source_hash(path=KERNEL_SRC):
    """Hash of the kernel source without its comments and blank lines, so
    that an edit of the comments does not invalidate recorded counters."""
    code = []
    for line in open(path, encoding="utf-8"):
        line = line.split("//", 1)[0].rstrip()
        if line:
            code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def run(workload, reps):
    import torch

    from sliding_window_attention_banded_amd import Plan
    from sliding_window_attention_banded_amd.workloads import WORKLOADS, make_inputs

    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.add(src, 1.0, out=dst)  # the calibration kernel: COPY_BYTES read, COPY_BYTES written
    torch.cuda.synchronize()
    wl = WORKLOADS[workload]
    x = {k: (v.to(dev) if v is not None else None) for k, v in make_inputs(wl, 0).items()}
    with Plan(wl.batch, wl.heads, wl.n, wl.d, wl.window, wl.dilation, wl.causal,
              wl.global_idx, wl.torch_dtype) as pl:
        o = torch.empty_like(x["q"])
        lse = torch.empty((wl.batch, wl.heads, wl.n), dtype=torch.float32, device=dev)
        for _ in range(reps):
            pl.forward(x["q"], x["k"], x["v"], x["qg"], x["kg"], x["vg"], out=o, lse=lse)
        torch.cuda.synchronize()
    print(f"traffic run: copy {COPY_BYTES} B, {reps} forwards of {workload}", flush=True)


def _per_kernel(dbdir, counter):
    """{kernel name: [counter value per dispatch]} from a rocprofv3 db."""
    dbs = glob.glob(os.path.join(dbdir, "**", "*.db"), recursive=True)
    if not dbs:
        raise SystemExit(f"no rocprofv3 database under {dbdir}")
    out = {}
    for db in dbs:
        c = sqlite3.connect(db)
        cols = [r[1] for r in c.execute("pragma table_info(counters_collection)")]
        ci = {n: i for i, n in enumerate(cols)}
        for r in c.execute("select * from counters_collection"):
            if r[ci["counter_name"]] != counter:
                continue
            out.setdefault(r[ci["kernel_name"]], []).append(float(r[ci["value"]]))
    return out


def _pick(per, key):
    hits = [v for k, v in per.items() if key in k]
    if not hits:
        raise SystemExit(f"no dispatch of a kernel matching {key!r}: {sorted(per)}")
    return [x for v in hits for x in v]


def summarize(fetch_dir, write_dir, workload, out):
    f = _per_kernel(fetch_dir, "FETCH_SIZE")
    w = _per_kernel(write_dir, "WRITE_SIZE")
    # the calibration copy is the only dispatch of a copy kernel of COPY_BYTES;
    # take the largest copy-like dispatch
    def copy_val(per):
        cands = [max(v) for k, v in per.items() if "copy" in k.lower() or "elementwise" in k.lower()]
        if not cands:
            raise SystemExit(f"no copy kernel among {sorted(per)}")
        return max(cands)
    f_scale = COPY_BYTES / copy_val(f)
    w_scale = COPY_BYTES / copy_val(w)
    fv = statistics.median(_pick(f, FWD_KERNEL)) * f_scale
    wv = statistics.median(_pick(w, FWD_KERNEL)) * w_scale
    rec = {}
    if os.path.exists(out):
        rec = json.load(open(out))
    if rec.get("kernel_sha256_16") != kernel_source_hash():
        rec = {"workloads": {}}
    rec["kernel_sha256_16"] = kernel_source_hash()
    rec["kernel"] = FWD_KERNEL
    rec["method"] = ("rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE (KiB per dispatch); "
                     "each scaled by COPY_BYTES / (the same counter for an elementwise kernel "
                     "that reads and writes COPY_BYTES bytes); median over dispatches")
    rec["commands"] = [
        "rocprofv3 --pmc FETCH_SIZE -d OUT_F -o t -- python -m "
        "sliding_window_attention_banded_amd.traffic run --workload W",
        "rocprofv3 --pmc WRITE_SIZE -d OUT_W -o t -- python -m "
        "sliding_window_attention_banded_amd.traffic run --workload W",
        "python -m sliding_window_attention_banded_amd.traffic summarize OUT_F OUT_W "
        "--workload W --out profiles/attn_fwd_traffic.json"]
    rec["copy_bytes"] = COPY_BYTES
    rec["workloads"][workload] = {
        "fetch_bytes_per_launch": fv, "write_bytes_per_launch": wv,
        "hbm_bytes_per_launch": fv + wv,
        "fetch_scale": f_scale, "write_scale": w_scale,
    }
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(rec["workloads"][workload]))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="mode", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", required=True)
    r.add_argument("--reps", type=int, default=5)
    s = sub.add_parser("summarize")
    s.add_argument("fetch_dir")
    s.add_argument("write_dir")
    s.add_argument("--workload", required=True)
    s.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.mode == "run":
        sys.path.insert(0, os.path.dirname(HERE))
        run(a.workload, a.reps)
    else:
        summarize(a.fetch_dir, a.write_dir, a.workload, a.out)


if __name__ == "__main__":
    main()
