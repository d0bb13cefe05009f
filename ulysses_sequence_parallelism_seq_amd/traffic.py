"""HBM traffic of the attention backward from rocprofv3 counter runs.

Two counter runs of bench.py (one with FETCH_SIZE, one with WRITE_SIZE, in
KiB per dispatch) give the bytes each kernel moved between L2 and memory. The
counters are calibrated with a plain device-to-device copy of known size in
the same run (bench.py copies one 1 GiB input tensor with torch's copy_, which
runs the HIP runtime's own copy kernel: it reads and writes every byte once),
independently of this library's kernels. The calibrated figures cover the
backward's kernels (the roofline's "traffic") and the two permute kernels
(their HBM bytes against the algorithmic read + write of every element). They
are stored with a hash of the compiled library they were taken with, so that
any change of its code invalidates them (and an edit that leaves the compiled
code byte-identical, such as a comment, does not).

  python -m ulysses_sequence_parallelism_seq_amd.traffic FETCH_DIR WRITE_DIR OUT.txt "COMMANDS"

reads the two counter_collection.csv files and writes OUT.txt; bench.py
calls read_traffic(OUT.txt) to fill its roofline "traffic" field.
"""

from __future__ import annotations

import csv
import glob
import hashlib
import os
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libulysses.so")
BWD_KERNELS = ("attn_dkdv_bf16_kernel<128,false>", "attn_dq_bf16_kernel<128,false>", "delta_bf16_kernel<128>")
PERMUTE_KERNELS = ("permute_seq_to_head", "permute_head_to_seq")
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def library_sha256() -> str | None:
    """sha256 of the built library, or None if it has not been built."""
    if not os.path.exists(LIBRARY):
        return None
    h = hashlib.sha256()
    with open(LIBRARY, "rb") as f:
        for block in iter(lambda: f.read(1 << 20), b""):
            h.update(block)
    return h.hexdigest()


def _short(name: str) -> str:
    """Kernel name without namespace, arguments or spaces (one token of the summary's lines)."""
    for prefix in ("void ", "(anonymous namespace)::"):
        if name.startswith(prefix):
            name = name[len(prefix):]
    return name.split("(")[0].replace(" ", "")


def _per_dispatch(csv_dir: str, counter: str) -> dict:
    """Average counter value per dispatch of each kernel. For the runtime's copy
    kernel only the dispatches of the largest grid (the calibration copies of
    one whole tensor) count; for the permute kernels only those of the smallest
    grid (one tensor per launch: bench.py also moves q, k, v and dq, dk, dv
    three to a launch)."""
    values = {}
    for path in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                k = _short(row["Kernel_Name"])
                values.setdefault(k, []).append((int(row.get("Grid_Size") or 0), float(row["Counter_Value"])))
    out = {}
    for k, vs in values.items():
        if k == COPY_KERNEL:
            g = max(gs for gs, _ in vs)
            vs = [x for x in vs if x[0] == g]
        elif k in PERMUTE_KERNELS:
            g = min(gs for gs, _ in vs)
            vs = [x for x in vs if x[0] == g]
        out[k] = sum(v for _, v in vs) / len(vs)
    return out


def write_traffic(fetch_dir: str, write_dir: str, out: str, commands: str, copy_bytes: int) -> None:
    fetch = _per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _per_dispatch(write_dir, "WRITE_SIZE")
    lines = [
        "# HBM traffic per dispatch (rocprofv3 FETCH_SIZE / WRITE_SIZE, KiB), long workload",
        f"# commands: {commands}",
        f"library_sha256 {library_sha256()}",
        f"copy {COPY_KERNEL} bytes={copy_bytes} fetch_kib={fetch[COPY_KERNEL]:.1f} write_kib={write[COPY_KERNEL]:.1f}",
    ]
    for k in BWD_KERNELS:
        lines.append(f"kernel {k} fetch_kib={fetch[k]:.1f} write_kib={write[k]:.1f}")
    for k in PERMUTE_KERNELS:
        lines.append(f"permute {k} fetch_kib={fetch[k]:.1f} write_kib={write[k]:.1f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def read_traffic(path: str):
    """Calibrated HBM bytes of one attention-backward call ("bytes") and of one
    call of each permute kernel ("permute": name -> bytes), or None if the
    figures are stale or missing."""
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            parts = line.split()
            if not parts or parts[0].startswith("#"):
                continue
            if parts[0] == "library_sha256":
                rec["sha"] = parts[1]
            elif parts[0] in ("copy", "kernel", "permute"):
                rec[(parts[0], parts[1])] = dict(p.split("=") for p in parts[2:])
    if rec.get("sha") is None or rec.get("sha") != library_sha256():
        return None
    entries = [(k, v) for k, v in rec.items() if isinstance(k, tuple)]
    copy = next(v for (kind, _), v in entries if kind == "copy")
    copy_kib = float(copy["bytes"]) / 1024.0  # the copy reads this many KiB and writes as many
    f_scale = copy_kib / float(copy["fetch_kib"])
    w_scale = copy_kib / float(copy["write_kib"])
    total = 0.0
    permute = {}
    for (kind, name), v in entries:
        kib = float(v["fetch_kib"]) * f_scale + float(v["write_kib"]) * w_scale
        if kind == "kernel":
            total += kib
        elif kind == "permute":
            permute[name] = kib * 1024.0
    return {"bytes": total * 1024.0, "fetch_scale": f_scale, "write_scale": w_scale, "permute": permute}


if __name__ == "__main__":
    write_traffic(sys.argv[1], sys.argv[2], sys.argv[3], sys.argv[4], int(sys.argv[5]))
