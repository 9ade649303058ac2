"""Summaries of rocprofv3 runs of bench.py, as the short text files kept with
the measurements.

  stats    kernel time per kernel from a --kernel-trace --stats run
           (<dir>/<prefix>_kernel_stats.csv), as a markdown table.
  traffic  HBM bytes per dispatch of the fused kernels from two --pmc runs,
           one with FETCH_SIZE and one with WRITE_SIZE.  The counters are
           scaled by what they read for the first device copy in the run:
           bench.py copies --copy-bytes (1 GiB) device to device before
           anything else, so that dispatch reads and writes a known size.
           Algorithmic bytes come from the kernel's template arguments (bits,
           group size) and the element count of one tensor: an encoder reads
           2 bytes and writes bits/8 + 4/group bytes per element, a decoder
           the reverse.  Writes a markdown table and, with --json, the file
           bench.py reads to fill its roofline's measured traffic (keyed by
           the sha256 of the fused-kernel source it was measured on).

usage:
  python -m kv_cache_compression_kvc_amd.profsum stats DIR [--prefix kt] [--top N]
  python -m kv_cache_compression_kvc_amd.profsum traffic FETCH_DIR WRITE_DIR --elements N
         [--prefix p] [--copy-bytes B] [--json OUT]
"""
import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CODEC_SRC = os.path.join(HERE, "csrc", "kvc_codec.hip")


def _short(name: str) -> str:
    name = name.strip()
    if name.endswith(")"):
        # drop the trailing parameter list (the parenthesis that closes last)
        depth = 0
        for i in range(len(name) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(name[i], 0)
            if depth == 0:
                name = name[:i]
                break
    name = name.replace("kvc::", "")
    name = name[5:].strip() if name.startswith("void ") else name.strip()
    return name if len(name) <= 96 else name[:93] + "..."


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern))
    if not hits:
        raise SystemExit(f"no file matches {pattern}")
    return hits[0]


def stats(d: str, prefix: str, top: int) -> str:
    path = _one(os.path.join(d, f"{prefix}_kernel_stats.csv"))
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = ["| kernel | calls | avg ms | min ms | max ms | share |", "|---|---|---|---|---|---|"]
    for r in rows[:top]:
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.3f} | "
                   f"{float(r['MinNs']) / 1e6:.3f} | {float(r['MaxNs']) / 1e6:.3f} | {float(r['Percentage']):.2f}% |")
    return "\n".join(out)


def _per_dispatch(path: str, counter: str):
    """{dispatch id: (kernel name, counter value summed over its rows)} in file order."""
    vals = collections.OrderedDict()
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        k = int(r["Dispatch_Id"])
        name, v = vals.get(k, (r["Kernel_Name"], 0.0))
        vals[k] = (name, v + float(r["Counter_Value"]))
    return vals


def _alg_bytes(short: str, elements: int):
    m = re.match(r"k_(encode|decode)_(channel|token|token_m)<(\d+), (\d+)", short)
    if m:
        bits, group = int(m.group(3)), int(m.group(4))
    else:
        m = re.match(r"k_decode_token_m<(\d+),", short)      # 2-bit codes, template argument: group
        if not m:
            return None
        bits, group = 2, int(m.group(1))
    small = elements * bits / 8 + elements * 4 / group
    big = elements * 2
    return (big, small) if "encode" in short else (small, big)


def traffic(fdir: str, wdir: str, prefix: str, elements: int, copy_bytes: int):
    fetch = _per_dispatch(_one(os.path.join(fdir, f"{prefix}_counter_collection.csv")), "FETCH_SIZE")
    write = _per_dispatch(_one(os.path.join(wdir, f"{prefix}_counter_collection.csv")), "WRITE_SIZE")

    def first_copy(vals):
        for name, v in vals.values():
            if "copyBuffer" in name:
                return v
        raise SystemExit("no device copy in the run")

    # counters are KiB per dispatch; the copy moves copy_bytes each way
    fscale = copy_bytes / (first_copy(fetch) * 1024.0)
    wscale = copy_bytes / (first_copy(write) * 1024.0)

    def per_kernel(vals, scale):
        acc = collections.defaultdict(list)
        for name, v in vals.values():
            acc[_short(name)].append(v * 1024.0 * scale)
        return {k: (sum(x) / len(x), len(x)) for k, x in acc.items()}

    fk, wk = per_kernel(fetch, fscale), per_kernel(write, wscale)
    res = {}
    for k in sorted(set(fk) | set(wk), key=lambda k: -(fk.get(k, (0, 0))[0] + wk.get(k, (0, 0))[0])):
        if not k.startswith("k_"):
            continue
        rd, n = fk.get(k, (0.0, 0))
        wr, _ = wk.get(k, (0.0, 0))
        res[k] = {"dispatches": n, "read_bytes": rd, "write_bytes": wr, "alg": _alg_bytes(k, elements)}
    return fscale, wscale, res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("dir")
    a.add_argument("--prefix", default="kt")
    a.add_argument("--top", type=int, default=24)
    b = sub.add_parser("traffic")
    b.add_argument("fetch_dir")
    b.add_argument("write_dir")
    b.add_argument("--prefix", default="p")
    b.add_argument("--elements", type=int, required=True, help="elements of one tensor (layers x tokens x heads x 128)")
    b.add_argument("--copy-bytes", type=int, default=1 << 30)
    b.add_argument("--json", default=None)
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        print(stats(args.dir, args.prefix, args.top))
        return
    fs, ws, res = traffic(args.fetch_dir, args.write_dir, args.prefix, args.elements, args.copy_bytes)
    sha = hashlib.sha256(open(CODEC_SRC, "rb").read()).hexdigest()
    print(f"Scaling: the first device copy ({args.copy_bytes} bytes each way) reads {1 / fs:.4f} and writes "
          f"{1 / ws:.4f} of its size in FETCH_SIZE / WRITE_SIZE, so counts are multiplied by {fs:.3f} "
          f"(fetch) and {ws:.3f} (write).\n")
    print(f"Fused-kernel source (kv_cache_compression_kvc_amd/csrc/kvc_codec.hip) sha256: `{sha}`\n")
    print("| kernel | dispatches | read GB | write GB | algorithmic read GB | algorithmic write GB | read / alg | write / alg |")
    print("|---|---|---|---|---|---|---|---|")
    for k, r in res.items():
        alg = r["alg"]
        cells = ["", "", "", ""] if alg is None else [
            f"{alg[0] / 1e9:.3f}", f"{alg[1] / 1e9:.3f}", f"{r['read_bytes'] / alg[0]:.3f}", f"{r['write_bytes'] / alg[1]:.3f}"]
        print(f"| `{k}` | {r['dispatches']} | {r['read_bytes'] / 1e9:.4f} | {r['write_bytes'] / 1e9:.4f} | " + " | ".join(cells) + " |")
    if args.json:
        kinds = {}
        for k, r in res.items():
            if r["alg"] is None:
                continue
            role = ("ENCODE" if "encode" in k else "DECODE") + ("_K" if "channel" in k else "_V")
            kinds[role] = {"name": k, "read_bytes": r["read_bytes"], "write_bytes": r["write_bytes"],
                           "alg_read_bytes": r["alg"][0], "alg_write_bytes": r["alg"][1]}
        with open(args.json, "w") as f:
            json.dump({"codec_sha256": sha, "fetch_scale": fs, "write_scale": ws, "kernels": kinds}, f, indent=1)
            f.write("\n")


if __name__ == "__main__":
    sys.exit(main())
