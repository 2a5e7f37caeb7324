"""Summaries of rocprofv3 output for the kernels of this library (the figures kept under profiles/).

  python profile_summary.py trace KERNEL_TRACE_CSV --kernel SUBSTR [--phases 500,200,200] [--period P]
      Per-phase duration statistics of the matching dispatches, in dispatch order.  bench.py launches
      the headline kernel `--warmup` times, then `--steps` times in the timed region, then `--steps`
      times each between its own pair of events, so --phases W,K,K splits the trace the same way and
      the middle phase is the timed region's average kernel duration.  With --period P every step
      launches P kernels (one per layer of a layer-by-layer network): the phases count steps, and
      each phase is also broken down by launch position within the step.
  python profile_summary.py counters COUNTER_CSV --kernel SUBSTR [--skip N] [--period P]
      Each counter's per-dispatch value (median, min, max) over the matching dispatches, the first N
      steps skipped; with --period P (P launches per step) separately for each launch position.
  python profile_summary.py traffic --fetch CSV --write CSV --copy-fetch CSV --copy-write CSV
          --kernel SUBSTR --workload KEY --label NAME --algorithmic-bytes B [--update]
      HBM bytes per dispatch: FETCH_SIZE and WRITE_SIZE (KiB) each scaled by what the same counter
      reads for bench.py's plain device copy (--copy-probe: 256 MiB read and written per launch);
      --update records the result, with the hash of the kernel sources, in profiles/traffic.json.
  python profile_summary.py static-mix [--kernel REGEX ...]
      Instruction counts of the fused kernels in the gfx950 assembly of mlp_kernels.hip, compiled with
      the library's own flags: the whole kernel and its largest basic block (the tile loop).
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import re
import statistics
import subprocess
import sys
import tempfile
from pathlib import Path

ROOT = Path(__file__).resolve().parent
COPY_PROBE_BYTES = 256 << 20  # bench.py --copy-probe: one 256 MiB device copy per launch


def _rows(path, kernel):
    with open(path, newline="") as f:
        return [r for r in csv.DictReader(f) if kernel in r["Kernel_Name"]]


def _stats(xs):
    return {"n": len(xs), "mean": statistics.fmean(xs), "median": statistics.median(xs), "min": min(xs),
            "max": max(xs)}


def trace(args) -> dict:
    rows = sorted(_rows(args.csv, args.kernel), key=lambda r: int(r["Start_Timestamp"]))
    if not rows:
        raise SystemExit("no dispatch of a kernel matching %r in %s" % (args.kernel, args.csv))
    us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    period = args.period
    if len(us) % period:
        raise SystemExit("%d matching dispatches, not a multiple of the period %d" % (len(us), period))
    phases = [int(p) * period for p in args.phases.split(",")] if args.phases else [len(us)]
    if sum(phases) != len(us):
        raise SystemExit("%d matching dispatches, phases add up to %d" % (len(us), sum(phases)))
    out, at = {"kernel": rows[0]["Kernel_Name"], "phases": []}, 0
    for n in phases:
        out["phases"].append(_stats(us[at:at + n]))
        at += n
    out["all"] = _stats(us)
    print("kernel:", out["kernel"])
    print("| Dispatches | Calls | Avg (us) | Median | Min | Max |")
    print("|---|---|---|---|---|---|")
    at = 0
    for n, s in zip(phases, out["phases"]):
        print("| %d..%d | %d | %.2f | %.2f | %.2f | %.2f |" % (at, at + n - 1, n, s["mean"], s["median"], s["min"], s["max"]))
        at += n
    s = out["all"]
    print("| all | %d | %.2f | %.2f | %.2f | %.2f |" % (s["n"], s["mean"], s["median"], s["min"], s["max"]))
    if period > 1:
        out["by_position"] = []
        print("\n| Phase | Position | Kernel | Calls | Avg (us) | Median | Min | Max |")
        print("|---|---|---|---|---|---|---|---|")
        at = 0
        for ph, n in enumerate(phases):
            for pos in range(period):
                sel = us[at + pos:at + n:period]
                st = _stats(sel)
                full = rows[at + pos]["Kernel_Name"]
                name = full[:full.rindex("(")].split("::")[-1]  # drop the argument list and scopes
                name = name[5:] if name.startswith("void ") else name  # and the return type
                out["by_position"].append({"phase": ph, "position": pos, "kernel": name, **st})
                print("| %d | %d | `%s` | %d | %.2f | %.2f | %.2f | %.2f |" % (ph, pos, name, st["n"], st["mean"], st["median"],
                                                                      st["min"], st["max"]))
            steps = [sum(us[at + i * period:at + (i + 1) * period]) for i in range(n // period)]
            print("| %d | sum per step | | %d | %.2f | %.2f | %.2f | %.2f |" % (ph, len(steps), statistics.fmean(steps),
                                                                            statistics.median(steps), min(steps), max(steps)))
            at += n
    return out


def _per_dispatch(path, kernel, skip=0):
    """counter -> [value per dispatch], dispatches in order, the first `skip` dropped."""
    per = collections.defaultdict(dict)
    for r in _rows(path, kernel):
        d = int(r["Dispatch_Id"])
        per[r["Counter_Name"]][d] = per[r["Counter_Name"]].get(d, 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit("no counters for a kernel matching %r in %s" % (kernel, path))
    return {c: [v for _, v in sorted(ds.items())][skip:] for c, ds in per.items()}


def counters(args) -> dict:
    per = _per_dispatch(args.csv, args.kernel, args.skip * args.period)
    out = {}
    for pos in range(args.period):
        if args.period > 1:
            print("\nlaunch position %d of %d per step:" % (pos, args.period))
        print("| Counter | Dispatches | Median | Min | Max |")
        print("|---|---|---|---|---|")
        for c in sorted(per):
            s = _stats(per[c][pos::args.period])
            out[(c, pos) if args.period > 1 else c] = s
            print("| %s | %d | %.1f | %.1f | %.1f |" % (c, s["n"], s["median"], s["min"], s["max"]))
    return out


def kernel_source_hash() -> str:
    sys.path.insert(0, str(ROOT))
    import bench  # noqa: E402  (the hash bench.py checks before it reports roofline.traffic)

    return bench.kernel_source_hash()


def traffic(args) -> dict:
    fetch = statistics.median(_per_dispatch(args.fetch, args.kernel)["FETCH_SIZE"])
    write = statistics.median(_per_dispatch(args.write, args.kernel)["WRITE_SIZE"])
    copy = "copyBuffer"
    cf = statistics.median(_per_dispatch(args.copy_fetch, copy)["FETCH_SIZE"])
    cw = statistics.median(_per_dispatch(args.copy_write, copy)["WRITE_SIZE"])
    known_kib = COPY_PROBE_BYTES / 1024
    fs, ws = known_kib / cf, known_kib / cw
    total = int(round((fetch * fs + write * ws) * 1024))
    kernel_name = _rows(args.fetch, args.kernel)[0]["Kernel_Name"]
    rec = {"fetch_kib": fetch, "write_kib": write, "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
           "bytes_per_launch": total, "algorithmic_bytes": args.algorithmic_bytes,
           "source_hash": kernel_source_hash(),
           "dispatches": len(_per_dispatch(args.fetch, args.kernel)["FETCH_SIZE"]), "profiled_kernel": kernel_name}
    print("| Counter | Kernel (KiB) | Copy probe (KiB) | Copy known (KiB) | Scale | Kernel scaled (bytes) |")
    print("|---|---|---|---|---|---|")
    print("| FETCH_SIZE | %.1f | %.1f | %.0f | %.4f | %d |" % (fetch, cf, known_kib, fs, int(fetch * fs * 1024)))
    print("| WRITE_SIZE | %.1f | %.1f | %.0f | %.4f | %d |" % (write, cw, known_kib, ws, int(write * ws * 1024)))
    print("scaled total %d B per launch; algorithmic %d B; ratio %.3f" % (total, args.algorithmic_bytes,
                                                                        total / args.algorithmic_bytes))
    if args.update:
        path = ROOT / "profiles" / "traffic.json"
        data = json.loads(path.read_text()) if path.exists() else {}
        data.setdefault(args.workload, {})[args.label] = rec
        path.write_text(json.dumps(data, indent=1) + "\n")
        print("recorded in", path)
    return rec


def _category(op: str) -> str:
    if op.startswith("v_mfma"):
        return "mfma"
    if op.startswith("v_"):
        return "valu"
    if op.startswith("ds_"):
        return "lds"
    if op.startswith(("global_", "buffer_", "flat_")):
        return "vmem"
    if op.startswith("s_waitcnt"):
        return "s_waitcnt"
    if op.startswith("s_nop"):
        return "s_nop"
    if op.startswith(("s_load", "s_buffer_load")):
        return "smem"
    if op.startswith("s_cbranch") or op.startswith("s_branch"):
        return "branch"
    if op.startswith("s_"):
        return "salu"
    return "other"


CATEGORIES = ["mfma", "valu", "lds", "vmem", "salu", "smem", "branch", "s_waitcnt", "s_nop"]


def static_mix(args) -> dict:
    sys.path.insert(0, str(ROOT))
    from mlp_neural_shading_amd import build as B  # noqa: E402

    with tempfile.TemporaryDirectory() as tmp:
        asm = Path(tmp) / "mlp_kernels.s"
        cmd = [B.HIPCC, "--offload-arch=" + B.ARCH, *B.COMMON, "-I", str(B.INCLUDE), "--cuda-device-only", "-S",
               "-x", "hip", str(B.CSRC / "mlp_kernels.hip"), "-o", str(asm)]
        subprocess.run(cmd, check=True, capture_output=True)
        lines = asm.read_text().splitlines()
        names = sorted({l.split(":")[0] for l in lines if re.match(r"^_Z\S*mlp_fused\S*:", l)})
        dem = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True,
                             text=True, check=True).stdout.splitlines()
    pats = [re.compile(p) for p in (args.kernel or [r"."])]
    out = {}
    for mangled, pretty in zip(names, dem):
        if not any(p.search(pretty) for p in pats):
            continue
        start = next(i for i, l in enumerate(lines) if l.startswith(mangled + ":"))
        end = next(i for i in range(start, len(lines)) if lines[i].startswith(".Lfunc_end"))
        blocks, cur = [], []
        for l in lines[start + 1:end]:
            if re.match(r"^\.LBB\S+:", l):
                blocks.append(cur)
                cur = []
                continue
            t = l.strip()
            if t and not t.startswith((";", ".")):
                cur.append(t.split()[0])
        blocks.append(cur)
        ops = [o for b in blocks for o in b]
        loop = max(blocks, key=len)
        whole = collections.Counter(_category(o) for o in ops)
        inner = collections.Counter(_category(o) for o in loop)
        valu_ops = collections.Counter(o for o in loop if _category(o) == "valu")
        out[pretty] = {"kernel": dict(whole), "loop": dict(inner), "loop_valu": dict(valu_ops.most_common(10))}
        print(pretty)
        print("  kernel: " + " ".join("%s=%d" % (c, whole[c]) for c in CATEGORIES) + " total=%d" % len(ops))
        print("  loop:   " + " ".join("%s=%d" % (c, inner[c]) for c in CATEGORIES) + " total=%d" % len(loop))
        print("  loop VALU by opcode: " + ", ".join("%s %d" % kv for kv in valu_ops.most_common(10)))
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("csv")
    t.add_argument("--kernel", required=True)
    t.add_argument("--phases", default="")
    t.add_argument("--period", type=int, default=1)
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("--kernel", required=True)
    c.add_argument("--skip", type=int, default=0)
    c.add_argument("--period", type=int, default=1)
    f = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--kernel", "--workload", "--label"):
        f.add_argument(a, required=True)
    f.add_argument("--algorithmic-bytes", type=int, required=True)
    f.add_argument("--update", action="store_true")
    s = sub.add_parser("static-mix")
    s.add_argument("--kernel", action="append")
    args = ap.parse_args(argv)
    {"trace": trace, "counters": counters, "traffic": traffic, "static-mix": static_mix}[args.cmd](args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
