"""Turn rocprofv3 CSV output into the short text summaries kept with the library.

    python -m mla_latent_kv_compress_amd.profiling stats  <kernel_stats.csv> --command "..." > summary.txt
    python -m mla_latent_kv_compress_amd.profiling traffic <fetch_dir> <write_dir> --kernel decode_attn \
        --workload dsv2_bf16 --splits 4 --command-fetch "..." --command-write "..."
    python -m mla_latent_kv_compress_amd.profiling counters <pmc_dir> [<pmc_dir> ...] --kernel decode_attn \
        --command "..." > counters.txt

`stats` prints rocprofv3's own per-kernel table (calls, total, average, min, max) for the
kernels of one run.  `traffic` reads two `--pmc` runs of the same program, one collecting
FETCH_SIZE and one WRITE_SIZE (KiB per dispatch), and scales each by what the same counter
reads for the plain device copy the program launches last (`bench.py --calibrate-copy`
copies 1 GiB after everything else: it fetches and writes 1 GiB, so the counters' ratio to
that is the factor that turns them into bytes).  It writes a JSON record with the HBM bytes per launch of the
named kernel, tagged with the sha256 of the kernel's source so that a reader can tell when
the record no longer describes the code.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30


def _csv(path, name):
    if os.path.isdir(path):
        hits = sorted(glob.glob(os.path.join(path, "**", name), recursive=True))
        if not hits:
            raise SystemExit(f"no {name} under {path}")
        path = hits[-1]
    return list(csv.DictReader(open(path)))


def _short(kernel_name):
    return kernel_name.split("(")[0].replace("void ", "").strip()


def stats_text(path, command, top=20):
    rows = _csv(path, "*kernel_stats.csv")
    out = [f"# rocprofv3 kernel statistics", f"# command: {command}", "",
           f"{'kernel':64s} {'calls':>6s} {'total_us':>10s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]
    for r in rows[:top]:
        ns = lambda k: float(r[k]) / 1e3
        out.append(f"{_short(r['Name'])[:64]:64s} {int(r['Calls']):6d} {ns('TotalDurationNs'):10.1f} "
                   f"{ns('AverageNs'):9.2f} {ns('MinNs'):9.2f} {ns('MaxNs'):9.2f} {float(r['Percentage']):6.2f}")
    return "\n".join(out) + "\n"


def _counter(path, counter):
    """{kernel: [value of each dispatch, in dispatch order]} for one counter."""
    per = {}
    rows = [r for r in _csv(path, "*counter_collection.csv") if r["Counter_Name"] == counter]
    for r in sorted(rows, key=lambda r: int(r["Dispatch_Id"])):
        per.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return per


def traffic_record(fetch_dir, write_dir, kernel, source, workload, splits, cmd_fetch, cmd_write):
    rec = {"kernel": kernel, "workload": workload, "splits": splits,
           "kernel_source": os.path.relpath(source, os.path.dirname(HERE)),
           "kernel_source_sha256": hashlib.sha256(open(source, "rb").read()).hexdigest(),
           "commands": {"FETCH_SIZE": cmd_fetch, "WRITE_SIZE": cmd_write}}
    total = 0.0
    for counter, path in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = _counter(path, counter)
        copy = per.get(COPY_KERNEL)
        names = [k for k in per if kernel in k]
        if not copy or len(names) != 1:
            raise SystemExit(f"{counter}: need the copy kernel and exactly one kernel matching {kernel!r}, "
                             f"found {sorted(per)}")
        copy_kib = copy[-1]                       # the 1 GiB calibration copy is the program's last copy
        factor = COPY_BYTES / (copy_kib * 1024.0)
        vals = per[names[0]]
        kib = statistics.median(vals)
        rec[counter] = {"kib_per_dispatch": kib, "dispatches": len(vals), "copy_kib": copy_kib,
                        "bytes_per_kib": factor * 1024.0, "bytes": kib * 1024.0 * factor}
        total += kib * 1024.0 * factor
        rec["kernel_name"] = names[0]
    rec["bytes_per_launch"] = total
    return rec


# Units of the gfx950 counters as summed over the device by rocprofv3: GRBM_GUI_ACTIVE counts
# shader-clock cycles once per XCD (8 XCDs); SQ_VALU_MFMA_BUSY_CYCLES counts matrix-core busy
# cycles summed over the 1024 SIMDs (it equals the sum over the kernel's MFMA instructions of
# their issue cycles: 16 per 16x16x32 bf16, 32 per 32x32x16 bf16); SQ_WAVE_CYCLES, SQ_WAIT_* and
# SQ_ACTIVE_INST_* count in units of 4 cycles summed over waves; SQ_LDS_BANK_CONFLICT and
# SQ_LDS_IDX_ACTIVE count cycles summed over the 256 CUs.
XCDS, SIMDS, CUS = 8, 1024, 256


def counters_text(dirs, kernel, command):
    """Per-dispatch medians of every counter in the PMC runs `dirs` for the kernel matching
    `kernel`, and the ratios derived from them."""
    vals, durs = {}, []
    for d in dirs:
        for r in _csv(d, "*counter_collection.csv"):
            if kernel not in r["Kernel_Name"]:
                continue
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            durs.append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    if not vals:
        raise SystemExit(f"no dispatch of {kernel!r}")
    med = {k: statistics.median(v) for k, v in vals.items()}
    dur_ns = statistics.median(durs)
    out = [f"# rocprofv3 counters of {kernel}", f"# command: {command}", "",
           f"median dispatch duration under the counters: {dur_ns / 1e3:.1f} us", ""]
    out += [f"{k:32s} {v:16.0f}   ({len(vals[k])} dispatches)" for k, v in sorted(med.items())]
    out += ["", "derived (see the units note in profiling.py):"]
    if "GRBM_GUI_ACTIVE" in med:
        cyc = med["GRBM_GUI_ACTIVE"] / XCDS
        out.append(f"  kernel cycles per XCD           {cyc:12.0f}  -> shader clock {cyc / dur_ns:.2f} GHz")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in med:
            out.append(f"  matrix-core busy                {med['SQ_VALU_MFMA_BUSY_CYCLES'] / (SIMDS * cyc):12.3f}"
                       "  (MFMA busy cycles per SIMD / kernel cycles)")
        if "SQ_LDS_BANK_CONFLICT" in med:
            out.append(f"  LDS bank-conflict cycles        {med['SQ_LDS_BANK_CONFLICT'] / (CUS * cyc):12.3f}"
                       "  (per CU / kernel cycles)")
        if "SQ_LDS_IDX_ACTIVE" in med:
            out.append(f"  LDS index unit active           {med['SQ_LDS_IDX_ACTIVE'] / (CUS * cyc):12.3f}"
                       "  (per CU / kernel cycles)")
    if "SQ_WAVE_CYCLES" in med:
        for k in ("SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_LDS",
                  "SQ_ACTIVE_INST_VALU", "SQ_WAIT_INST_LDS"):
            if k in med:
                out.append(f"  {k[3:].lower() + ' / wave cycles':32s}{med[k] / med['SQ_WAVE_CYCLES']:12.3f}")
    return "\n".join(out) + "\n"


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("path")
    s.add_argument("--command", required=True)
    s.add_argument("--top", type=int, default=20)
    t = sub.add_parser("traffic")
    t.add_argument("fetch")
    t.add_argument("write")
    t.add_argument("--kernel", required=True)
    t.add_argument("--source", default=os.path.join(HERE, "csrc", "k_decode.hip"))
    t.add_argument("--workload", required=True)
    t.add_argument("--splits", type=int, required=True)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--command", required=True)
    a = p.parse_args(argv)
    if a.what == "stats":
        sys.stdout.write(stats_text(a.path, a.command, a.top))
    elif a.what == "counters":
        sys.stdout.write(counters_text(a.dirs, a.kernel, a.command))
    else:
        rec = traffic_record(a.fetch, a.write, a.kernel, a.source, a.workload, a.splits,
                             a.command_fetch, a.command_write)
        json.dump(rec, sys.stdout, indent=1)
        sys.stdout.write("\n")


if __name__ == "__main__":
    main()
