"""Summaries of rocprofv3 output, for the text files kept with the measurements.

  python -m bit_ternary_attention_amd.profsum trace <results.db> [name-filter]
      per-kernel calls and durations from a --kernel-trace database
  python -m bit_ternary_attention_amd.profsum traffic <fetch.csv> <write.csv> <calib-name> <calib-bytes>
      per-kernel FETCH_SIZE / WRITE_SIZE (KiB per dispatch) from two --pmc runs, and the
      HBM bytes per dispatch after scaling each counter by what it reads for the
      calibration kernel (a plain copy that reads and writes calib-bytes)
  python -m bit_ternary_attention_amd.profsum record <fetch.csv> <write.csv> <calib-name> <calib-bytes>
      <kernel-filter> <workload> <out.json> <source>...
      the traffic of one kernel as a JSON record, with the SHA-256 of the sources it was
      built from (a reader can tell whether the kernel has changed since)
  python -m bit_ternary_attention_amd.profsum calls <results.db> <name-filter>
      per-call durations of the matching kernels, in launch order
  python -m bit_ternary_attention_amd.profsum counters <name-filter> <counter_collection.csv>...
      per-dispatch averages of every counter in the given --pmc runs, over the dispatches of
      the matching kernel with the largest grid (one launch shape out of a run that mixes several)
  python -m bit_ternary_attention_amd.profsum record-counters <name-filter> <workload> <units> <out.json>
      <counter_collection.csv>... -- <source>...
      the counters mode's averages of one kernel as a JSON record (with the instruction counts
      divided by the attended 16-token units of one launch), keyed by kernel kind and workload,
      with the SHA-256 of its sources
  --largest (traffic, record): average only each kernel's dispatches that fetch at least
      90% of its largest one (one launch size out of a run that mixes several)
"""
import csv
import hashlib
import json
import os
import sqlite3
import sys


# kernel kinds as the library's timing hooks name them
KINDS = {"k_absmean_partial": "absmean", "k_gamma_finalize": "finalize", "k_pack": "pack",
         "k_decode_mfma": "decode", "k_decode<": "decode", "k_merge": "merge", "k_retier": "retier"}


def trace(db_path: str, name_filter: str = "vk::"):
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, count(*), sum(duration), avg(duration), min(duration), max(duration) "
                      "from kernels group by name order by sum(duration) desc").fetchall()
    out = []
    for name, n, tot, avg, mn, mx in rows:
        if name_filter and name_filter not in name:
            continue
        out.append((name, n, tot / 1e3, avg / 1e3, mn / 1e3, mx / 1e3))
    return out


def short(name: str) -> str:
    for junk in ("vk::(anonymous namespace)::", "(vk::AppendArgs)", "(vk::DecodeArgs)", "(vk::QuantArgs)",
                 "(vk::RetierArgs)"):
        name = name.replace(junk, "")
    return name


def _counter(path: str, counter: str, largest: bool = False):
    per = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    if largest:
        per = {k: [x for x in v if x >= 0.9 * max(v)] for k, v in per.items()}
    return {k: sum(v) / len(v) for k, v in per.items()}, {k: len(v) for k, v in per.items()}


def traffic(fetch_csv: str, write_csv: str, calib_name: str, calib_bytes: float, largest: bool = False):
    fetch, n_f = _counter(fetch_csv, "FETCH_SIZE", largest)
    write, _ = _counter(write_csv, "WRITE_SIZE", largest)
    cf = [v for k, v in fetch.items() if calib_name in k]
    cw = [v for k, v in write.items() if calib_name in k]
    if not cf or not cw:
        raise SystemExit(f"calibration kernel '{calib_name}' not found")
    f_scale = cf[0] * 1024.0 / calib_bytes  # counter bytes per true byte
    w_scale = cw[0] * 1024.0 / calib_bytes
    rows = []
    for k in fetch:
        if k not in write:
            continue
        hbm = fetch[k] * 1024.0 / f_scale + write[k] * 1024.0 / w_scale
        rows.append((k, n_f[k], fetch[k], write[k], hbm))
    rows.sort(key=lambda r: -r[4] * r[1])
    return f_scale, w_scale, rows


def sources_sha256(paths):
    h = hashlib.sha256()
    for p in paths:
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_averages(path: str, filt: str):
    """(kernel, grid, dispatches, {counter: average}) over the dispatches of the matching kernel
    with the largest grid in one --pmc csv, or None."""
    rows = [r for r in csv.DictReader(open(path)) if filt in r["Kernel_Name"]]
    if not rows:
        return None
    grid = max(int(r["Grid_Size"]) for r in rows)
    per = {}
    for r in rows:
        if int(r["Grid_Size"]) == grid:
            per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    n = len(next(iter(per.values())))
    return short(rows[0]["Kernel_Name"]), grid, n, {k: sum(v) / len(v) for k, v in per.items()}


def main():
    largest = "--largest" in sys.argv
    sys.argv = [a for a in sys.argv if a != "--largest"]
    mode = sys.argv[1]
    if mode == "trace":
        filt = sys.argv[3] if len(sys.argv) > 3 else "vk::"
        print(f"{'kernel':70s} {'calls':>6s} {'total_us':>10s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}")
        for name, n, tot, avg, mn, mx in trace(sys.argv[2], filt):
            print(f"{short(name)[:70]:70s} {n:6d} {tot:10.1f} {avg:9.3f} {mn:9.3f} {mx:9.3f}")
    elif mode == "traffic":
        f_scale, w_scale, rows = traffic(sys.argv[2], sys.argv[3], sys.argv[4], float(sys.argv[5]), largest)
        print(f"calibration: FETCH_SIZE reads {f_scale:.5f} and WRITE_SIZE {w_scale:.5f} of the copied bytes")
        print(f"{'kernel':70s} {'n':>4s} {'FETCH KiB':>12s} {'WRITE KiB':>12s} {'HBM bytes/dispatch':>20s}")
        for k, n, fk, wk, hbm in rows:
            if "vk::" in k:
                print(f"{short(k)[:70]:70s} {n:4d} {fk:12.1f} {wk:12.1f} {hbm:20.0f}")
    elif mode == "record":
        fetch_csv, write_csv, calib, cbytes, kfilt, workload, out = sys.argv[2:9]
        srcs = sys.argv[9:]
        f_scale, w_scale, rows = traffic(fetch_csv, write_csv, calib, float(cbytes), largest)
        hit = [r for r in rows if kfilt in r[0]]
        if not hit:
            raise SystemExit(f"kernel '{kfilt}' not found")
        k, n, fk, wk, hbm = hit[0]
        rec = json.load(open(out)) if os.path.exists(out) else {}
        kind = next((v for key, v in KINDS.items() if key in k), "other")
        rec[f"{kind}|{workload}"] = {
            "kind": kind, "kernel": short(k), "workload": workload, "dispatches": n,
            "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
            "fetch_scale": f_scale, "write_scale": w_scale, "hbm_bytes_per_dispatch": hbm,
            "sources": [os.path.relpath(p) for p in srcs], "source_sha256": sources_sha256(srcs)}
        with open(out, "w") as f:
            json.dump(rec, f, indent=1, sort_keys=True)
        print(json.dumps(rec[f"{kind}|{workload}"], indent=1))
    elif mode == "calls":
        db = sqlite3.connect(sys.argv[2])
        rows = db.execute("select name, duration from kernels order by start").fetchall()
        durs = [d / 1e3 for n, d in rows if sys.argv[3] in n]
        print(f"{len(durs)} calls of '{sys.argv[3]}' (us, launch order): " + " ".join(f"{d:.2f}" for d in durs))
    elif mode == "counters":
        filt, paths = sys.argv[2], sys.argv[3:]
        for path in paths:
            got = counter_averages(path, filt)
            if got is None:
                continue
            name, grid, n, per = got
            print(f"{name} (grid {grid} threads, {n} dispatches averaged; {os.path.relpath(path)}):")
            for k in sorted(per):
                print(f"  {k:28s} {per[k]:18.2f}")
    elif mode == "record-counters":
        filt, workload, units, out = sys.argv[2], sys.argv[3], float(sys.argv[4]), sys.argv[5]
        rest = sys.argv[6:]
        cut = rest.index("--")
        paths, srcs = rest[:cut], rest[cut + 1:]
        vals, name = {}, None
        for path in paths:
            got = counter_averages(path, filt)
            if got is not None:
                name = got[0]
                vals.update(got[3])
        if not vals:
            raise SystemExit(f"kernel '{filt}' not found")
        per_unit = {k[len("SQ_INSTS_"):].lower() + "_per_unit": round(v / units, 2)
                    for k, v in vals.items() if k.startswith("SQ_INSTS_")}
        rec = json.load(open(out)) if os.path.exists(out) else {}
        kind = next((v for key, v in KINDS.items() if key in name), "other")
        rec[f"{kind}|{workload}"] = {
            "kind": kind, "kernel": name, "workload": workload, "units_per_launch": units,
            "counters": {k: round(v, 2) for k, v in sorted(vals.items())}, "per_unit": per_unit,
            "sources": [os.path.relpath(p) for p in srcs], "source_sha256": sources_sha256(srcs)}
        with open(out, "w") as f:
            json.dump(rec, f, indent=1, sort_keys=True)
        print(json.dumps(rec[f"{kind}|{workload}"], indent=1))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main()
