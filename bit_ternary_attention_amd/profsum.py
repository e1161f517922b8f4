"""Summarises a rocprofv3 kernel-trace database: per-kernel calls and durations.

Usage: python -m bit_ternary_attention_amd.profsum <results.db> [name-filter]
"""
import sqlite3
import sys


def summarise(db_path: str, name_filter: str = "vk::"):
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, count(*), sum(duration), avg(duration), min(duration), max(duration) "
                      "from kernels group by name order by sum(duration) desc").fetchall()
    out = []
    for name, n, tot, avg, mn, mx in rows:
        if name_filter and name_filter not in name:
            continue
        out.append((name, n, tot / 1e3, avg / 1e3, mn / 1e3, mx / 1e3))
    return out


def main():
    path = sys.argv[1]
    filt = sys.argv[2] if len(sys.argv) > 2 else "vk::"
    print(f"{'kernel':70s} {'calls':>6s} {'total_us':>10s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}")
    for name, n, tot, avg, mn, mx in summarise(path, filt):
        short = name.replace("vk::(anonymous namespace)::", "").replace("(vk::AppendArgs)", "").replace(
            "(vk::DecodeArgs)", "")
        print(f"{short[:70]:70s} {n:6d} {tot:10.1f} {avg:9.3f} {mn:9.3f} {mx:9.3f}")


if __name__ == "__main__":
    main()
