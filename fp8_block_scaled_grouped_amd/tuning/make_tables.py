"""Writes the measured plan tables the library compiles in, from sweep records.

    python bench.py --sweep dense   > fp8_block_scaled_grouped_amd/tuning/dense_sweep.jsonl
    python bench.py --sweep block_m > fp8_block_scaled_grouped_amd/tuning/block_m_sweep.jsonl
    python -m fp8_block_scaled_grouped_amd.tuning.make_tables
    python -c "import __graft_entry__ as g; g.build()"

csrc/dense_tuned.h: per (N, K) and M range, the tiling (tile_m, tile_n, K splits) that
timed fastest, where it beat the rule's own plan (timed in the same sweep, so the table
does not depend on the table it replaces) by more than MARGIN; other M ranges keep
the rule.  tile_n 16 is the small-M kernel (K split inside the workgroup, no workspace).  A split is kept only while its fp32 partials fit the static scratch of the
allocation-free entry point, so that entry point runs every plan the table holds.

csrc/block_m_tuned.h: the M tile of the grouped GEMMs by mean token-expert pairs per
expert (T * topk / E): the fastest whole-layer time per swept token count.

Only sweep records are read (lines with a "sweep" key); the script is pure host code.
"""
import argparse
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "csrc")
MARGIN = 0.03
STATIC_SCRATCH_BYTES = 32 << 20  # MOE355_STATIC_SCRATCH_BYTES


def read(path, kind):
    out = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line.startswith("{"):
                continue
            r = json.loads(line)
            if r.get("sweep") == kind:
                out.append(r)
    return out


def kb_per_split(K, splits):
    KB = -(-K // 128)
    kbs = -(-KB // max(1, min(splits, KB)))
    return kbs, -(-KB // kbs)


def dense_rows(records):
    """[(m_min, m_max, n, k, bm, bnb, splits, us, default_us)] per record where a plan wins."""
    by_shape = {}
    for r in records:
        by_shape.setdefault((r["N"], r["K"]), []).append(r)
    rows = []
    for (N, K), rs in sorted(by_shape.items()):
        rs.sort(key=lambda r: r["M"])
        prev = 0
        for r in rs:
            M = r["M"]
            # plans whose split-K partials fit the static scratch (16-column tiles need none)
            ok = [p for p in r["plans"]
                  if p[1] == 16 or kb_per_split(K, p[2])[1] == 1
                  or kb_per_split(K, p[2])[1] * M * N * 4 + 256 <= STATIC_SCRATCH_BYTES]
            if ok:
                bm, bnb, sp, us = min(ok, key=lambda p: p[3])
                base = r["rule"][3] if "rule" in r else r["default_us"]  # the rule's plan, timed
                if us < (1.0 - MARGIN) * base:
                    rows.append((prev + 1, M, N, K, bm, bnb, sp, us, base))
            prev = M
    return rows


def write_dense(rows, src, out_dir=CSRC):
    lines = ["// Measured tilings of the dense FP8 block-scale GEMM per shape, written by",
             "// fp8_block_scaled_grouped_amd/tuning/make_tables.py from %s." % src,
             "// An entry serves m_min <= M <= m_max for its N and K; M outside every entry of",
             "// a shape takes the rule in dense_plan.  Timings (microseconds, this tiling vs the",
             "// rule's plan) are the sweep's.",
             "#pragma once", "", "namespace moe355 {", "", "struct DenseTuned {",
             "  int m_min, m_max, n, k;", "  int bm, bnb, splits;", "};", ""]
    if rows:
        lines.append("static const DenseTuned kDenseTuned[] = {")
        for m0, m1, n, k, bm, bnb, sp, us, dus in rows:
            lines.append("    {%d, %d, %d, %d, %d, %d, %d},  // %.1f vs %.1f" % (m0, m1, n, k, bm, bnb, sp, us, dus))
        lines.append("};")
    else:
        lines.append("static const DenseTuned kDenseTuned[] = {{1, 0, 0, 0, 16, 128, 1}};  // no entries")
    lines += ["", "}  // namespace moe355", ""]
    with open(os.path.join(out_dir, "dense_tuned.h"), "w") as f:
        f.write("\n".join(lines))


def block_m_rows(records):
    """[(pairs_per_expert_max, block_m, ms, {bm: ms})] in ascending pairs per expert."""
    by_t = {}
    for r in records:
        ppe = r["tokens"] * r["topk"] / r["experts"]
        by_t.setdefault(ppe, {})[r["block_m"]] = r["ms"]
    rows = []
    for ppe in sorted(by_t):
        times = by_t[ppe]
        bm = min(times, key=times.get)
        rows.append((ppe, bm, times[bm], times))
    # merge neighbours that pick the same tile
    merged = []
    for row in rows:
        if merged and merged[-1][1] == row[1]:
            merged[-1] = row
        else:
            merged.append(row)
    return merged


def write_block_m(rows, src, out_dir=CSRC):
    lines = ["// M tile of the grouped GEMMs by mean token-expert pairs per expert, written by",
             "// fp8_block_scaled_grouped_amd/tuning/make_tables.py from %s." % src,
             "// An entry serves T * topk / E <= ppe_max (the first such entry); above the last,",
             "// the last entry's tile.  Whole-layer milliseconds per swept tile in comments.",
             "#pragma once", "", "namespace moe355 {", "", "struct BlockMTuned {", "  double ppe_max;",
             "  int block_m;", "};", ""]
    if rows:
        lines.append("static const BlockMTuned kBlockMTuned[] = {")
        for ppe, bm, ms, times in rows:
            lines.append("    {%.6g, %d},  // %s" % (ppe, bm, " ".join("%d:%.3f" % (b, t) for b, t in sorted(times.items()))))
        lines.append("};")
    else:
        lines.append("static const BlockMTuned kBlockMTuned[] = {{0.0, 0}};  // no entries")
    lines += ["", "}  // namespace moe355", ""]
    with open(os.path.join(out_dir, "block_m_tuned.h"), "w") as f:
        f.write("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--dense", default=os.path.join(HERE, "dense_sweep.jsonl"))
    ap.add_argument("--block-m", default=os.path.join(HERE, "block_m_sweep.jsonl"))
    ap.add_argument("--out-dir", default=CSRC)
    a = ap.parse_args()
    if os.path.exists(a.dense):
        rows = dense_rows(read(a.dense, "dense"))
        write_dense(rows, os.path.basename(a.dense), a.out_dir)
        print("dense_tuned.h: %d entries" % len(rows))
    if os.path.exists(a.block_m):
        rows = block_m_rows(read(a.block_m, "block_m"))
        write_block_m(rows, os.path.basename(a.block_m), a.out_dir)
        print("block_m_tuned.h: %d entries" % len(rows))


if __name__ == "__main__":
    main()
