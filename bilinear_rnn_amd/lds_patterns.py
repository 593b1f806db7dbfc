"""LDS access patterns of the chunk forward, replayed one at a time through
``comba_lds_probe`` so that a profiler's bank-conflict counters can be read
for each.

The address functions below restate the kernel's LDS layouts (q / k tiles,
packed T / P tiles, fp32 scratch blocks, staging rows) for the 64 lanes of
one wavefront instruction; alternative swizzles of the q / k tiles are
listed beside the kernel's for comparison. Run under rocprofv3, one pass
(REPO: the repository root):

    PYTHONPATH=REPO rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS SQ_WAVES \\
        --output-format csv -d OUT -o p -- python3 -m bilinear_rnn_amd.lds_patterns
    python3 -m bilinear_rnn_amd.lds_patterns --summarize OUT

The first command launches every pattern once (in the order of
``patterns()``); the second reads the counters back by dispatch order and
prints one line per pattern family: conflict cycles over LDS-active cycles,
and LDS-active cycles per wavefront instruction.
"""
import argparse
import collections
import csv
import glob
import os

KSS = 20  # row stride, in floats, of the fp32 16x16 scratch blocks


def perm32(p):
    return 8 * (p >> 2) + (p & 3) if p < 16 else 8 * ((p - 16) >> 2) + 4 + (p & 3)


def perm_col(c):
    return (c & ~31) | perm32(c & 31)


def qk_swizzle(K, row):
    """The kernel's q / k tile swizzle (16-byte chunk index XOR)."""
    return ((row & 3) << 1) ^ (9 * ((row >> 2) & 1)) if K == 128 else row & 7


QK_ALTERNATIVES = {
    "kernel": qk_swizzle,
    "plain (row mod chunks)": lambda K, r: r & (K // 8 - 1),
    "row bits 0, 1, 2 -> chunk bits {2}, {0, 1}, {1, 2} (K=64)": lambda K, r: (
        (((r & 3) << 1) ^ (9 * ((r >> 2) & 1))) if K == 128
        else (4 * ((r >> 1) & 1)) ^ (3 * ((r >> 2) & 1)) ^ (6 * ((r >> 3) & 1))),
    "row bits 0-1 up, 2-3 down": lambda K, r: (((r & 3) << 2) | ((r >> 2) & 3)) if K == 128
    else ((((r >> 1) & 1) << 2) | ((r >> 2) & 3)),
}


def qk_off(K, sw, row, pos):
    return row * K + (((pos >> 3) ^ sw(K, row)) << 3) + (pos & 7)


def tp_off(row, pos):
    big = row >> 5
    base = row * (32 << big) - 1024 * big
    s = ((row >> 1) & 7) if big else ((row >> 2) & 3)
    return base + (((pos >> 3) ^ s) << 3) + (pos & 7)


def qk_row(K, ptid, j, spread=True):
    """Row of producer thread ptid's q / k staging piece j (four producer
    waves); spread: the K=128 map of the instantiations without in-kernel
    normalisation (two rows per 16-lane group)."""
    if K == 128 and spread:
        return 16 * j + ((ptid >> 6) & 1) + (((ptid >> 5) & 1) << 1) + (((ptid >> 3) & 1) << 2) + ((ptid >> 7) << 3)
    if K == 128:
        return 16 * j + 4 * ((ptid >> 4) & 3) + (ptid >> 6)
    ph, grp = ptid >> 5, (ptid >> 3) & 3
    return 32 * j + (ph & 1) * 2 + (ph >> 1) * 8 + (grp & 1) + 4 * (grp >> 1)


def qk_col(K, ptid, spread=True):
    """Column (16-byte piece) of producer thread ptid's q / k pieces."""
    if K == 128 and spread:
        return (ptid & 7) | (((ptid >> 4) & 1) << 3)
    return ptid % (K // 8)


def _g(lane):
    return lane >> 4


def _l16(lane):
    return lane & 15


def patterns():
    """(family, kind, 64 byte offsets) for every access pattern measured."""
    out = []
    for K in (128, 64):
        for name, sw in QK_ALTERNATIVES.items():
            fam = f"q/k tile K={K} [{name}]"
            for r4 in range(4):
                for s in range(K // 32):
                    out.append((f"{fam}: row fragment (16-byte read)", "read16",
                                [2 * qk_off(K, sw, 16 * r4 + _l16(l), 32 * s + 8 * _g(l)) for l in range(64)]))
            for kb in range(K // 16):
                for s2 in range(2):
                    for hi in range(2):
                        out.append((f"{fam}: K^T transposed read", "read8_tr",
                                    [2 * qk_off(K, sw, 32 * s2 + 16 * hi + 4 * _g(l) + (_l16(l) >> 2),
                                                perm_col(16 * kb + 4 * (_l16(l) & 3))) for l in range(64)]))
            kp = K // 8
            for spread in ((True, False) if K == 128 else (True,)):
                tag = "" if K == 64 else (" (rows spread)" if spread else " (one row per 16 lanes, normalising form)")
                for w in range(4):
                    for j in range(64 * kp // 256):
                        for half in (0, 4):
                            out.append((f"{fam}: staging write (8-byte){tag}", "write8",
                                        [2 * qk_off(K, sw, qk_row(K, w * 64 + l, j, spread),
                                                    perm_col(qk_col(K, w * 64 + l, spread) * 8 + half))
                                         for l in range(64)]))
    for r4 in range(2):
        out.append(("T/P tile rows 0-31: fragment", "read16", [2 * tp_off(16 * r4 + _l16(l), 8 * _g(l)) for l in range(64)]))
    for r in range(2):
        for c0 in (0, 32):
            out.append(("T/P tile rows 32-63: fragment", "read16",
                        [2 * tp_off(32 + 16 * r + _l16(l), c0 + 8 * _g(l)) for l in range(64)]))
    for R, C in [(0, 0), (1, 0), (1, 1), (2, 0), (2, 1), (2, 2), (3, 0), (3, 1), (3, 2), (3, 3)]:
        out.append(("T/P tile: producers' 8-byte block writes", "write8",
                    [2 * tp_off(16 * R + _l16(l), perm_col(16 * C + 4 * _g(l))) for l in range(64)]))
    out.append(("fp32 scratch: 16-byte row write", "write16", [4 * (_l16(l) * KSS + 4 * _g(l)) for l in range(64)]))
    out.append(("fp32 scratch: 16-byte row read", "read16", [4 * (_l16(l) * KSS + 4 * _g(l)) for l in range(64)]))
    for j in range(4):
        out.append(("fp32 scratch: column read", "read4", [4 * ((4 * _g(l) + j) * KSS + _l16(l)) for l in range(64)]))
    for r in range(4):
        for j4 in range(4):
            out.append(("fp32 scratch: inverse's broadcast row read", "read16",
                        [4 * ((4 * (l & 3) + r) * KSS + 4 * j4) for l in range(64)]))
    return out


def run(iters=2048):
    import torch
    from . import api
    dev = torch.device("cuda:0")
    sink = torch.empty(256 * 256, dtype=torch.int32, device=dev)
    for fam, kind, offs in patterns():
        api.lds_probe(kind, offs, iters, sink)
    torch.cuda.synchronize()


def summarize(pmc_dir):
    rows = []
    for path in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        rows += list(csv.DictReader(open(path)))
    by = collections.defaultdict(dict)
    for r in rows:
        if "lds_probe_kernel" in r["Kernel_Name"]:
            by[int(r["Dispatch_Id"])][r["Counter_Name"]] = float(r["Counter_Value"])
    pats = patterns()
    ids = sorted(by)
    if len(ids) != len(pats):
        raise SystemExit(f"{len(ids)} probe dispatches counted, {len(pats)} patterns expected")
    fam = collections.OrderedDict()
    for i, (name, kind, _) in zip(ids, pats):
        v = by[i]
        fam.setdefault((name, kind), []).append(
            (v["SQ_LDS_BANK_CONFLICT"] / max(v["SQ_LDS_IDX_ACTIVE"], 1.0), v["SQ_LDS_IDX_ACTIVE"] / max(v["SQ_INSTS_LDS"], 1.0)))
    lines = ["| Pattern | Access | Cases | Conflict / active cycles (mean, max) | Active cycles per wave instruction |",
             "|---|---|---|---|---|"]
    for (name, kind), vals in fam.items():
        c = [x for x, _ in vals]
        a = [y for _, y in vals]
        lines.append(f"| {name} | {kind} | {len(vals)} | {sum(c) / len(c):.2f}, {max(c):.2f} | {sum(a) / len(a):.2f} |")
    print("\n".join(lines))


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--summarize", metavar="PMC_DIR")
    ap.add_argument("--iters", type=int, default=2048)
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize)
    else:
        run(args.iters)
