"""Summaries of rocprofv3 CSV output for the library's kernels.

    python -m weight_quantized_linear_qlinear_amd.profile_summary kernels TRACE.csv [--top N]
    python -m weight_quantized_linear_qlinear_amd.profile_summary family TRACE.csv REGEX
    python -m weight_quantized_linear_qlinear_amd.profile_summary mfma COUNTERS.csv AGENT_INFO.csv [--match RE]
    python -m weight_quantized_linear_qlinear_amd.profile_summary traffic FETCH.csv WRITE.csv [--match RE]
    python -m weight_quantized_linear_qlinear_amd.profile_summary counters PASS.csv [PASS.csv ...] [--match RE] [--brief]

`kernels` reads a `--kernel-trace` CSV and prints, per kernel and launch size
(workgroups), the call count and the duration's mean, p10, p50, p90, min and max;
`family` the same statistics over every dispatch whose kernel name matches REGEX.

`mfma` reads a `--pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE ...` CSV and prints per
kernel and launch size the MFMA utilisation: the matrix-pipe busy cycles over all
SIMDs divided by the SIMD count times the GPU-active cycles of one XCD
(GRBM_GUI_ACTIVE is summed over the XCDs), plus the MFMA FLOPs the MOPS counters
report when they were collected.

`counters` reads any number of `--pmc` CSVs (one pass each) and prints per kernel and
launch size each counter's mean per dispatch, plus the ratios whose counters are present:
the mean vector-memory instruction latency (VmemLatency, cycles), the mean L1->L2 read
latency (TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ, cycles), the L2 hit rate, the mean
L2->fabric read latency (TCC_EA0_RDREQ_LEVEL / TCC_EA0_RDREQ, cycles), the vector-memory
reads a wave keeps in flight on average (Little's law) and the L1 address translation miss
rate.

`traffic` reads one FETCH_SIZE and one WRITE_SIZE run (KiB per dispatch) and prints
per kernel and launch size the bytes between the L2s and the fabric (the 256 MB
last-level cache can serve them, so they are an upper bound on HBM bytes, not HBM
bytes), scaled by what the same counters read for the largest device-to-device
copy in the run (bytes known: it reads and writes its size).
"""
from __future__ import annotations

import argparse
import collections
import csv
import re
import sys

import numpy as np


def short_name(name: str) -> str:
    """qlq kernels without namespaces and argument lists; others truncated."""
    n = name.replace("void ", "").replace("qlq::(anonymous namespace)::", "").replace("qlq::", "")
    if "(" in n and n.index("(") > 0 and n.startswith(("gemm", "quant", "pack", "absmax", "finalize", "kv_", "zero",
                                                        "unpack", "clear")):
        n = n[:n.index("(")]
    return n if len(n) <= 110 else n[:107] + "..."


def _wgs(grid: int, wg: int) -> int:
    return grid // wg if wg else grid


def kernels(path: str, top: int):
    groups = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        key = (short_name(r["Kernel_Name"]), _wgs(int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"])),
               int(r["Workgroup_Size_X"]))
        groups[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in groups.values())
    rows = sorted(groups.items(), key=lambda kv: -sum(kv[1]))[:top]
    print("# kernel | workgroups x threads | calls | mean us | p10 | p50 | p90 | min | max | % of GPU time")
    for (name, wgs, wg), d in rows:
        a = np.array(d)
        print(f"{name} | {wgs} x {wg} | {a.size} | {a.mean():.2f} | {np.percentile(a, 10):.2f} | "
              f"{np.percentile(a, 50):.2f} | {np.percentile(a, 90):.2f} | {a.min():.2f} | {a.max():.2f} | "
              f"{100 * a.sum() / total:.2f}")


def family(path: str, match: str):
    """Duration statistics over every dispatch whose kernel name matches `match`."""
    rx = re.compile(match)
    d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in csv.DictReader(open(path))
         if rx.search(r["Kernel_Name"])]
    if not d:
        raise SystemExit(f"no dispatch matches {match!r}")
    a = np.array(d)
    print(f"family {match!r}: {a.size} dispatches, mean {a.mean():.2f} us, p10 {np.percentile(a, 10):.2f}, "
          f"p50 {np.percentile(a, 50):.2f}, p90 {np.percentile(a, 90):.2f}, min {a.min():.2f}, max {a.max():.2f}")
    print(f"family_mean_us: {a.mean():.3f}")


def _pivot(path: str, match: str | None):
    disp = collections.defaultdict(dict)
    rx = re.compile(match) if match else None
    for r in csv.DictReader(open(path)):
        if rx and not rx.search(r["Kernel_Name"]):
            continue
        d = disp[int(r["Dispatch_Id"])]
        d["name"] = r["Kernel_Name"]
        d["wgs"] = _wgs(int(r["Grid_Size"]), int(r["Workgroup_Size"]))
        d["wg"] = int(r["Workgroup_Size"])
        d["us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    return disp


def _gpu_agent(path: str):
    for r in csv.DictReader(open(path)):
        if r.get("Agent_Type") == "GPU":
            return int(r["Simd_Count"]), int(r["Num_Xcc"])
    raise SystemExit("no GPU agent in " + path)


def mfma(path: str, agent_path: str, match: str | None):
    simds, xcc = _gpu_agent(agent_path)
    groups = collections.defaultdict(list)
    for d in _pivot(path, match).values():
        if "SQ_VALU_MFMA_BUSY_CYCLES" not in d or not d.get("GRBM_GUI_ACTIVE"):
            continue
        util = d["SQ_VALU_MFMA_BUSY_CYCLES"] / (simds * d["GRBM_GUI_ACTIVE"] / xcc)
        flops = 512 * sum(d.get(c, 0.0) for c in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F8",
                                                   "SQ_INSTS_VALU_MFMA_MOPS_I8", "SQ_INSTS_VALU_MFMA_MOPS_F16"))
        groups[(short_name(d["name"]), d["wgs"], d["wg"])].append((util, flops, d["us"]))
    print(f"# {simds} SIMDs, {xcc} XCDs; MFMA utilisation = SQ_VALU_MFMA_BUSY_CYCLES / "
          f"({simds} x GRBM_GUI_ACTIVE / {xcc})")
    print("# kernel | workgroups x threads | dispatches | MFMA util % (mean) | min | max | MFMA GFLOP per dispatch | "
          "us per dispatch (under the profiler)")
    for (name, wgs, wg), v in sorted(groups.items(), key=lambda kv: -sum(x[2] for x in kv[1])):
        a = np.array(v)
        print(f"{name} | {wgs} x {wg} | {len(v)} | {100 * a[:, 0].mean():.1f} | {100 * a[:, 0].min():.1f} | "
              f"{100 * a[:, 0].max():.1f} | {a[:, 1].mean() / 1e9:.3f} | {a[:, 2].mean():.2f}")


def traffic(fetch_path: str, write_path: str, match: str | None):
    fetch = _pivot(fetch_path, None)
    write = _pivot(write_path, None)

    def calib(disp, counter):
        cp = [d for d in disp.values() if "copyBuffer" in d["name"] or "copy" in d["name"].lower()]
        if not cp:
            raise SystemExit("no copy dispatch to calibrate against (run with the copy calibration)")
        return max(cp, key=lambda d: d.get(counter, 0.0))

    cf, cw = calib(fetch, "FETCH_SIZE"), calib(write, "WRITE_SIZE")
    copy_bytes = 256 << 20
    kf = copy_bytes / (cf["FETCH_SIZE"] * 1024)
    kw = copy_bytes / (cw["WRITE_SIZE"] * 1024)
    print(f"# calibration: a {copy_bytes >> 20} MiB device copy reads FETCH_SIZE {cf['FETCH_SIZE']:.0f} KiB and "
          f"WRITE_SIZE {cw['WRITE_SIZE']:.0f} KiB: factors {kf:.3f} (fetch), {kw:.3f} (write)")
    rx = re.compile(match) if match else None
    groups = collections.defaultdict(lambda: [[], []])
    for d in fetch.values():
        if rx and not rx.search(d["name"]):
            continue
        groups[(short_name(d["name"]), d["wgs"], d["wg"])][0].append(d["FETCH_SIZE"] * 1024 * kf)
    for d in write.values():
        if rx and not rx.search(d["name"]):
            continue
        groups[(short_name(d["name"]), d["wgs"], d["wg"])][1].append(d["WRITE_SIZE"] * 1024 * kw)
    print("# kernel | workgroups x threads | dispatches | fetched MB per dispatch | written MB per dispatch | "
          "L2<->fabric MB per dispatch")
    tot_f = tot_w = n_all = 0
    for (name, wgs, wg), (f, w) in sorted(groups.items(), key=lambda kv: -sum(kv[1][0])):
        if not f or not w:
            continue
        mf, mw = float(np.mean(f)), float(np.mean(w))
        tot_f += sum(f)
        tot_w += sum(w)
        n_all += len(f)
        print(f"{name} | {wgs} x {wg} | {len(f)} | {mf / 1e6:.2f} | {mw / 1e6:.2f} | {(mf + mw) / 1e6:.2f}")
    if n_all:
        print(f"fabric_bytes_per_launch: {(tot_f + tot_w) / n_all:.0f}")
        print(f"dispatches: {n_all}")


_RATIOS = [
    ("vmem latency (cycles)", lambda c: c.get("VmemLatency")),
    ("L1->L2 read latency (cycles)", lambda c: c["TCP_TCC_READ_REQ_LATENCY_sum"] / c["TCP_TCC_READ_REQ_sum"]
     if c.get("TCP_TCC_READ_REQ_sum") else None),
    ("L2 hit %", lambda c: 100 * c["TCC_HIT_sum"] / (c["TCC_HIT_sum"] + c["TCC_MISS_sum"])
     if c.get("TCC_HIT_sum", 0) + c.get("TCC_MISS_sum", 0) > 0 else None),
    ("L2->fabric read latency (cycles)", lambda c: c["TCC_EA0_RDREQ_LEVEL_sum"] / c["TCC_EA0_RDREQ_sum"]
     if c.get("TCC_EA0_RDREQ_sum") else None),
    # Little's law: read instructions per wave x their mean latency / the dispatch's cycles
    # (its duration at 2.4 GHz; GRBM_GUI_ACTIVE also counts the profiler's window around
    # short dispatches)
    ("vmem reads in flight per wave", lambda c: c["VmemLatency"] * c["SQ_INSTS_VMEM_RD"] / c["SQ_WAVES"] /
     (c["_us"] * 2400.0) if c.get("VmemLatency") and c.get("SQ_WAVES") else None),
    ("L1 translation miss %", lambda c: 100 * c["TCP_UTCL1_TRANSLATION_MISS_sum"] /
     (c["TCP_UTCL1_TRANSLATION_MISS_sum"] + c["TCP_UTCL1_TRANSLATION_HIT_sum"])
     if c.get("TCP_UTCL1_TRANSLATION_MISS_sum", 0) + c.get("TCP_UTCL1_TRANSLATION_HIT_sum", 0) > 0 else None),
]


def counters(paths, match: str | None, brief: bool = False):
    """Per kernel and launch size: mean of every counter per dispatch over all passes,
    and the ratios above (each pass is a separate run of the same program, so a kernel's
    dispatches line up by their order within the kernel and launch size)."""
    groups = collections.defaultdict(lambda: collections.defaultdict(list))
    us = collections.defaultdict(list)
    for path in paths:
        for d in _pivot(path, match).values():
            key = (short_name(d["name"]), d["wgs"], d["wg"])
            for k, v in d.items():
                if k not in ("name", "wgs", "wg", "us"):
                    groups[key][k].append(v)
            us[key].append(d["us"])
    print("# kernel | workgroups x threads | dispatches (all passes) | us per dispatch (under the profiler) | "
          "ratios | counter means per dispatch")
    for key, cs in sorted(groups.items(), key=lambda kv: -sum(us[kv[0]])):
        mean = {k: float(np.mean(v)) for k, v in cs.items()}
        mean["_us"] = float(np.mean(us[key]))
        ratios = []
        for label, f in _RATIOS:
            try:
                r = f(mean)
            except (KeyError, ZeroDivisionError):
                r = None
            if r is not None:
                ratios.append(f"{label} {r:.1f}")
        keep = ("MeanOccupancyPerCU", "SQ_WAVES", "SQ_INSTS_VMEM_RD")
        raw = ", ".join(f"{k} {v:.4g}" for k, v in sorted(mean.items())
                        if not k.startswith("_") and (not brief or k in keep))
        name, wgs, wg = key
        print(f"{name} | {wgs} x {wg} | {len(us[key])} | {np.mean(us[key]):.2f} | {'; '.join(ratios)} | {raw}")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("trace")
    k.add_argument("--top", type=int, default=40)
    f = sub.add_parser("family")
    f.add_argument("trace")
    f.add_argument("match")
    m = sub.add_parser("mfma")
    m.add_argument("counters")
    m.add_argument("agent_info")
    m.add_argument("--match")
    c = sub.add_parser("counters")
    c.add_argument("passes", nargs="+")
    c.add_argument("--match")
    c.add_argument("--brief", action="store_true", help="ratios, occupancy, waves and read instructions only")
    t = sub.add_parser("traffic")
    t.add_argument("fetch")
    t.add_argument("write")
    t.add_argument("--match")
    a = ap.parse_args(argv)
    if a.cmd == "kernels":
        kernels(a.trace, a.top)
    elif a.cmd == "family":
        family(a.trace, a.match)
    elif a.cmd == "mfma":
        mfma(a.counters, a.agent_info, a.match)
    elif a.cmd == "counters":
        counters(a.passes, a.match, a.brief)
    else:
        traffic(a.fetch, a.write, a.match)


if __name__ == "__main__":
    sys.exit(main())
