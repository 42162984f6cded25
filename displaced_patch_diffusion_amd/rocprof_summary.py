"""Text summaries of rocprofv3 output, for the profiles kept with the library.

Three summaries, each from the CSV files one or more rocprofv3 runs wrote:

``trace``
    kernel statistics of any run (``--kernel-trace``): calls, average, min and
    max duration per kernel and per launch shape.
``ops-trace``
    durations per op of a ``bench.py --profile-ops R`` run, whose dispatch
    records split into one segment per op at the spin kernels the run puts
    between the ops (the run prints the segment labels on a ``PROFILE_OPS``
    line).
``ops-counters``
    hardware counters per op of ``--profile-ops`` runs under ``--pmc`` (one
    run per counter pass), per call of the op: MFMA busy and VALU busy shares,
    LDS and any-wait shares of wave time, MFMA bf16 flops, and the bytes the
    L2 exchanged with the memory fabric (32/64/128-byte read requests and
    32/64-byte write requests), checked against the plain copy of known size
    that closes every ``--profile-ops`` run.

Every summary states the commands that made it and the SHA-256 of the library
sources it was taken on; a ``RESULT`` line closes it with the figures as JSON.

Usage::

    python -m displaced_patch_diffusion_amd.rocprof_summary trace DIR --label L --cmd CMD --out FILE
    python -m displaced_patch_diffusion_amd.rocprof_summary ops-trace DIR --log LOG --cmd CMD --out FILE
    python -m displaced_patch_diffusion_amd.rocprof_summary ops-counters DIR [DIR ...] --log LOG \\
        --cmd CMD [--cmd CMD ...] --out FILE
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import json
import os

from .build import source_digest

SPIN = "spin_kernel"
FLUSH = "FillFunctor"
N_CU = 256
N_SIMD = 4 * N_CU
N_XCC = 8
PEAK_CLOCK_MHZ = 2400.0

# counter passes of an ops-counters summary (at most 8 SQ, 4 TCC, 2 GRBM each)
PASSES = {
    "sq": ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
           "SQ_ACTIVE_INST_VALU", "SQ_WAIT_INST_LDS", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE"],
    "rd": ["TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum", "TCC_EA0_RDREQ_sum"],
    "wr": ["TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "TCC_EA0_RDREQ_DRAM_sum", "TCC_EA0_WRREQ_DRAM_sum"],
    "lds": ["SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS_LOAD_BANDWIDTH", "SQ_INSTS_LDS_STORE_BANDWIDTH",
            "GRBM_GUI_ACTIVE"],
}


def _rows(d: str, suffix: str) -> list[dict]:
    out = []
    for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(f) as fh:
            out += list(csv.DictReader(fh))
    if not out:
        raise SystemExit(f"no *{suffix} under {d}")
    return out


def short(name: str) -> str:
    """A kernel's name without its parameter list and anonymous namespaces."""
    n = name.replace("(anonymous namespace)::", "")
    if n.startswith("void "):
        n = n[5:]
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and i > 0:
            return n[:i].strip()
    return n.strip()


def _profile_line(log: str) -> dict:
    rec = None
    with open(log) as f:
        for line in f:
            if line.startswith("PROFILE_OPS "):
                rec = json.loads(line[len("PROFILE_OPS "):])
    if rec is None:
        raise SystemExit(f"no PROFILE_OPS line in {log}")
    return rec


def segments(dispatches: list, labels: list[str]) -> dict:
    """Split dispatch records (sorted by dispatch id; each has a "name") at the
    spin kernels: the last len(labels)+1 spins bound one segment per label."""
    spins = [i for i, d in enumerate(dispatches) if SPIN in d["name"]]
    if len(spins) < len(labels) + 1:
        raise SystemExit(f"{len(spins)} spin kernels for {len(labels)} ops")
    spins = spins[-(len(labels) + 1):]
    return {lab: dispatches[spins[i] + 1:spins[i + 1]] for i, lab in enumerate(labels)}


def _header(title: str, cmds: list[str]) -> list[str]:
    dig = source_digest()
    L = [f"# {title}"]
    L += [f"# command: {c}" for c in cmds]
    L.append("# library sources (sha256): " + ", ".join(f"{k} {v[:16]}" for k, v in dig.items()))
    return L


# ------------------------------------------------------------------- traces
def _trace_dispatches(d: str) -> list[dict]:
    out = []
    for r in _rows(d, "kernel_trace.csv"):
        out.append({"id": int(r["Dispatch_Id"]), "name": r["Kernel_Name"],
                    "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3,
                    "grid": (int(r["Grid_Size_X"]), int(r.get("Grid_Size_Y") or 1), int(r.get("Grid_Size_Z") or 1)),
                    "vgpr": int(r.get("VGPR_Count") or 0), "lds": int(r.get("LDS_Block_Size") or 0)})
    out.sort(key=lambda x: x["id"])
    return out


def trace(d: str, label: str, cmd: str, attn: str = "attn_bf16_d64", last: int = 20) -> str:
    ds = _trace_dispatches(d)
    by, shapes = collections.OrderedDict(), collections.OrderedDict()
    for x in ds:
        n = short(x["name"])
        by.setdefault(n, []).append(x["us"])
        shapes.setdefault((n, x["grid"]), []).append(x["us"])
    tot = sum(sum(v) for v in by.values())
    L = _header(f"rocprofv3 kernel statistics, {label}", [cmd])
    L += ["#", f"# {'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}"]
    for n, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        L.append(f"  {n[:60]:60s} {len(v):6d} {sum(v) / len(v):10.2f} {min(v):10.2f} {max(v):10.2f} "
                 f"{100 * sum(v) / tot:6.2f}")
    L += ["#", f"# per launch shape (grid in work-items); last_avg_us = mean of the last {last} launches of "
               "that shape"]
    for (n, g), v in sorted(shapes.items(), key=lambda kv: -sum(kv[1])):
        tail = v[-last:]
        L.append(f"  {n[:56]:56s} grid={g} n={len(v)} avg_us={sum(v) / len(v):.2f} "
                 f"last_avg_us={sum(tail) / len(tail):.2f}")
    at = [x["us"] for x in ds if attn in x["name"]]
    res = {"label": label}
    if at:
        tail = at[-last:]
        res[f"{attn}_last_avg_us"] = round(sum(tail) / len(tail), 2)
        L += ["#", f"# {attn}, last {len(tail)} launches: avg_us={sum(tail) / len(tail):.2f} "
                   f"min_us={min(tail):.2f} max_us={max(tail):.2f}"]
    L.append("RESULT " + json.dumps(res))
    return "\n".join(L) + "\n"


def ops_trace(d: str, log: str, cmd: str) -> str:
    rec = _profile_line(log)
    reps, labels = rec["reps"], rec["labels"]
    ds = _trace_dispatches(d)
    if rec.get("flush"):
        ds = [x for x in ds if FLUSH not in x["name"]]
    seg = segments(ds, labels)
    how = "after a 1 GiB cache flush each (the flush kernels left out)" if rec.get("flush") else "in a row"
    L = _header(f"per-op kernel durations, workload {rec['workload']} (qkv {rec['qkv']}, gn_sums "
                f"{rec['gn_sums']}), each op launched {reps} times {how}", [cmd])
    L += ["#", f"# {'op':12s} {'kernels/call':>12s} {'us/call':>10s} {'min_us':>10s}  "
               "kernels (grid, vgpr, lds bytes, avg us)"]
    res = {"workload": rec["workload"], "reps": reps, "ops": {}}
    for lab in labels:
        xs = seg[lab]
        per = len(xs) // reps
        tot = sum(x["us"] for x in xs) / reps
        calls = [sum(x["us"] for x in xs[i * per:(i + 1) * per]) for i in range(reps)] if per else [0.0]
        kinds = collections.OrderedDict()
        for x in xs:
            kinds.setdefault((short(x["name"]), x["grid"], x["vgpr"], x["lds"]), []).append(x["us"])
        desc = "; ".join(f"{n} {g} v{v} l{l} {sum(t) / len(t):.2f}" for (n, g, v, l), t in kinds.items())
        L.append(f"  {lab:12s} {per:12d} {tot:10.2f} {min(calls):10.2f}  {desc}")
        res["ops"][lab] = {"kernels_per_call": per, "us_per_call": round(tot, 2), "min_us": round(min(calls), 2)}
    L.append("RESULT " + json.dumps(res))
    return "\n".join(L) + "\n"


# ----------------------------------------------------------------- counters
def _counter_dispatches(d: str) -> list[dict]:
    acc = collections.OrderedDict()
    for r in _rows(d, "counter_collection.csv"):
        k = int(r["Dispatch_Id"])
        x = acc.setdefault(k, {"id": k, "name": r["Kernel_Name"], "c": collections.defaultdict(float)})
        x["c"][r["Counter_Name"]] += float(r["Counter_Value"])
    return sorted(acc.values(), key=lambda x: x["id"])


def _derive(c: dict, n_calls: int) -> dict:
    """Per-call figures from counters summed over an op's dispatches."""
    out = {}
    per = {k: v / n_calls for k, v in c.items()}
    if "GRBM_GUI_ACTIVE" in per:
        # summed over the XCDs' GRBM instances: one XCD's figure is the clock count
        cyc = per["GRBM_GUI_ACTIVE"] / N_XCC
        out["gui_cycles"] = round(cyc)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in per and cyc:
            out["mfma_busy_pct"] = round(100 * per["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * N_SIMD), 2)
        if "SQ_ACTIVE_INST_VALU" in per and cyc:
            out["valu_busy_pct"] = round(100 * per["SQ_ACTIVE_INST_VALU"] / (cyc * N_CU), 2)
        if "SQ_BUSY_CU_CYCLES" in per and cyc:
            out["cu_busy_pct"] = round(100 * 4 * per["SQ_BUSY_CU_CYCLES"] / (cyc * N_CU), 2)
    if "SQ_WAVE_CYCLES" in per and per["SQ_WAVE_CYCLES"]:
        wc = per["SQ_WAVE_CYCLES"]
        for k, name in (("SQ_WAIT_INST_LDS", "lds_wait_pct_of_wave"), ("SQ_WAIT_ANY", "any_wait_pct_of_wave"),
                        ("SQ_ACTIVE_INST_VALU", "valu_pct_of_wave")):
            if k in per:
                out[name] = round(100 * per[k] / wc, 2)
        if "SQ_LDS_IDX_ACTIVE" in per and cyc:
            out["lds_active_pct"] = round(100 * per["SQ_LDS_IDX_ACTIVE"] / (cyc * N_CU), 2)
        if "SQ_LDS_BANK_CONFLICT" in per and cyc:
            out["lds_bank_conflict_pct"] = round(100 * per["SQ_LDS_BANK_CONFLICT"] / (cyc * N_CU), 2)
    for k, name in (("SQ_INSTS_LDS_LOAD_BANDWIDTH", "lds_read_bytes"), ("SQ_INSTS_LDS_STORE_BANDWIDTH", "lds_write_bytes")):
        if k in per:
            out[name] = per[k] * 64
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in per:
        out["mfma_bf16_flop"] = per["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
    if "TCC_EA0_RDREQ_sum" in per:
        n32, n64, n128 = (per.get(f"TCC_EA0_RDREQ_{s}B_sum", 0.0) for s in (32, 64, 128))
        out["read_bytes"] = 32 * n32 + 64 * n64 + 128 * n128
        out["read_req_unclassified"] = per["TCC_EA0_RDREQ_sum"] - n32 - n64 - n128
    if "TCC_EA0_WRREQ_sum" in per:
        w64 = per.get("TCC_EA0_WRREQ_64B_sum", 0.0)
        out["write_bytes"] = 64 * w64 + 32 * (per["TCC_EA0_WRREQ_sum"] - w64)
        if "TCC_EA0_WRREQ_DRAM_sum" in per and per["TCC_EA0_WRREQ_sum"]:
            out["write_dram_share"] = round(per["TCC_EA0_WRREQ_DRAM_sum"] / per["TCC_EA0_WRREQ_sum"], 4)
    if "TCC_EA0_RDREQ_DRAM_sum" in per and "read_bytes" in out:
        out["read_dram_requests"] = per["TCC_EA0_RDREQ_DRAM_sum"]
    out["raw_per_call"] = {k: round(v, 1) for k, v in per.items()}
    return out


def ops_counters(dirs: list[str], log: str, cmds: list[str], durations: str | None = None) -> str:
    """Counters per op call.  `durations` names an ops-trace summary of the
    same workload: with it, MFMA busy is also given as a share of the traced
    kernel time at the 2.4 GHz peak clock, the basis of the peak flop rate."""
    rec = _profile_line(log)
    reps, labels = rec["reps"], rec["labels"]
    # per pass, each op's counters summed over its dispatches; a counter that
    # more than one pass collected (the clock) is averaged over those passes
    sums = {lab: {} for lab in labels}
    seen = {lab: collections.Counter() for lab in labels}
    for d in dirs:
        seg = segments(_counter_dispatches(d), labels)
        for lab in labels:
            acc = collections.defaultdict(float)
            for x in seg[lab]:
                for k, v in x["c"].items():
                    acc[k] += v
            for k, v in acc.items():
                n = seen[lab][k]
                sums[lab][k] = (sums[lab].get(k, 0.0) * n + v) / (n + 1)
                seen[lab][k] = n + 1
    res = {"workload": rec["workload"], "reps": reps, "sources_sha256": source_digest(), "ops": {}}
    dur = (read_result(durations) or {}).get("ops", {}) if durations else {}
    for lab in labels:
        o = res["ops"][lab] = _derive(sums[lab], reps)
        us = dur.get(lab, {}).get("us_per_call")
        if us and "SQ_VALU_MFMA_BUSY_CYCLES" in o["raw_per_call"]:
            o["traced_us"] = us
            o["mfma_busy_pct_at_peak_clock"] = round(
                100 * o["raw_per_call"]["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMD / (us * PEAK_CLOCK_MHZ), 2)
    cal = res["ops"].get("splice_copy", {})
    sb = rec["splice_bytes"]
    L = _header(f"hardware counters per op call, workload {rec['workload']} (qkv {rec['qkv']}, gn_sums "
                f"{rec['gn_sums']}), each op launched {reps} times in a row", cmds)
    L += ["# mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (clock cycles x 1024 SIMDs); clock cycles = GRBM_GUI_ACTIVE / 8 XCDs",
          "# valu_busy = SQ_ACTIVE_INST_VALU / (clock cycles x 256 CUs); waits as shares of SQ_WAVE_CYCLES",
          "# mfma bf16 flop = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512",
          "# read bytes = 32 x RDREQ_32B + 64 x RDREQ_64B + 128 x RDREQ_128B; write bytes = 64 x WRREQ_64B + "
          "32 x (WRREQ - WRREQ_64B) (L2 <-> fabric; last-level cache hits included)",
          "# lds active / bank conflict = SQ_LDS_IDX_ACTIVE / SQ_LDS_BANK_CONFLICT over (clock cycles x 256 CUs); "
          "LDS bytes = SQ_INSTS_LDS_{LOAD,STORE}_BANDWIDTH x 64; a counter two passes took is averaged"]
    if "read_bytes" in cal or "write_bytes" in cal:
        half = sb / 2
        L.append(f"# calibration: splice_copy reads {half:.0f} bytes and writes {half:.0f} bytes per call; "
                 f"counted read {cal.get('read_bytes', 0) / half:.4f}x, write {cal.get('write_bytes', 0) / half:.4f}x "
                 "of that")
    L.append("# gui cycles include the counter set-up around each dispatch: busy shares of short kernels "
             "are underestimates")
    if dur:
        L.append(f"# mfma@2.4 = SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (traced us x 2400 MHz); traced durations "
                 f"from {os.path.basename(durations)}")
    L += ["#", f"# {'op':12s} {'mfma%':>7s} {'mfma@2.4':>8s} {'valu%':>7s} {'ldsw%':>7s} {'wait%':>7s} {'GFLOP':>9s} "
               f"{'read MB':>9s} {'write MB':>9s} {'cycles':>9s} {'lds%':>6s} {'ldsMB':>8s}"]
    for lab in labels:
        o = res["ops"][lab]

        def f(k, scale=1.0, fmt="7.2f"):
            return format(o[k] * scale, fmt) if k in o else " " * int(fmt.split(".")[0])
        L.append(f"  {lab:12s} {f('mfma_busy_pct')} {f('mfma_busy_pct_at_peak_clock', 1, '8.2f')} {f('valu_busy_pct')} {f('lds_wait_pct_of_wave')} "
                 f"{f('any_wait_pct_of_wave')} {f('mfma_bf16_flop', 1e-9, '9.2f')} {f('read_bytes', 1e-6, '9.2f')} "
                 f"{f('write_bytes', 1e-6, '9.2f')} {f('gui_cycles', 1, '9.0f')} {f('lds_active_pct', 1, '6.1f')} "
                 f"{f('lds_read_bytes', 1e-6, '8.0f')}")
    L.append("RESULT " + json.dumps(res))
    return "\n".join(L) + "\n"


def read_result(path: str) -> dict | None:
    """The RESULT record of a summary file, or None."""
    rec = None
    try:
        with open(path) as f:
            for line in f:
                if line.startswith("RESULT "):
                    rec = json.loads(line[len("RESULT "):])
    except (OSError, ValueError):
        return None
    return rec


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("mode", choices=("trace", "ops-trace", "ops-counters"))
    ap.add_argument("dirs", nargs="+")
    ap.add_argument("--log")
    ap.add_argument("--label", default="")
    ap.add_argument("--cmd", action="append", default=[])
    ap.add_argument("--durations", help="ops-counters: an ops-trace summary of the same workload")
    ap.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.mode == "trace":
        text = trace(a.dirs[0], a.label, a.cmd[0] if a.cmd else "")
    elif a.mode == "ops-trace":
        text = ops_trace(a.dirs[0], a.log, a.cmd[0] if a.cmd else "")
    else:
        text = ops_counters(a.dirs, a.log, a.cmd, a.durations)
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


if __name__ == "__main__":
    main()
