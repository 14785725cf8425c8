"""Summaries of rocprofv3 runs of bench.py, written under profiles/ (text tables) and
profiles/traffic.json (the HBM bytes per launch that bench.py reports as `traffic`).

Inputs are the CSV files rocprofv3 writes for these commands (run from /tmp on the GPU machine, the
output directories under gpurun_out/):

  rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/prof_bench -o bench -- \
      python3 -u /root/repo/bench.py --steps 5 --warmup 2 --no-cpu-baseline
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/pmc_fetch -o f -- \
      python3 -u /root/repo/bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-graph --extras mlp
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/pmc_write -o w -- \
      python3 -u /root/repo/bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-graph --extras mlp
  rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/pmc_copyf -o cf -- \
      python3 -u /root/repo/bench.py --copy-calibration 256
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/pmc_copyw -o cw -- \
      python3 -u /root/repo/bench.py --copy-calibration 256
  rocprofv3 --pmc MfmaUtil --output-format csv -d <dir>/pmc_mfma -o m -- \
      python3 -u /root/repo/bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-graph \
      --extras mlp,attention,backward

Usage: python bench_profiles.py <dir>   (the directory holding the six output folders)

Dispatches of the shrink+expand sweep are named after their workload (shrink_tok<T>,
expand_tok<T>, and pair_tok<T> for the single launch of lora_shrink_expand): the two passes that
open each benchmark run (lora_shrink and lora_expand per token count, in order, then one
lora_shrink_expand per token count) fix which kernel and grid each workload launches; every
later dispatch with the same kernel and grid gets that name (several names when two workloads
launch the same kernel and grid). Dispatches after the sweep belong to the objects timed after it (fused MLP, attention
projections, backward, embedding).
"""

from __future__ import annotations

import csv
import json
import os
import statistics
import sys
from collections import defaultdict

import numpy as np

import bench
import lora_inputs as li

HERE = os.path.dirname(os.path.abspath(__file__))
_RUN = "python3 -u /root/repo/bench.py"
COMMANDS = {
    "fetch": f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d $GRAFT_REPO_ROOT/gpurun_out/pmc_fetch -o f -- "
             f"{_RUN} --steps 2 --warmup 1 --no-cpu-baseline --no-graph --extras mlp",
    "write": f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d $GRAFT_REPO_ROOT/gpurun_out/pmc_write -o w -- "
             f"{_RUN} --steps 2 --warmup 1 --no-cpu-baseline --no-graph --extras mlp",
    "copyf": f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d $GRAFT_REPO_ROOT/gpurun_out/pmc_copyf -o cf -- "
             f"{_RUN} --copy-calibration 256",
    "copyw": f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d $GRAFT_REPO_ROOT/gpurun_out/pmc_copyw -o cw -- "
             f"{_RUN} --copy-calibration 256",
    "mfma": f"rocprofv3 --pmc MfmaUtil --output-format csv -d $GRAFT_REPO_ROOT/gpurun_out/pmc_mfma -o m -- "
            f"{_RUN} --steps 2 --warmup 1 --no-cpu-baseline --no-graph --extras mlp,attention,backward",
}


def command_block(*keys: str) -> str:
    body = "\n".join(COMMANDS[k] for k in keys)
    return ("```\ncd /tmp && export TMPDIR=/tmp\n" + body +
            "\ncd $GRAFT_REPO_ROOT && python bench_profiles.py gpurun_out\n```\n\n")
SGMV_SHRINK = ("shrink_kernel", "shrink_lds_kernel", "shrink_gemv_kernel")
GEMM_LABEL = {
    "gemm_lora_kernel<0": "plain LoRA-in-K GEMM (mlp down, mlp and projection backward dx, attention q/k/v, o)",
    "gemm_lora_kernel<1": "mlp gate/up + SwiGLU (forward)",
    "gemm_lora_kernel<2": "mlp gate/up + SwiGLU (training forward, stores e, v)",
    "gemm_lora_kernel<3": "mlp backward: dhmid + SwiGLU backward",
}


def short(name: str) -> str:
    n = name.replace("void ", "").replace("lmx::", "")
    return n.split("(")[0]


def rows_of(path: str) -> list[dict]:
    with open(path) as f:
        return list(csv.DictReader(f))


def grid_of(r: dict) -> tuple[int, int]:
    if "Grid_Size_X" in r:
        return (int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]),
                int(r["Grid_Size_Y"]) // int(r["Workgroup_Size_Y"]))
    return (int(r["Grid_Size"]) // int(r["Workgroup_Size"]), 1)


def label_dispatches(disp: list[tuple[str, tuple]]) -> list[str]:
    """Workload names for a run's lmx dispatches (in dispatch order)."""
    toks = li.SWEEP_TOKENS
    keymap: dict[tuple, list[str]] = defaultdict(list)
    case, stage, i = 0, "shrink", 0
    # the opening passes: positional (separate calls, then lora_shrink_expand per case, whose
    # launches from 1024 tokens repeat the separate calls' kernels and grids)
    case2 = 0
    while i < len(disp) and case2 < len(toks):
        name, grid = disp[i]
        if case >= len(toks):
            if "pair_kernel" in name:
                lab = f"pair_tok{toks[case2]}"
                if lab not in keymap[(name, grid)]:
                    keymap[(name, grid)].append(lab)
                case2 += 1
            elif "expand" in name:
                case2 += 1
            i += 1
            continue
        if any(s in name for s in SGMV_SHRINK) or "sk_reduce" in name or "zero_ints" in name:
            lab = f"shrink_tok{toks[case]}" + (" reduce" if "sk_reduce" in name else "") + \
                  (" counter clear" if "zero_ints" in name else "")
        elif "expand" in name:
            lab = f"expand_tok{toks[case]}"
            case += 1
        else:
            i += 1
            continue
        if lab not in keymap[(name, grid)]:
            keymap[(name, grid)].append(lab)
        i += 1
    labels, in_sweep = [], True
    last_shrink: set = set()  # token counts the latest shrink dispatch can belong to
    for name, grid in disp:
        if "gemm_lora_kernel" in name or "embedding" in name or "sums_kernel" in name or "scale_lora_b" in name:
            in_sweep = False
        labs = keymap.get((name, grid), []) if in_sweep else []
        if labs and all(l.startswith("shrink_tok") and " " not in l for l in labs):
            last_shrink = {l[len("shrink_tok"):] for l in labs}
        cand = {l[len("expand_tok"):] for l in labs if l.startswith("expand_tok")} & last_shrink
        if len(labs) > 1 and "expand" in name and len(cand) == 1:
            # grids that coincide once flattened (counter runs give only the total size): every
            # call sequence runs a case's shrink right before its expand
            labels.append(f"expand_tok{cand.pop()}")
        elif labs:
            labels.append(" / ".join(labs))
        elif "gemm_lora_kernel" in name:
            key = name[:name.index("<") + 2]
            labels.append(GEMM_LABEL.get(key, name))
        else:
            labels.append("mlp / attention / backward" if not in_sweep else "sweep (other)")
    return labels


def trace_table(path: str) -> tuple[str, dict]:
    rows = sorted(rows_of(path), key=lambda r: int(r["Start_Timestamp"]))
    rows = [r for r in rows if "lmx::" in r["Kernel_Name"]]
    disp = [(short(r["Kernel_Name"]), grid_of(r)) for r in rows]
    labels = label_dispatches(disp)
    groups = defaultdict(list)
    for r, (name, grid), lab in zip(rows, disp, labels):
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups[(name, grid, lab)].append(d)
    lines = ["| kernel | grid | workload | dispatches | median us | mean us |",
             "|---|---:|---|---:|---:|---:|"]
    per_label = {}
    for (name, grid, lab), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{name}` | {grid[0]} x {grid[1]} | {lab} | {len(v)} | "
                     f"{statistics.median(v):.2f} | {statistics.mean(v):.2f} |")
        per_label[lab] = statistics.median(v)
    return "\n".join(lines), per_label


def counter_per_label(path: str) -> dict:
    rows = sorted(rows_of(path), key=lambda r: int(r["Dispatch_Id"]))
    rows = [r for r in rows if "lmx::" in r["Kernel_Name"]]
    disp = [(short(r["Kernel_Name"]), grid_of(r)) for r in rows]
    labels = label_dispatches(disp)
    out = defaultdict(list)
    for r, (name, grid), lab in zip(rows, disp, labels):
        out[(name, grid, lab)].append(float(r["Counter_Value"]))
    return {k: statistics.median(v) for k, v in out.items()}


def copy_kib(path: str) -> float:
    rows = [r for r in rows_of(path) if "copy" in r["Kernel_Name"].lower() or "elementwise" in r["Kernel_Name"]]
    vals = [float(r["Counter_Value"]) for r in rows]
    return statistics.median(vals) if vals else float("nan")


def main() -> int:
    d = sys.argv[1]
    os.makedirs(os.path.join(HERE, "profiles"), exist_ok=True)
    alg = {}
    for T in li.SWEEP_TOKENS:
        a = bench.algorithmic(li.sweep_case(T))
        alg[f"shrink_tok{T}"] = a["shrink_bytes"]
        alg[f"expand_tok{T}"] = a["expand_bytes"]
        alg[f"pair_tok{T}"] = a["shrink_bytes"] + a["expand_bytes"]

    table, per_label = trace_table(os.path.join(d, "prof_bench", "bench_kernel_trace.csv"))
    with open(os.path.join(HERE, "profiles", "sgmv_sweep_and_mlp_kernel_trace.md"), "w") as f:
        f.write("# Kernel trace: decode-QKV LoRA shrink+expand sweep (tok 50..8192), fused LoRA+SwiGLU "
                "MLP (forward, training forward, backward), LoRA attention projections, embedding LoRA-A\n\n"
                "Command (MI355X, one GPU):\n\n```\ncd /tmp && export TMPDIR=/tmp && rocprofv3 "
                "--kernel-trace --stats --output-format csv -d $GRAFT_REPO_ROOT/gpurun_out/prof_bench "
                "-o bench -- python3 -u /root/repo/bench.py --steps 5 --warmup 2 --no-cpu-baseline\n"
                "python bench_profiles.py gpurun_out\n```\n\n"
                "Durations are rocprofv3 kernel-trace start/end per dispatch, in microseconds, over every "
                "phase of the benchmark (eager warm-up and breakdown, 30 cold calls per workload after a "
                "512 MiB write, graph replays). Sweep workload: bf16, 4 adapters of rank 16, K = 4096, "
                "slices N = 4096 + 1024 + 1024. MLP: bf16 M = 4096, H = 4096, I = 12288, r = 16; "
                "attention projections M = 4096, H = 4096, Nq = 4096, Nkv = 1024, r = 16.\n\n")
        f.write(table + "\n")

    ff_kib = copy_kib(os.path.join(d, "pmc_copyf", "cf_counter_collection.csv"))
    fw_kib = copy_kib(os.path.join(d, "pmc_copyw", "cw_counter_collection.csv"))
    copy_mib = 256.0
    fetch_factor = copy_mib * 1024 / ff_kib
    write_factor = copy_mib * 1024 / fw_kib
    fetch = counter_per_label(os.path.join(d, "pmc_fetch", "f_counter_collection.csv"))
    write = counter_per_label(os.path.join(d, "pmc_write", "w_counter_collection.csv"))
    lines = ["| kernel | workgroups | workload | FETCH KiB | WRITE KiB | HBM bytes (scaled) | algorithmic bytes | ratio |",
             "|---|---:|---|---:|---:|---:|---:|---:|"]
    kernels = {}
    mlp_bytes = 0.0
    for key in sorted(set(fetch) & set(write), key=lambda k: (k[2], k[0])):
        name, grid, lab = key
        fk, wk = fetch[key], write[key]
        hbm = fk * 1024 * fetch_factor + wk * 1024 * write_factor
        a = alg.get(lab)
        ratio = f"{hbm / a:.3f}" if a else ""
        lines.append(f"| `{name}` | {grid[0] * grid[1]} | {lab} | {fk:.1f} | {wk:.1f} | {hbm:,.0f} | "
                     f"{'' if a is None else f'{a:,}'} | {ratio} |")
        if a is not None:
            kernels[lab] = {"hbm_bytes_per_launch": int(round(hbm)), "fetch_kib": fk, "write_kib": wk}
        elif not lab.startswith(("shrink_tok", "expand_tok", "pair_tok")):
            mlp_bytes += hbm  # these runs time only the fused MLP after the sweep: one call each
    kernels["mlp_fused"] = {"hbm_bytes_per_launch": int(round(mlp_bytes)),
                            "note": "sum over the launches of one lora_mlp_fused call"}
    lines.append(f"| (sum) | | one lora_mlp_fused call | | | {mlp_bytes:,.0f} | | |")
    with open(os.path.join(HERE, "profiles", "hbm_traffic_counters.md"), "w") as f:
        f.write("# HBM traffic per launch: FETCH_SIZE and WRITE_SIZE\n\n"
                "Commands (MI355X, one GPU; each counter in its own run):\n\n" +
                command_block("fetch", "write", "copyf", "copyw") +
                f"Calibration: a plain device copy of 256 MiB reads {ff_kib / 1024:.1f} MiB by FETCH_SIZE "
                f"and writes {fw_kib / 1024:.1f} MiB by WRITE_SIZE, so FETCH_SIZE is scaled by "
                f"{fetch_factor:.3f} and WRITE_SIZE by {write_factor:.3f} below. Medians over the "
                "dispatches of each kernel, grid and workload.\n\n")
        f.write("\n".join(lines) + "\n")
    json.dump({"source_sha": bench._kernel_source_sha(), "fetch_factor": fetch_factor,
               "write_factor": write_factor, "kernels": kernels},
              open(os.path.join(HERE, "profiles", "traffic.json"), "w"), indent=1)

    mf = counter_per_label(os.path.join(d, "pmc_mfma", "m_counter_collection.csv"))
    lines = ["| kernel | workgroups | workload | median MfmaUtil % |", "|---|---:|---|---:|"]
    for (name, grid, lab), v in sorted(mf.items(), key=lambda kv: kv[0][0]):
        if "gemm" in name or "sums_kernel" in name or "shrink_lds" in name:
            lines.append(f"| `{name}` | {grid[0] * grid[1]} | {lab} | {v:.1f} |")
    with open(os.path.join(HERE, "profiles", "mfma_utilisation.md"), "w") as f:
        f.write("# MFMA utilisation of the GEMM launches: fused MLP forward, training forward, backward, "
                "attention projections\n\nCommand (MI355X, one GPU):\n\n" + command_block("mfma") +
                "`MfmaUtil` is rocprofv3's derived metric: the percentage of the kernel's active cycles in "
                "which the matrix cores are busy (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE times the "
                "SIMD count), per dispatch; the median over the run's dispatches is listed.\n\n")
        f.write("\n".join(lines) + "\n")
    print("wrote profiles/ summaries; fetch factor", round(fetch_factor, 3), "write factor",
          round(write_factor, 3))
    return 0


if __name__ == "__main__":
    sys.exit(main())
