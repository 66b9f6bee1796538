"""Benchmark of the Gated DeltaNet replay path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ID] [--no-cpu]

One step is one pass of the whole path over one batch of synthetic input
already resident in HBM.  The default workload (3) is the largest: one
32768-token sequence through 32 heads with dk = dv = 128, bf16 inputs, fp32
state, zero start state, outputs o (fp32) for every token and the final
state -- the full-prefill shape that the Tail-Replay page compares replay
against (section 4, Table 2, at 32K).  Other workloads: 1 = a tail replay of
one request, the latest 3277 tokens (10% of a 32768-token prefix), final
state only (section 3, Eq. (2)); 2 = 16 packed tails of 410..3277 tokens
with outputs; 4 = 64 chunk operators of 512 tokens and their composition;
0 = one fp32 head.

``--decode N`` instead times single-token decode of N requests from given
states (the serving step after a replay).  ``--front-end`` instead times
the front end (normalised q and k, activated gates) on the tail-replay
shape (with ``--with-replay`` also the front end followed by a replay
against gdn_replay_raw, the front end inside the replay, on the tail and on
the 32768-token prefill with outputs).
``--overlap MIB`` instead times a pinned-host -> device copy of MIB MiB on
a copy stream beside ``--layers`` tail replays: alone, serialised and
overlapped.  ``--scalar-ops`` instead times the scalar-decay (Mamba-2
family) chunk operators and their composition on the chunk-operator shape.  ``--tail-curve`` instead
reports the tail-replay state error against the
replayed fraction (the latest k tokens of a 32768-token prefix replayed
from zero, against the full replay) next to the stored fp64 oracle curve.

Prints ONE JSON line.  ``value`` is replayed tokens x heads per second;
``roofline`` compares the dominant kernel's algorithmic HBM bytes per launch
over its average launch time (HIP events on the launch stream) against the
8 TB/s HBM3E peak; ``cpu_baseline`` is the fp64 oracle timed on this host's
cores on the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN replay tokens·heads/s (H=32,d=128) + % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2516.6


def algorithmic(inp, want_o: bool, o_bytes: int, C: int = 64):
    """Algorithmic HBM bytes and flops of one replay launch.

    Bytes: every input read once (q only with outputs), o written once,
    S_final written once (no S0).  Flops: the chunked form's products,
    2C(3dk + 2dv) + 6 dk dv per token x head with outputs, 2C(2dk + dv) +
    4 dk dv state-only.
    """
    import numpy as np
    T, H, dk, dv = inp.n_tokens, inp.H, inp.dk, inp.dv
    es = 2 if inp.dtype == "bf16" else 4
    per_tok = (dk + dv) * es + 2 * es + ((dk * es + dv * o_bytes) if want_o else 0)
    byt = T * H * per_tok + inp.n_seqs * H * dv * dk * 4
    if want_o:
        fl = T * H * (2 * C * (3 * dk + 2 * dv) + 6 * dk * dv)
    else:
        fl = T * H * (2 * C * (2 * dk + dv) + 4 * dk * dv)
    return int(byt), int(fl)


def to_dev(inp, torch, np):
    def t(a):
        if inp.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return dict(q=t(inp.q), k=t(inp.k), v=t(inp.v), alpha=t(inp.alpha), beta=t(inp.beta),
                cu=torch.from_numpy(inp.cu_seqlens.astype(np.int32)).cuda())


def measured_traffic(workload_name, kernel=None):
    """HBM bytes per call (or per launch of the kernels whose names start
    with ``kernel``) from the committed counter summary for this workload,
    or None when the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload_name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("workload") != workload_name or rec.get("sources_sha256") != sources_sha256():
        return None
    if kernel is not None:
        ks = [v for n, v in rec["kernels"].items() if n.startswith(kernel)]
        return int(sum(v["fetch_bytes"] + v["write_bytes"] for v in ks)) if ks else None
    return int(rec["hbm_bytes_per_call"])


def uninstrumented_ms(fn, steps, torch):
    """Wall-clock milliseconds per call of ``steps`` back-to-back calls with
    no events between them, synchronised on both sides (the throughput pass;
    event pairs around each call add a few microseconds per call)."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def code_text(src):
    """C/C++/HIP source without its comments and whitespace (string and
    character literals kept as written): what the compiler sees as code."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            if not c.isspace():
                out.append(c)
            i += 1
    return "".join(out)


def sources_sha256():
    """Hash of the kernel and library sources as code (comments and
    whitespace left out): the counter summaries in profiles/ carry it, and
    their traffic figures count only while it matches."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for src in sorted(glob.glob(os.path.join(ROOT, "gated_deltanet_state_amd", "csrc", "*"))):
        with open(src, encoding="utf-8") as f:
            h.update(code_text(f.read()).encode("utf-8"))
    return h.hexdigest()


def _csv_rows(folder, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(folder, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit("no *%s under %s" % (suffix, folder))
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _short(name):
    # names with a bf16 template argument stay mangled in the trace
    # (gdn::(anonymous)::NAME<int, bf16|float>(...))
    m = re.match(r"_ZN3gdn12_GLOBAL__N_1(\d+)", name)
    if m:
        n = int(m.group(1))
        base = name[m.end():m.end() + n]
        args = re.findall(r"Li(\d+)E|(DF16b)|(?<=E)(f)(?=E)", name[m.end() + n:])
        parts = [a or ("bf16" if b else "float") for a, b, c in args if a or b or c]
        return "%s<%s>" % (base, ", ".join(parts)) if parts else base
    name = name.replace("void ", "").replace("gdn::(anonymous namespace)::", "")
    return name.split("(")[0]


def _counter_kib(folder, counter):
    """Mean counter value per dispatch of each kernel (KiB for FETCH_SIZE and
    WRITE_SIZE), summed over the counter's instances within a dispatch."""
    import collections
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for r in _csv_rows(folder, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        per[_short(r["Kernel_Name"])][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in per.items()}


ISSUE_COUNTERS = ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                  "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "GRBM_GUI_ACTIVE"]


def issue_table(mfma_dir, stats):
    """Rows of the MFMA / issue table from one --pmc run of ISSUE_COUNTERS:
    per kernel, the executed bf16 MFMA flops (SQ_INSTS_VALU_MFMA_MOPS_BF16
    counts them in units of 512) over the kernel's average time from the
    trace, as a fraction of the 2.52 PFLOP/s dense bf16 peak, and the vector,
    MFMA, LDS and scalar instructions issued per wave."""
    vals = {c: _counter_kib(mfma_dir, c) for c in ISSUE_COUNTERS}
    avg_us = {_short(r["Name"]): float(r["AverageNs"]) / 1e3 for r in stats}
    rows = {}
    for k in sorted(vals["SQ_WAVES"]):
        if "rocclr" in k:
            continue
        waves = vals["SQ_WAVES"].get(k, 0.0) or float("nan")
        flops = vals["SQ_INSTS_VALU_MFMA_MOPS_BF16"].get(k, 0.0) * 512
        t = avg_us.get(k)
        rows[k] = dict(waves=waves, valu_per_wave=vals["SQ_INSTS_VALU"].get(k, 0.0) / waves,
                       mfma_per_wave=vals["SQ_INSTS_MFMA"].get(k, 0.0) / waves,
                       lds_per_wave=vals["SQ_INSTS_LDS"].get(k, 0.0) / waves,
                       salu_per_wave=vals["SQ_INSTS_SALU"].get(k, 0.0) / waves,
                       mfma_bf16_flops=flops,
                       mfma_tflops=(flops / (t * 1e-6) / 1e12) if t else None,
                       mfma_busy_cycles=vals["SQ_VALU_MFMA_BUSY_CYCLES"].get(k, 0.0),
                       sq_busy_cycles=vals["SQ_BUSY_CYCLES"].get(k, 0.0),
                       grbm_gui_active=vals["GRBM_GUI_ACTIVE"].get(k, 0.0))
        if t:
            rows[k]["mfma_frac_of_peak"] = rows[k]["mfma_tflops"] / BF16_MFMA_PEAK_TFLOPS
    return rows


CYCLE_COUNTERS = ["SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
                  "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"]


def cycle_table(cycle_dir):
    """Rows of the wave-cycle table from one --pmc run of CYCLE_COUNTERS: per
    kernel, the share of its waves' cycles spent issuing any instruction,
    vector-ALU and LDS instructions, waiting on a dependency (s_waitcnt,
    barrier), and ready but not chosen for issue (another wave of the SIMD
    issued); and the share of the LDS's active cycles lost to bank
    conflicts."""
    vals = {c: _counter_kib(cycle_dir, c) for c in CYCLE_COUNTERS}
    rows = {}
    for k in sorted(vals["SQ_WAVE_CYCLES"]):
        if "rocclr" in k:
            continue
        wc = vals["SQ_WAVE_CYCLES"][k] or float("nan")
        idx = vals["SQ_LDS_IDX_ACTIVE"].get(k, 0.0)
        rows[k] = dict(active=vals["SQ_ACTIVE_INST_ANY"].get(k, 0.0) / wc,
                       valu=vals["SQ_ACTIVE_INST_VALU"].get(k, 0.0) / wc,
                       lds=vals["SQ_ACTIVE_INST_LDS"].get(k, 0.0) / wc,
                       wait=vals["SQ_WAIT_ANY"].get(k, 0.0) / wc,
                       wait_issue=vals["SQ_WAIT_INST_ANY"].get(k, 0.0) / wc,
                       lds_conflict=(vals["SQ_LDS_BANK_CONFLICT"].get(k, 0.0) / idx) if idx else None)
    return rows


def summarize_counters(wid, stats_dir, fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, command="",
                       name=None, mfma_dir=None, cycle_dir=None):
    """profiles/<workload>.md and profiles/traffic_<workload>.json from
    rocprofv3 runs of this script: a --kernel-trace --stats run, one --pmc
    FETCH_SIZE run, one --pmc WRITE_SIZE run, and the same two counters on a
    --calibrate-copy run (bytes = counter x 1024 / (counter bytes per byte
    copied))."""
    import workloads
    wname = name or workloads.WORKLOADS[wid]["name"]
    stats = [r for r in _csv_rows(stats_dir, "kernel_stats.csv") if "rocclr" not in r["Name"]]
    fetch, write = _counter_kib(fetch_dir, "FETCH_SIZE"), _counter_kib(write_dir, "WRITE_SIZE")
    cf, cw = _counter_kib(cal_fetch_dir, "FETCH_SIZE"), _counter_kib(cal_write_dir, "WRITE_SIZE")
    copy_kib = {k: v for k, v in cf.items() if "copy" in k.lower()}
    copy_wkib = {k: v for k, v in cw.items() if "copy" in k.lower()}
    if not copy_kib or not copy_wkib:
        raise SystemExit("no copy kernel in the calibration runs")
    cal_mib = 256
    ff = list(copy_kib.values())[0] / (cal_mib * 1024.0)
    wf = list(copy_wkib.values())[0] / (cal_mib * 1024.0)
    kernels, total = {}, 0.0
    for k in sorted((set(fetch) | set(write)) - {k for k in set(fetch) | set(write) if "rocclr" in k}):
        fb, wb = fetch.get(k, 0.0) * 1024 / ff, write.get(k, 0.0) * 1024 / wf
        kernels[k] = dict(fetch_kib=fetch.get(k, 0.0), write_kib=write.get(k, 0.0), fetch_bytes=fb, write_bytes=wb)
        total += fb + wb
    rec = dict(workload=wname, sources_sha256=sources_sha256(),
               calibration=dict(copy_mib=cal_mib, fetch_factor=round(ff, 4), write_factor=round(wf, 4)),
               kernels=kernels, hbm_bytes_per_call=int(total))
    issue = issue_table(mfma_dir, stats) if mfma_dir else None
    if issue:
        rec["issue"] = issue
    cycles = cycle_table(cycle_dir) if cycle_dir else None
    if cycles:
        rec["wave_cycles"] = cycles
    with open(os.path.join(ROOT, "profiles", "traffic_%s.json" % wname), "w") as f:
        json.dump(rec, f, indent=1)
    lines = ["# %s: kernel times and HBM traffic" % wname, "",
             "Kernel trace (rocprofv3 `--kernel-trace --stats`):", "", "```", command or "(command not recorded)",
             "```", "", "| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    tot_avg = 0.0
    for r in stats:
        avg = float(r["AverageNs"]) / 1e3
        tot_avg += avg
        lines.append("| %s | %s | %.2f | %.2f | %.2f | %.1f%% |" % (
            _short(r["Name"]), r["Calls"], avg, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
            float(r["Percentage"])))
    lines += ["", "Sum of the kernel averages: %.1f us per call." % tot_avg, "",
              "HBM traffic per dispatch (one `--pmc` counter per run; a %d MiB device copy reads %.3f KiB of "
              "FETCH_SIZE and writes %.3f KiB of WRITE_SIZE per KiB moved):" % (cal_mib, ff, wf), "",
              "| kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | read (MB) | written (MB) |", "|---|---|---|---|---|"]
    for k, v in kernels.items():
        lines.append("| %s | %.0f | %.0f | %.1f | %.1f |" % (k, v["fetch_kib"], v["write_kib"], v["fetch_bytes"] / 1e6,
                                                           v["write_bytes"] / 1e6))
    lines += ["", "HBM bytes per call: %.1f MB." % (total / 1e6), ""]
    if issue:
        lines += ["MFMA use and instruction issue per dispatch (one `--pmc` run of %s; executed bf16 MFMA "
                  "flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, over the kernel's average time above, against "
                  "the %.1f TFLOP/s dense bf16 peak; instructions per wave = SQ_INSTS_* / SQ_WAVES):"
                  % (", ".join(ISSUE_COUNTERS), BF16_MFMA_PEAK_TFLOPS), "",
                  "| kernel | waves | executed bf16 MFMA (GFLOP) | MFMA TFLOP/s | of bf16 peak | VALU / wave | "
                  "MFMA / wave | LDS / wave | SALU / wave | SQ_VALU_MFMA_BUSY_CYCLES | GRBM_GUI_ACTIVE |",
                  "|---|---|---|---|---|---|---|---|---|---|---|"]
        for k, v in issue.items():
            lines.append("| %s | %.0f | %.2f | %s | %s | %.0f | %.0f | %.0f | %.0f | %.3g | %.3g |" % (
                k, v["waves"], v["mfma_bf16_flops"] / 1e9,
                "%.1f" % v["mfma_tflops"] if v["mfma_tflops"] is not None else "-",
                "%.1f%%" % (100 * v["mfma_frac_of_peak"]) if "mfma_frac_of_peak" in v else "-",
                v["valu_per_wave"], v["mfma_per_wave"], v["lds_per_wave"], v["salu_per_wave"],
                v["mfma_busy_cycles"], v["grbm_gui_active"]))
        lines.append("")
    if cycles:
        lines += ["Where the waves' cycles go (one `--pmc` run of %s; shares of SQ_WAVE_CYCLES: issuing any "
                  "instruction (SQ_ACTIVE_INST_ANY), of which vector ALU and LDS, waiting on a dependency or "
                  "barrier (SQ_WAIT_ANY), ready but not issued because another wave of the SIMD issued "
                  "(SQ_WAIT_INST_ANY); LDS bank conflicts = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE):"
                  % ", ".join(CYCLE_COUNTERS), "",
                  "| kernel | issuing | vector ALU | LDS | waiting | not chosen | LDS bank-conflict cycles |",
                  "|---|---|---|---|---|---|---|"]
        for k, v in cycles.items():
            lines.append("| %s | %.1f%% | %.1f%% | %.1f%% | %.1f%% | %.1f%% | %s |" % (
                k, 100 * v["active"], 100 * v["valu"], 100 * v["lds"], 100 * v["wait"], 100 * v["wait_issue"],
                "%.1f%%" % (100 * v["lds_conflict"]) if v["lds_conflict"] is not None else "-"))
        lines.append("")
    with open(os.path.join(ROOT, "profiles", "%s.md" % wname), "w") as f:
        f.write("\n".join(lines))
    print("wrote profiles/%s.md and profiles/traffic_%s.json" % (wname, wname))


def cpu_baseline(inp, want_o, wid, min_seconds=10.0):
    """fp64 oracle on the same workload: whole heads, repeated to >= min_seconds,
    or a subset of heads when one full pass would be long."""
    import oracle
    f = inp.f64
    heads = list(range(inp.H))
    # estimate: ~1.2 GFLOP/s per thread for the plain fp64 loops
    thr = oracle.threads()
    est = inp.n_tokens * inp.H * (6 if want_o else 4) * inp.dk * inp.dv / (1.2e9 * thr)
    if est > 20.0:
        keep = max(1, int(inp.H * 20.0 / est))
        heads = heads[:keep]
    sel = heads
    args = (f["q"][:, sel] if want_o else None, f["k"][:, sel], f["v"][:, sel],
            f["alpha"][:, sel], f["beta"][:, sel], inp.cu_seqlens)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.replay(*args, want_o=want_o)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    th = reps * inp.n_tokens * len(heads) / el
    sample = "%d full pass(es) of the workload over %d of %d heads, %s, fp64" % (
        reps, len(heads), inp.H, "with o" if want_o else "state only")
    return dict(value=th, unit="tokens·heads/s", cores=thr, kind="oracle", sample=sample,
                seconds=el)


def tail_curve_gpu(law, gdn, torch, np):
    """Relative state error ||S_tail - S_full|| / ||S_full|| of replaying only
    the latest k tokens of the 32768-token prefix from zero (Tail-Replay,
    section 3), for every k of workloads.TAIL_CURVE_KS, with gdn_replay: one
    call for the full prefix, one packed call for all the tails."""
    import workloads
    inp = workloads.tail_curve_inputs(law)
    d = to_dev(inp, torch, np)
    m, ks = workloads.TAIL_CURVE_M, workloads.TAIL_CURVE_KS
    _, S_full = gdn.replay(None, d["k"], d["v"], d["alpha"], d["beta"], d["cu"], want_o=False)
    idx = torch.cat([torch.arange(m - kk, m, device="cuda") for kk in ks])
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(ks)]).astype(np.int32)).cuda()
    sel = {n: d[n][idx].contiguous() for n in ("k", "v", "alpha", "beta")}
    _, S_tail = gdn.replay(None, sel["k"], sel["v"], sel["alpha"], sel["beta"], cu, want_o=False)
    torch.cuda.synchronize()
    S_full = S_full.double().cpu().numpy()
    S_tail = S_tail.double().cpu().numpy()
    return [float(np.linalg.norm(S_tail[i] - S_full[0]) / np.linalg.norm(S_full)) for i in range(len(ks))]


def tail_curve_report(gdn, torch, np):
    """One JSON line: the GPU tail-error curve next to the stored fp64 oracle
    curve and its bound (tests/golden/tail_curve.json)."""
    import workloads
    with open(os.path.join(ROOT, "tests", "golden", "tail_curve.json")) as fh:
        ref = json.load(fh)
    out = dict(metric="tail-replay relative state error ||S_tail - S_full|| / ||S_full||",
               m=workloads.TAIL_CURVE_M, k=workloads.TAIL_CURVE_KS,
               fraction=[round(kk / workloads.TAIL_CURVE_M, 6) for kk in workloads.TAIL_CURVE_KS], laws={})
    for law in workloads.TAIL_CURVE_LAWS:
        gpu = tail_curve_gpu(law, gdn, torch, np)
        out["laws"][law] = dict(gate_scale=workloads.TAIL_CURVE_LAWS[law], gpu=[float("%.3e" % x) for x in gpu],
                                oracle=[float("%.3e" % x) for x in ref["laws"][law]["err"]],
                                bound=[float("%.3e" % x) for x in ref["laws"][law]["bound"]])
    print(json.dumps(out))


def decode_report(args, gdn, torch, np):
    """One JSON line: batched single-token decode (gdn_decode) from given
    states, the serving step after a replay; HBM-bound (every state read and
    written once)."""
    import workloads
    N, H, d = args.decode, 32, 128
    inp = workloads.generate([1] * N, H=H, dk=d, dv=d, dtype="bf16", seed=5)
    dd = to_dev(inp, torch, np)
    rng = np.random.Generator(np.random.PCG64(6))
    S_in = torch.from_numpy((rng.standard_normal((N, H, d, d)) * 0.3).astype(np.float32)).cuda()
    S = torch.empty_like(S_in)
    o = torch.empty((N, H, d), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        gdn.decode(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], S_in=S_in, out=o, S_out=S)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t_wall = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        call()
        ends[i].record(stream)
    torch.cuda.synchronize()
    instr_ms = (time.perf_counter() - t_wall) * 1e3 / args.steps
    kern_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    avg = sum(kern_ms) / len(kern_ms)
    step_ms = uninstrumented_ms(call, args.steps, torch)
    # per (sequence, head): state read and written (fp32), q, k, v (bf16), gates, o (fp32)
    byt = N * H * (2 * d * d * 4 + 3 * d * 2 + 2 * 2 + d * 4)
    achieved = byt / (avg / 1e3) / 1e9
    line = dict(metric="GDN decode tokens·heads/s (one token per request from its state)",
                value=round(N * H / (step_ms / 1e3), 1), unit="tokens·heads/s", n_gpus=1,
                steps=args.steps, warmup=args.warmup, ms_per_step=round(step_ms, 5), higher_is_better=True,
                scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
                config=dict(workload="decode-%dx1-H32-d128-bf16" % N, n_seqs=N, n_tokens=N, heads=H, dk=d, dv=d,
                            outputs="o,S_final", state="fp32 in and out"),
                roofline=dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                              frac=round(achieved / HBM_PEAK_GBS, 4),
                              traffic=measured_traffic("decode-%dx1-H32-d128-bf16" % N), kernel="decode_kernel",
                              algorithmic_bytes=byt, kernel_ms_avg=round(avg, 5),
                              kernel_ms_min=round(min(kern_ms), 5)))
    line["gpu_ms_per_step"] = round(avg, 5)
    line["instrumented_ms_per_step"] = round(instr_ms, 5)
    print(json.dumps(line), flush=True)


FRONT_NAME = "front-end-T3277-H32-d128-bf16"
SCALAR_NAME = "scalar-ops-64x512-H32-d128-bf16"


def scalar_ops_report(args, gdn, torch, np):
    """One JSON line: scalar-decay chunk operators (the Mamba-2 family) on
    the chunk-operator workload's shape (64 chunks of 512 tokens, 32 heads,
    d = 128, bf16) and their composition; the operator kernel is HBM-bound
    (keys, values and gates read once, S_local written once)."""
    import workloads
    w = workloads.WORKLOADS[4]
    inp = workloads.make_workload(4)
    d = to_dev(inp, torch, np)
    cu = torch.from_numpy(workloads.chunk_bounds(inp.n_tokens, w["chunk"])).cuda()
    C, H, dk, dv, T = cu.shape[0] - 1, inp.H, inp.dk, inp.dv, inp.n_tokens
    S = torch.empty((H, dv, dk), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    ops = [None, None]

    def op():
        ops[:] = gdn.scalar_chunk_operator(d["k"], d["alpha"], d["beta"], cu, v=d["v"])

    def comp():
        gdn.scalar_compose(ops[0], ops[1], out=S)

    def timed(fns):
        for _ in range(args.warmup):
            for f in fns:
                f()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(args.steps)]
        for e in ev:
            e[0].record(stream)
            for i, f in enumerate(fns):
                f()
                e[i + 1].record(stream)
        torch.cuda.synchronize()
        per = [sum(e[i].elapsed_time(e[i + 1]) for e in ev) / len(ev) for i in range(len(fns))]
        return per

    t_op, t_comp = timed([op, comp])

    def both():
        op()
        comp()
    wall = uninstrumented_ms(both, args.steps, torch)
    # keys and values (bf16), gates (bf16) read; S_local (fp32) and gamma written
    byt = T * H * (dk + dv) * 2 + T * H * 2 * 2 + C * H * (dv * dk + 1) * 4
    achieved = byt / (t_op / 1e3) / 1e9
    line = dict(metric="GDN scalar-decay chunk operators + composition, tokens·heads/s",
                value=round(T * H / (wall / 1e3), 1), unit="tokens·heads/s", n_gpus=1, steps=args.steps,
                warmup=args.warmup, ms_per_step=round(wall, 5), higher_is_better=True, scaling="weak",
                vs_baseline=None, dtype="bf16", data="synthetic",
                config=dict(workload=SCALAR_NAME, n_chunks=C, chunk=w["chunk"], n_tokens=T, heads=H, dk=dk, dv=dv,
                            outputs="gamma,S_local,S"),
                roofline=dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                              frac=round(achieved / HBM_PEAK_GBS, 4), traffic=measured_traffic(SCALAR_NAME, "scalar_op"),
                              kernel="scalar_op_dma_kernel", algorithmic_bytes=byt, kernel_ms_avg=round(t_op, 5)),
                compose_ms=round(t_comp, 5))
    line["gpu_ms_per_step"] = round(t_op + t_comp, 5)
    print(json.dumps(line), flush=True)


def overlap_report(args, gdn, torch, np):
    """One JSON line: a pinned-host -> device copy of a synthetic attention
    KV buffer on a copy stream, concurrent with tail replays on the compute
    stream (the Tail-Replay page, section 3: the replay does not need the
    attention layers' cached keys and values, so their transfer can run
    beside it and is waited for only before the query's forward).  The
    replays are the tail-replay workload (3277 tokens, 32 heads, d = 128,
    state only), one per linear-attention layer of the group."""
    import workloads
    mib, layers = args.overlap, args.layers
    inp = workloads.make_workload(1)
    d = to_dev(inp, torch, np)
    host = torch.empty(mib << 20, dtype=torch.uint8, pin_memory=True)
    host.copy_(torch.from_numpy(np.random.Generator(np.random.PCG64(8)).integers(0, 256, mib << 20, dtype=np.uint8)))
    dst = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    comp = torch.cuda.current_stream()
    copy = torch.cuda.Stream()    # default priority

    def replays():
        for _ in range(layers):
            gdn.replay(None, d["k"], d["v"], d["alpha"], d["beta"], d["cu"], want_o=False, stream=comp)

    def run(mode):
        """Enqueue one step of the mode: the copy alone, the replays alone,
        the copy then the replays on one stream (serialised), or the copy on
        the copy stream beside the replays, joined at the end (overlapped)."""
        if mode == "overlap":
            ev0 = torch.cuda.Event()
            ev0.record(comp)
            copy.wait_event(ev0)
            with torch.cuda.stream(copy):
                dst.copy_(host, non_blocking=True)
            evc = torch.cuda.Event()
            evc.record(copy)
            replays()
            comp.wait_event(evc)
            return
        if mode != "replay":
            dst.copy_(host, non_blocking=True)
        if mode != "copy":
            replays()

    modes = ("copy", "replay", "serial", "overlap")
    for mode in modes:
        for _ in range(args.warmup):
            run(mode)
    torch.cuda.synchronize()
    # the modes take turns, each step timed alone from an idle device (wall
    # clock around synchronisations, as a time to first token would see it,
    # and HIP events on the compute stream)
    wall = {m: [] for m in modes}
    gpu = {m: [] for m in modes}
    for _ in range(args.steps):
        for mode in modes:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            a.record(comp)
            run(mode)
            b.record(comp)
            torch.cuda.synchronize()
            wall[mode].append((time.perf_counter() - t0) * 1e3)
            gpu[mode].append(a.elapsed_time(b))
    res = {m: float(np.median(gpu[m])) for m in modes}
    res_wall = {m: float(np.median(wall[m])) for m in modes}
    assert torch.equal(dst[:4096].cpu(), host[:4096])
    hidden = (res["serial"] - res["overlap"]) / min(res["copy"], res["replay"])
    tok = layers * inp.n_tokens * inp.H
    line = dict(metric="GDN replay tokens·heads/s beside a host-to-device KV copy (overlapped)",
                value=round(tok / (res["overlap"] / 1e3), 1), unit="tokens·heads/s", n_gpus=1, steps=args.steps,
                warmup=args.warmup, ms_per_step=round(res["overlap"], 5), higher_is_better=True, scaling="weak",
                vs_baseline=None, dtype="bf16", data="synthetic",
                config=dict(workload="overlap-%dMiB-%dx-tail-replay-T3277-H32-d128-bf16" % (mib, layers),
                            copy_mib=mib, replays=layers, n_tokens=inp.n_tokens, heads=inp.H),
                ms=dict((k, round(v, 5)) for k, v in res.items()),
                wall_ms=dict((k, round(v, 5)) for k, v in res_wall.items()),
                copy_gbs=round((mib << 20) / (res["copy"] / 1e3) / 1e9, 2),
                reduction_vs_serial=round(1 - res["overlap"] / res["serial"], 4),
                hidden_fraction_of_shorter=round(hidden, 4))
    print(json.dumps(line), flush=True)


def front_end_report(args, gdn, torch, np):
    """One JSON line: gdn_front_end on the tail-replay shape (3277 tokens,
    32 heads, dk = 128, bf16, queries and keys); HBM-bound (every raw input
    read once and every prepared output written once).  With
    ``--with-replay`` also: the front end without queries followed by the
    state-only replay, the replay of prepared inputs, and gdn_replay_raw
    (the front end inside the replay) on that shape; and the same three on
    the 32768-token prefill with outputs."""
    import workloads
    T, H, d = workloads.tail_length(32768, "0.1"), 32, 128
    raw = workloads.generate_raw([T], H=H, dk=d, dv=d, dtype="bf16", seed=7)

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    qr, kr, g, b, v = t(raw.q_raw), t(raw.k_raw), t(raw.g), t(raw.b), t(raw.v)
    cu = torch.from_numpy(raw.cu_seqlens).cuda()
    out = (torch.empty_like(qr), torch.empty_like(kr), torch.empty_like(g), torch.empty_like(b))
    out_k = (None,) + out[1:]
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for a, e in ev:
            a.record(stream)
            fn()
            e.record(stream)
        torch.cuda.synchronize()
        ms = [a.elapsed_time(e) for a, e in ev]
        return sum(ms) / len(ms), min(ms)

    avg, mn = timed(lambda: gdn.front_end(qr, kr, g, b, out=out))
    wall = uninstrumented_ms(lambda: gdn.front_end(qr, kr, g, b, out=out), args.steps, torch)
    extra = {}
    if args.with_replay:
        both, _ = timed(lambda: gdn.replay(None, gdn.front_end(None, kr, g, b, out=out_k)[1], v, out[2], out[3],
                                              cu, want_o=False))
        alone, _ = timed(lambda: gdn.replay(None, out[1], v, out[2], out[3], cu, want_o=False))
        fused, _ = timed(lambda: gdn.replay_raw(None, kr, v, g, b, cu, want_o=False))
        extra = dict(state_only_replay=dict(prepared_inputs_ms=round(alone, 5), with_front_end_ms=round(both, 5),
                                            fused_front_end_ms=round(fused, 5)))
        # the 32768-token prefill with outputs from raw projections: the
        # front end then the replay, against gdn_replay_raw
        TP = 32768
        rp = workloads.generate_raw([TP], H=H, dk=d, dv=d, dtype="bf16", seed=8)
        qp, kp, gp, bp, vp = t(rp.q_raw), t(rp.k_raw), t(rp.g), t(rp.b), t(rp.v)
        del rp
        cup = torch.tensor([0, TP], dtype=torch.int32, device="cuda")
        outp = (torch.empty_like(qp), torch.empty_like(kp), torch.empty_like(gp), torch.empty_like(bp))
        op = torch.empty((TP, H, d), dtype=torch.float32, device="cuda")
        Sp = torch.empty((1, H, d, d), dtype=torch.float32, device="cuda")

        def two_calls():
            gdn.front_end(qp, kp, gp, bp, out=outp)
            gdn.replay(outp[0], outp[1], vp, outp[2], outp[3], cup, want_o=True, out=op, S_out=Sp)
        two, _ = timed(two_calls)
        fusedp, _ = timed(lambda: gdn.replay_raw(qp, kp, vp, gp, bp, cup, want_o=True, out=op, S_out=Sp))
        prepared, _ = timed(lambda: gdn.replay(outp[0], outp[1], vp, outp[2], outp[3], cup, want_o=True, out=op,
                                               S_out=Sp))
        extra["prefill_with_outputs"] = dict(n_tokens=TP, prepared_inputs_ms=round(prepared, 5),
                                             with_front_end_ms=round(two, 5), fused_front_end_ms=round(fusedp, 5))
    # q_raw, k_raw read and q, k written (bf16); g, b read and alpha, beta written (bf16)
    byt = T * H * (4 * d * 2 + 4 * 2)
    achieved = byt / (avg / 1e3) / 1e9
    line = dict(metric="GDN front end tokens·heads/s (normalised q, k and activated gates)",
                value=round(T * H / (wall / 1e3), 1), unit="tokens·heads/s", n_gpus=1, steps=args.steps,
                warmup=args.warmup, ms_per_step=round(wall, 5), higher_is_better=True, scaling="weak",
                vs_baseline=None, dtype="bf16", data="synthetic",
                config=dict(workload=FRONT_NAME, n_tokens=T, heads=H, dk=d, outputs="q,k,alpha,beta"),
                roofline=dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                              frac=round(achieved / HBM_PEAK_GBS, 4), traffic=measured_traffic(FRONT_NAME),
                              kernel="front_kernel", algorithmic_bytes=byt, kernel_ms_avg=round(avg, 5),
                              kernel_ms_min=round(mn, 5)), **extra)
    line["gpu_ms_per_step"] = round(avg, 5)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", type=int, default=3, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--o-bf16", action="store_true", help="write o in bf16 (workloads 2, 3)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB MiB (HBM counter calibration)")
    ap.add_argument("--summarize-counters", nargs=5, metavar=("STATS", "FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE"),
                    help="write profiles/ summaries from rocprofv3 output folders (no GPU needed)")
    ap.add_argument("--command", default="", help="with --summarize-counters: the command line profiled")
    ap.add_argument("--issue-counters", default=None, metavar="DIR",
                    help="with --summarize-counters: a --pmc run of the MFMA / issue counters (ISSUE_COUNTERS)")
    ap.add_argument("--cycle-counters", default=None, metavar="DIR",
                    help="with --summarize-counters: a --pmc run of the wave-cycle counters (CYCLE_COUNTERS)")
    ap.add_argument("--tail-curve", action="store_true",
                    help="only report the tail-replay state error against the replayed fraction")
    ap.add_argument("--decode", type=int, default=0, metavar="N",
                    help="only time single-token decode of N requests (H=32, d=128) from given states")
    ap.add_argument("--front-end", action="store_true",
                    help="only time the front end (normalised q, k and gates) on the tail-replay shape")
    ap.add_argument("--overlap", type=int, default=0, metavar="MIB",
                    help="only time a MIB pinned-host -> device copy beside tail replays (serial and overlapped)")
    ap.add_argument("--layers", type=int, default=3,
                    help="with --overlap: tail replays per copy (linear-attention layers of one group)")
    ap.add_argument("--scalar-ops", action="store_true",
                    help="only time scalar-decay chunk operators and their composition (64 x 512 tokens)")
    ap.add_argument("--with-replay", action="store_true",
                    help="with --front-end: also time a state-only replay with and without the front end")
    args = ap.parse_args()
    if args.summarize_counters:
        name = (("decode-%dx1-H32-d128-bf16" % args.decode) if args.decode else FRONT_NAME if args.front_end
                else SCALAR_NAME if args.scalar_ops else None)
        summarize_counters(args.workload, *args.summarize_counters, command=args.command, name=name,
                           mfma_dir=args.issue_counters, cycle_dir=args.cycle_counters)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the replay path is a single-GPU kernel library "
              "(heads and requests shard across GPUs without any exchange); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy:
        # also the practical ceiling of a streaming kernel: a device copy
        # (each byte read once and written once), timed with HIP events
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        print(json.dumps(dict(calibration="copy", bytes_read=n * 4, bytes_written=n * 4,
                              launches=args.warmup + args.steps, ms_per_copy=round(ms, 5),
                              read_plus_write_GBps=round(2 * n * 4 / (ms / 1e3) / 1e9, 1))))
        return

    import gated_deltanet_state_amd as gdn
    import workloads

    if args.tail_curve:
        tail_curve_report(gdn, torch, np)
        return
    if args.decode:
        decode_report(args, gdn, torch, np)
        return
    if args.front_end:
        front_end_report(args, gdn, torch, np)
        return
    if args.overlap:
        overlap_report(args, gdn, torch, np)
        return
    if args.scalar_ops:
        scalar_ops_report(args, gdn, torch, np)
        return

    wid = args.workload
    wdef = workloads.WORKLOADS[wid]
    inp = workloads.make_workload(wid)
    d = to_dev(inp, torch, np)
    H, dk, dv, T = inp.H, inp.dk, inp.dv, inp.n_tokens
    want_o = wid in (0, 2, 3)
    o_dtype = torch.bfloat16 if args.o_bf16 else torch.float32
    o_bytes = 2 if args.o_bf16 else 4
    stream = torch.cuda.current_stream()
    dev = torch.device("cuda:0")

    if wid == 4:
        cu_chunks = torch.from_numpy(workloads.chunk_bounds(T, wdef["chunk"])).cuda()
        n_chunks = cu_chunks.shape[0] - 1

        def launches():
            TC, SL = gdn.chunk_operator(d["k"], d["alpha"], d["beta"], cu_chunks, v=d["v"])
            return TC, SL
        # bytes of the chunk-operator kernel: k, v, alpha, beta read; T_C, S_local written
        byt = T * H * (dk + dv + 2) * 2 + n_chunks * H * (dk * dk + dv * dk) * 4
        fl = T * H * (2 * 64 * (2 * dk + dv) + 4 * dk * (dk + dv))
    else:
        o_buf = torch.empty((T, H, dv), dtype=o_dtype, device=dev) if want_o else None
        S_buf = torch.empty((inp.n_seqs, H, dv, dk), dtype=torch.float32, device=dev)

        def launches():
            return gdn.replay(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu"],
                              want_o=want_o, out=o_buf, S_out=S_buf)
        byt, fl = algorithmic(inp, want_o, o_bytes)

    for _ in range(args.warmup):
        res = launches()
    torch.cuda.synchronize()
    if wid == 4:
        TC, SL = res
        comp_out = torch.empty((H, dv, dk), dtype=torch.float32, device=dev)

    # ---- timed region: exactly K steps, no instrumentation, synchronised on both sides ----
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(args.steps):
        res = launches()
        if wid == 4:
            TC, SL = res
            gdn.compose(TC, SL, out=comp_out)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    step_ms = wall * 1e3 / args.steps

    # ---- then K steps with one event pair per dominant launch (the
    # roofline's per-launch durations; the event packets themselves cost a
    # few microseconds per step, so the throughput comes from the pass
    # above, which also leaves the device at its working clocks) ----
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    cstarts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    cends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        res = launches()
        ends[i].record(stream)
        if wid == 4:
            TC, SL = res
            cstarts[i].record(stream)
            gdn.compose(TC, SL, out=comp_out)
            cends[i].record(stream)
    torch.cuda.synchronize()
    instr_ms = (time.perf_counter() - t_wall) * 1e3 / args.steps
    kern_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    comp_ms = [s.elapsed_time(e) for s, e in zip(cstarts, cends)] if wid == 4 else []
    avg_kern = sum(kern_ms) / len(kern_ms)
    med_kern = sorted(kern_ms)[len(kern_ms) // 2]
    gpu_ms = avg_kern + (sum(comp_ms) / len(comp_ms) if comp_ms else 0.0)
    tok_heads = T * H
    value = tok_heads / (step_ms / 1e3)
    achieved = byt / (avg_kern / 1e3) / 1e9
    roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(achieved / HBM_PEAK_GBS, 4), traffic=measured_traffic(wdef["name"]),
                kernel=("chunk-operator call" if wid == 4 else "replay call (all kernels of one gdn_replay)"),
                algorithmic_bytes=byt, kernel_ms_avg=round(avg_kern, 5),
                kernel_ms_median=round(med_kern, 5), kernel_ms_min=round(min(kern_ms), 5),
                mfma_frac=round(fl / (avg_kern / 1e3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                algorithmic_flops=fl)
    config = dict(workload=wdef["name"], n_seqs=inp.n_seqs, n_tokens=T, heads=H, dk=dk, dv=dv,
                  outputs=("T_C,S_local" if wid == 4 else ("o,S_final" if want_o else "S_final")),
                  chunk=64)
    if wid == 4:
        config["compose_ms_avg"] = round(sum(comp_ms) / len(comp_ms), 5)
    line = dict(metric=METRIC, value=round(value, 1), unit="tokens·heads/s", n_gpus=1,
                steps=args.steps, warmup=args.warmup, ms_per_step=round(step_ms, 5),
                higher_is_better=True, scaling="weak", vs_baseline=None,
                dtype="bf16" if inp.dtype == "bf16" else "f32", data="synthetic",
                config=config, roofline=roof)
    line["gpu_ms_per_step"] = round(gpu_ms, 5)
    line["instrumented_ms_per_step"] = round(instr_ms, 5)
    if not args.no_cpu and wid != 4:
        line["cpu_baseline"] = cpu_baseline(inp, want_o, wid)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
