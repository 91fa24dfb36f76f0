"""Benchmark: compressed-KV decode attention GB/s (fraction of HBM peak) and
quantize-append Mtok/s on one MI355X.

Workload (default): batch 4, 8 KV heads, 32 query heads, head_dim 128,
context 32768, K 3-bit / V 4-bit (3.5 bits), 36 layers.  One step is, per
layer in order: quantize-append an 8192-token prefill chunk per sequence at
positions [24576, 32768), then one decode step attending over all 32768
positions.  Inputs are seeded synthetic fp16 (per-channel log-normal(0, 0.5)
scales with 1% x8 outlier channels; q N(0, 1)); every layer has its own
buffers.  The codebook build and the cache fill are set-up, outside the
timed region.

Prints one JSON line.  `value` is the decode GB/s over the algorithmic bytes
(every packed code word and norm of positions [0, 32768) for K and V, plus q
and out); quantize-append Mtok/s rides along in the same line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

WORKLOADS = {
    "c4_tq35_32k": dict(batch=4, kv_heads=8, q_heads=32, head_dim=128, tokens=32768, layers=36,
                        k=("packed", 3), v=("packed", 4), prefill=8192, dist="channel",
                        outlier_frac=0.01),
    # the small parity case: quantize all 256 positions, then one decode step
    "c1_tq35_d64_256": dict(batch=1, kv_heads=2, q_heads=4, head_dim=64, tokens=256, layers=1,
                            k=("packed", 3), v=("packed", 4), prefill=256, dist="iid", outlier_frac=0.0),
    "c2_sym4_4k": dict(batch=1, kv_heads=8, q_heads=32, head_dim=128, tokens=4096, layers=36,
                       k=("packed", 4), v=("packed", 4), prefill=0, dist="channel", outlier_frac=0.01),
    "c3_asym_16k": dict(batch=8, kv_heads=8, q_heads=32, head_dim=128, tokens=16384, layers=36,
                        k=("fp16", 0), v=("packed", 4), prefill=0, append=1, dist="channel",
                        outlier_frac=0.01),
    # the pages' int8 mode (per-token absmax) at the asymmetric workload's
    # shape, a comparison point on the same matrix-core kernel
    "c3_int8_16k": dict(batch=8, kv_heads=8, q_heads=32, head_dim=128, tokens=16384, layers=36,
                        k=("int8", 0), v=("int8", 0), prefill=0, append=1, dist="channel",
                        outlier_frac=0.01),
    # the pages' turbo3-asym mode (fp16 K, 3-bit V) at the same shape
    "c3_turbo3_asym_16k": dict(batch=8, kv_heads=8, q_heads=32, head_dim=128, tokens=16384, layers=36,
                               k=("fp16", 0), v=("packed", 3), prefill=0, append=1, dist="channel",
                               outlier_frac=0.01),
    # 2.5 bits (2-bit K, 3-bit V: the lower end of the pages' 2-4 bit range)
    # at the 32K shape
    "c4_tq25_32k": dict(batch=4, kv_heads=8, q_heads=32, head_dim=128, tokens=32768, layers=36,
                        k=("packed", 2), v=("packed", 3), prefill=8192, dist="channel",
                        outlier_frac=0.01),
    # the 32K workload's widths with 16 query heads per KV head (64 query
    # heads over 4 KV heads: head groups on the matrix cores)
    "c4_tq35_32k_g16": dict(batch=4, kv_heads=4, q_heads=64, head_dim=128, tokens=32768, layers=36,
                            k=("packed", 3), v=("packed", 4), prefill=8192, dist="channel",
                            outlier_frac=0.01),
    # the 32K workload with a peaked softmax (heavy-hitter keys at the first
    # 4 positions of every 512; the sparse-V comparison)
    "c4_tq35_32k_peaked": dict(batch=4, kv_heads=8, q_heads=32, head_dim=128, tokens=32768, layers=36,
                               k=("packed", 3), v=("packed", 4), prefill=8192, dist="channel",
                               outlier_frac=0.01, peaked=(512, 4, 9.0)),
    "c5_delegated_64k": dict(batch=16, kv_heads=4, q_heads=32, head_dim=128, tokens=65536, layers=48,
                             k=("fp16", 0), v=("delegated", 4), prefill=0, dist="channel",
                             outlier_frac=0.0, hot=256),
}


def side_bytes_per_token(mode: str, bits: int, d: int) -> int:
    if mode == "fp16":
        return 2 * d
    if mode == "int8":
        return d + 4
    return 4 * ((bits * d + 31) // 32) + 4


def decode_bytes(w) -> int:
    """Algorithmic bytes one decode launch must move."""
    d, T = w["head_dim"], w["tokens"]
    units = w["batch"] * w["kv_heads"]
    kb = side_bytes_per_token(w["k"][0], w["k"][1], d) * T
    if w["v"][0] == "delegated":
        hot = min(w.get("hot", 256), T)
        vb = side_bytes_per_token("packed", w["v"][1], d) * (T - hot) + 2 * d * hot
    else:
        vb = side_bytes_per_token(w["v"][0], w["v"][1], d) * T
    q = w["batch"] * w["q_heads"] * d * 2
    out = w["batch"] * w["q_heads"] * d * 4
    return units * (kb + vb) + q + out


def append_bytes(w, n_new: int) -> int:
    """Algorithmic bytes of one quantize-append launch (fp16 read + packed write)."""
    d = w["head_dim"]
    units = w["batch"] * w["kv_heads"]
    per = 0
    for mode, bits in (w["k"], w["v"]):
        per += 2 * d + (2 * d if mode == "fp16" else side_bytes_per_token(mode, bits, d))
    return units * n_new * per


def _oracle_side(w, mode, bits, x, R):
    """Storage of one side as the oracle builds it (set-up, not timed)."""
    import numpy as np

    import oracle
    d = w["head_dim"]
    if mode == "fp16":
        return ("fp16", x)
    if mode == "int8":
        return ("int8",) + oracle.int8_quantize(x)
    c, t = oracle.lloyd_max(d, bits)
    codes, n, _ = oracle.quantize(x, R, t)
    return ("packed", oracle.pack_codes(codes, bits), n.astype(np.float32), c, bits)


def _oracle_rows(w, st, R):
    """Rows the decode reads, rebuilt from the storage (timed)."""
    import oracle
    if st[0] == "fp16":
        return st[1].astype("float64")
    if st[0] == "int8":
        return oracle.int8_dequantize(st[1], st[2])
    _, words, n, c, bits = st
    return oracle.dequantize(oracle.unpack_codes(words, bits, w["head_dim"]), n, R, c)


def _oracle_decode_unit(w, seed):
    """One (batch, KV head) unit of one layer's decode through the oracle:
    storage built untimed, then unpack + dequantize + float64 attention timed.
    Returns (seconds, algorithmic bytes of the unit)."""
    import oracle
    import synth
    d, T, G = w["head_dim"], w["tokens"], w["q_heads"] // w["kv_heads"]
    R = oracle.rotation_matrix(0, d)
    k, v = synth.kv_numpy(seed, 1, 1, T, d, dist=w["dist"], outlier_frac=w["outlier_frac"])
    q = synth.q_numpy(seed, 1, G, d)
    ks, vs = _oracle_side(w, w["k"][0], w["k"][1], k, R), _oracle_side(w, w["v"][0], w["v"][1], v, R)
    t0 = time.perf_counter()
    oracle.decode_attention(q, _oracle_rows(w, ks, R), _oracle_rows(w, vs, R))
    dt = time.perf_counter() - t0
    nbytes = (side_bytes_per_token(w["k"][0], w["k"][1], d) + side_bytes_per_token(w["v"][0], w["v"][1], d)) * T
    return dt, nbytes


def _pool_worker(args):
    """All-cores leg: one unit per process with single-threaded BLAS; the
    processes start their timed part together (barrier)."""
    w, seed = args
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        _oracle_decode_unit(w, seed + 50000)  # warm the imports and caches (untimed)
        _POOL_BARRIER.wait()
        return _oracle_decode_unit(w, seed)


def _pool_init(barrier):
    global _POOL_BARRIER
    _POOL_BARRIER = barrier


def cpu_baseline(w, budget_s: float = 8.0, max_workers: int = 16):
    """Time the oracle (float64 NumPy, as it stands) on bounded samples of the
    workload on this host's cores: the decode with one core (BLAS pinned to
    one thread) over whole (batch, KV head) units until ~budget_s, the decode
    with all cores (one unit per process, up to max_workers processes, the
    box's CPU share), and the prefill quantize-append (norm, rotation,
    threshold count, packing) of one unit's new rows for K and V."""
    import multiprocessing as mp
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import synth

    nproc = os.cpu_count() or 1
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    d, T = w["head_dim"], w["tokens"]
    total_units = w["batch"] * w["kv_heads"]

    # one core
    units, spent, nbytes = 0, 0.0, 0
    with threadpool_limits(1):
        while spent < budget_s and units < total_units:
            dt, nb = _oracle_decode_unit(w, 1000 + units)
            spent, nbytes, units = spent + dt, nbytes + nb, units + 1
    one = {"value": nbytes / spent / 1e9, "unit": "GB/s", "cores": 1,
           "sample": f"{units} of {total_units} (batch, KV head) units of one layer's decode at context {T} "
                     f"(unpack + dequantize + float64 attention), {spent:.1f} s"}

    # all cores: one unit per process, timed together
    workers = max(1, min(nproc, max_workers, total_units))
    barrier = mp.get_context("fork").Barrier(workers)
    with mp.get_context("fork").Pool(workers, initializer=_pool_init, initargs=(barrier,)) as pool:
        res = pool.map(_pool_worker, [(w, 2000 + i) for i in range(workers)])
    wall = max(r[0] for r in res)
    allc = {"value": sum(r[1] for r in res) / wall / 1e9, "unit": "GB/s", "cores": workers,
            "sample": f"{workers} (batch, KV head) units of one layer's decode at context {T}, one per process "
                      f"(BLAS single-threaded), timed together: {wall:.1f} s"}

    # prefill quantize-append: one unit's new rows of K and V
    qa = None
    n_new = w.get("prefill", 0) or w.get("append", 0)
    if n_new:
        R = oracle.rotation_matrix(0, d)
        k, v = synth.kv_numpy(3000, 1, 1, n_new, d, dist=w["dist"], outlier_frac=w["outlier_frac"])
        with threadpool_limits(1):
            t0 = time.perf_counter()
            for (mode, bits), x in ((w["k"], k), (w["v"], v)):
                if mode in ("packed", "delegated"):
                    _, th = oracle.lloyd_max(d, bits)
                    codes, n, _ = oracle.quantize(x, R, th)
                    oracle.pack_codes(codes, bits)
                    n.astype(np.float32)
                elif mode == "int8":
                    oracle.int8_quantize(x)
            dt = time.perf_counter() - t0
        # positions per second with every KV head of a sequence (the metric's unit)
        qa = {"value": n_new / (dt * w["kv_heads"]) / 1e6, "unit": "Mtok/s", "cores": 1,
              "sample": f"one (batch, KV head) unit's {n_new} new rows of K and V quantized and packed, "
                        f"{dt:.2f} s, scaled to {w['kv_heads']} KV heads per position"}
    out = {"value": allc["value"], "unit": "GB/s", "cores": workers, "kind": "oracle",
           "sample": allc["sample"], "one_core": one, "all_cores": allc, "nproc": nproc, "cpu_model": model}
    if qa:
        out["quantize_append"] = qa
    return out


# the decode kernels whose counters can be recorded, by name prefix, with the
# source each one is built from
DECODE_SOURCES = {
    "decode_mfma": os.path.join(ROOT, "compressed_decode_attention_append_amd", "csrc", "decode_mfma.hip"),
    "decode_split": os.path.join(ROOT, "compressed_decode_attention_append_amd", "csrc", "decode_ref.hip"),
}
DECODE_SOURCE = DECODE_SOURCES["decode_mfma"]


def source_digest(path=DECODE_SOURCE) -> str:
    """sha256 of the kernel's code: the source with its comments removed and
    its whitespace collapsed, so that editing a comment does not void the
    counters recorded for the kernel."""
    import hashlib
    import re
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()


def traffic_key(workload: str, sparse_v: float = 0.0) -> str:
    """Name under which a decode's byte counters are recorded: the workload,
    and the sparse-V threshold when one is set (a skip changes the bytes)."""
    return f"{workload}_sparse_v{sparse_v:g}" if sparse_v else workload


def traffic_file(workload: str, kernel: str = "decode_mfma") -> str:
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.txt")


def recorded_traffic(workload: str):
    """HBM bytes per launch of the workload's decode kernel from the committed
    counter summary, or None when there is none or the kernel's source
    changed since it was taken (or a decode variant is forced through the
    environment, so the recorded kernel may not be the one that runs)."""
    if os.environ.get("TQ_DECODE_VARIANT"):
        return None
    for kernel, src in DECODE_SOURCES.items():
        path = traffic_file(workload, kernel)
        if not os.path.exists(path):
            continue
        fields = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("source_sha256") != source_digest(src):
            return None
        try:
            return int(float(fields["traffic_bytes_per_launch"]))
        except (KeyError, ValueError):
            return None
    return None


def counter_summary(fetch_csv: str, write_csv: str, workload: str, copy_mib: int, cmds: list,
                    append_last: int = 0):
    """Summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch) of `bench.py --copy-mib N`: the plain copy kernel of known size
    calibrates each counter, the decode kernel's per-launch HBM bytes follow.
    With append_last > 0, the quantize-append kernel's bytes too, over its
    last append_last dispatches (the step's appends, not the cache fill)."""
    import csv
    import collections

    def read(path, counter, last_of=None, last=0):
        acc = collections.defaultdict(list)
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    acc[r["Kernel_Name"]].append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
        lastid = {}
        for k in acc:
            acc[k].sort()
            lastid[k] = acc[k][-1][0]
            if last_of and last_of in k and last:
                acc[k] = acc[k][-last:]
        return ({k: sum(x[1] for x in v) / len(v) for k, v in acc.items()},
                {k: len(v) for k, v in acc.items()}, lastid)

    fetch, nf, last_f = read(fetch_csv, "FETCH_SIZE", "quantize", append_last)
    write, nw, _ = read(write_csv, "WRITE_SIZE", "quantize", append_last)
    copy_name = next(k for k in fetch if "neg_kernel" in k)
    dec_name = next(k for k in fetch if "decode_mfma_kernel" in k or "decode_split_kernel" in k)
    src = DECODE_SOURCES["decode_mfma" if "decode_mfma_kernel" in dec_name else "decode_split"]
    kib = copy_mib * 1024.0
    f_fetch = kib / fetch[copy_name]
    f_write = kib / write[copy_name]
    w = WORKLOADS[workload]
    traffic = (fetch[dec_name] * f_fetch + write[dec_name] * f_write) * 1024.0
    short = dec_name.replace("void tq::(anonymous namespace)::", "").split("(tq::")[0]
    out = [f"# rocprofv3 hardware byte counters: {short}, workload {workload}",
           "# commands (from the repository root):"]
    out += [f"#   {c}" for c in cmds]
    out += ["#",
            f"# calibration: a plain copy of {copy_mib} MiB (torch.neg, reads and writes {copy_mib} MiB)",
            f"#   FETCH_SIZE {fetch[copy_name]:.1f} KiB -> factor {f_fetch:.4f}; "
            f"WRITE_SIZE {write[copy_name]:.1f} KiB -> factor {f_write:.4f}",
            f"# {short}: {nf[dec_name]} dispatches; FETCH_SIZE {fetch[dec_name]:.1f} KiB, "
            f"WRITE_SIZE {write[dec_name]:.1f} KiB per dispatch (raw)",
            f"kernel: {short}",
            f"workload: {workload}",
            f"source: {os.path.relpath(src, ROOT)}",
            f"source_sha256: {source_digest(src)}",
            f"fetch_bytes_per_launch: {fetch[dec_name] * f_fetch * 1024.0:.0f}",
            f"write_bytes_per_launch: {write[dec_name] * f_write * 1024.0:.0f}",
            f"traffic_bytes_per_launch: {traffic:.0f}",
            f"algorithmic_bytes_per_launch: {decode_bytes(w)}",
            f"traffic_over_algorithmic: {traffic / decode_bytes(w):.4f}"]
    n_new = w.get("prefill", 0) or w.get("append", 0)
    # the encoder of the step's appends: the quantize kernel dispatched last
    # (the cache fill may use the other encoder)
    q_names = [k for k in fetch if "quantize" in k and k in write]
    q_name = max(q_names, key=lambda k: last_f[k]) if q_names else None
    if append_last and n_new and q_name:
        qshort = q_name.replace("void ", "").replace("tq::(anonymous namespace)::", "").split("(tq::")[0]
        q_traffic = (fetch[q_name] * f_fetch + write[q_name] * f_write) * 1024.0
        ab = append_bytes(w, n_new)
        out += ["#",
                f"# {qshort}: its last {nf[q_name]} dispatches (the appends of {n_new} positions per "
                f"sequence); FETCH_SIZE {fetch[q_name]:.1f} KiB, WRITE_SIZE {write[q_name]:.1f} KiB per "
                "dispatch (raw)",
                f"append_kernel: {qshort}",
                f"append_fetch_bytes_per_launch: {fetch[q_name] * f_fetch * 1024.0:.0f}",
                f"append_write_bytes_per_launch: {write[q_name] * f_write * 1024.0:.0f}",
                f"append_traffic_bytes_per_launch: {q_traffic:.0f}",
                f"append_algorithmic_bytes_per_launch: {ab}",
                f"append_traffic_over_algorithmic: {q_traffic / ab:.4f}"]
    return "\n".join(out) + "\n"


def stats_summary(stats_csv: str, workload: str, cmds: list):
    """Format a rocprofv3 --kernel-trace --stats kernel table (this library's
    kernels only)."""
    import csv
    rows = []
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            name = r["Name"]
            if "tq::" not in name:
                continue
            short = name.replace("void ", "").replace("tq::(anonymous namespace)::", "").split("(tq::")[0]
            rows.append((short, int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3))
    w = WORKLOADS[workload]
    out = [f"# rocprofv3 kernel statistics, workload {workload}: batch {w['batch']}, {w['kv_heads']} KV heads, "
           f"{w['q_heads']} query heads, head_dim {w['head_dim']}, context {w['tokens']}, "
           f"K {w['k'][0]}{w['k'][1] or ''}, V {w['v'][0]}{w['v'][1] or ''}",
           "# commands (from the repository root):"]
    out += [f"#   {c}" for c in cmds]
    out += [f"# decode algorithmic bytes per launch: {decode_bytes(w)}",
            "", f"{'kernel':44s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    for short, calls, avg, mn, mx in sorted(rows):
        out.append(f"{short:44s} {calls:6d} {avg:9.2f} {mn:9.2f} {mx:9.2f}")
        if "decode_mfma" in short or "decode_split" in short:
            out.append(f"#   -> {decode_bytes(w) / (avg * 1e-6) / 1e9:.1f} GB/s over the algorithmic bytes")
    return "\n".join(out) + "\n"


# per-dispatch counters the --pmc-summary mode explains, and the ratios it derives
PMC_RATIOS = [
    ("valu issue share of wave time", "SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES"),
    ("lds issue share of wave time", "SQ_ACTIVE_INST_LDS", "SQ_WAVE_CYCLES"),
    ("share of wave time waiting on any instruction", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
    ("share of wave time waiting on LDS", "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES"),
    ("lds bank-conflict cycles per LDS issue cycle", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS"),
]


def pmc_summary(csvs: list, workload: str, cmds: list, title: str):
    """Summarise rocprofv3 --pmc runs (any counters, one or more CSV files)
    of this script: each counter's average per dispatch for each of the
    library's kernels, divided by the workload's (batch, KV head, 32-position)
    chunks for the decode kernels, and a few ratios of cycle counters."""
    import collections
    import csv
    w = WORKLOADS[workload]
    chunks = w["batch"] * w["kv_heads"] * w["tokens"] // 32
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    # ratios only between counters of the same file (one profiled run)
    ratio = collections.defaultdict(lambda: collections.defaultdict(float))
    for path in csvs:
        one = collections.defaultdict(lambda: collections.defaultdict(float))
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"]
                if "tq::" not in name:
                    continue
                short = name.replace("void ", "").replace("tq::(anonymous namespace)::", "").split("(tq::")[0]
                acc[short][r["Counter_Name"]].append(float(r["Counter_Value"]))
                one[short][r["Counter_Name"]] += float(r["Counter_Value"])
        for short, cs in one.items():
            for _, a, b in PMC_RATIOS:
                if a in cs and b in cs:
                    ratio[short][a] += cs[a]
                    ratio[short][(a, b)] += cs[b]
    out = [f"# rocprofv3 hardware counters ({title}), workload {workload}: batch {w['batch']}, "
           f"{w['kv_heads']} KV heads, {w['q_heads']} query heads, head_dim {w['head_dim']}, context {w['tokens']}",
           "# commands (from the repository root):"]
    out += [f"#   {c}" for c in cmds]
    out += [f"# values are averages per dispatch; 'per chunk' divides by the {chunks} (batch, KV head, "
            "32-position) chunks of one decode", ""]
    for short in sorted(acc):
        cs = acc[short]
        n = max(len(v) for v in cs.values())
        out.append(f"kernel: {short} ({n} dispatches)")
        is_decode = "decode" in short
        for c in sorted(cs):
            avg = sum(cs[c]) / len(cs[c])
            extra = f"   per chunk {avg / chunks:10.2f}" if is_decode and c.startswith("SQ_INSTS") else ""
            out.append(f"  {c:32s} {avg:18.1f}{extra}")
        for label, a, b in PMC_RATIOS:
            num, den = ratio[short].get(a, 0.0), ratio[short].get((a, b), 0.0)
            if den > 0:
                out.append(f"  ratio {a} / {b} = {num / den:.4f}   ({label}; both from the same runs)")
        out.append("")
    return "\n".join(out) + "\n"


def trace_summary(trace_csv: str, workload: str, last: int, cmds: list, n_new: int = 0):
    """Per-kernel durations from a rocprofv3 --kernel-trace CSV of this
    script, over each kernel's last `last` dispatches only (the timed steps:
    steps x layers), so the cache fill and the warm-up do not enter the
    averages; with the decode and quantize-append throughput they imply."""
    import collections
    import csv
    w = dict(WORKLOADS[workload])
    per = collections.defaultdict(list)
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if "tq::" not in name:
                continue
            short = name.replace("void ", "").replace("tq::(anonymous namespace)::", "").split("(tq::")[0]
            per[short].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    out = [f"# rocprofv3 kernel trace, workload {workload}: batch {w['batch']}, {w['kv_heads']} KV heads, "
           f"{w['q_heads']} query heads, head_dim {w['head_dim']}, context {w['tokens']}, "
           f"K {w['k'][0]}{w['k'][1] or ''}, V {w['v'][0]}{w['v'][1] or ''}",
           "# commands (from the repository root):"]
    out += [f"#   {c}" for c in cmds]
    out += [f"# each kernel's last {last} dispatches (the timed steps); durations in microseconds",
            f"# decode algorithmic bytes per launch: {decode_bytes(w)}"]
    if n_new:
        out.append(f"# quantize-append: {n_new} new positions per sequence per launch, "
                   f"algorithmic bytes per launch {append_bytes(w, n_new)}")
    out += ["", f"{'kernel':44s} {'calls':>6s} {'avg_us':>9s} {'median':>9s} {'min_us':>9s} {'max_us':>9s}"]
    for short in sorted(per):
        d = [x[1] / 1e3 for x in sorted(per[short])[-last:]]
        d_sorted = sorted(d)
        avg = sum(d) / len(d)
        out.append(f"{short:44s} {len(d):6d} {avg:9.2f} {d_sorted[len(d) // 2]:9.2f} {d_sorted[0]:9.2f} "
                   f"{d_sorted[-1]:9.2f}")
        if "decode_mfma" in short or "decode_split" in short:
            out.append(f"#   -> {decode_bytes(w) / (avg * 1e-6) / 1e9:.1f} GB/s over the algorithmic bytes, "
                       f"{decode_bytes(w) / (avg * 1e-6) / 1e9 / HBM_PEAK_GBS:.4f} of {HBM_PEAK_GBS:.0f} GB/s")
        if n_new and "quantize" in short:
            out.append(f"#   -> {w['batch'] * n_new / (avg * 1e-6) / 1e6:.1f} Mtok/s, "
                       f"{append_bytes(w, n_new) / (avg * 1e-6) / 1e9:.1f} GB/s over the algorithmic bytes")
        elif "quantize" in short:
            out.append("#   (the cache fill before the timed steps: this workload's step appends nothing)")
    return "\n".join(out) + "\n"


def attainable_read_gbs(stream, nbytes=4 << 30, reps=10) -> float:
    """HBM read bandwidth of the library's streaming-read probe over a fresh
    `nbytes` buffer (the attainable ceiling the decode can be read against;
    the roofline itself stays the published peak)."""
    import torch
    import compressed_decode_attention_append_amd as tq
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda:0")
    with torch.cuda.stream(stream):
        buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    for _ in range(2):
        tq.read_probe(buf, sink, stream=stream)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        tq.read_probe(buf, sink, stream=stream)
    b.record(stream)
    b.synchronize()
    gbs = nbytes * reps / (a.elapsed_time(b) / 1e3) / 1e9
    del buf
    return gbs


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c4_tq35_32k", choices=sorted(WORKLOADS))
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (profiling only)")
    ap.add_argument("--tokens", type=int, default=0, help="override the context length (profiling only)")
    ap.add_argument("--block-size", type=int, default=0,
                    help="paged storage with blocks of this many positions (a multiple of 32), "
                         "each layer's blocks in a random order; 0 = contiguous")
    ap.add_argument("--sparse-v", type=float, default=0.0,
                    help="decode with tq_decode_attention_sparse at this weight threshold "
                         "(an approximation; 0 = the exact decode)")
    ap.add_argument("--fused-append", action="store_true",
                    help="workloads that append one position a step: each layer's append and decode "
                         "in one tq_decode_attention_append call (timed as the decode group)")
    ap.add_argument("--splits", type=int, default=0,
                    help="context splits per (batch, KV head); 0 = the library's choice")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size "
                         "calibration kernel for hardware byte counters)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--counter-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                         "script with --copy-mib and print the traffic summary; runs nothing")
    ap.add_argument("--command", action="append", default=[],
                    help="with --counter-summary: a command line to record in the summary")
    ap.add_argument("--stats-summary", metavar="KERNEL_STATS_CSV",
                    help="format a rocprofv3 --stats kernel table of this script's run; runs nothing")
    ap.add_argument("--pmc-summary", nargs="+", metavar="COUNTER_CSV",
                    help="summarise rocprofv3 --pmc runs (any counters) of this script; runs nothing")
    ap.add_argument("--title", default="", help="with --pmc-summary: what the counters were taken of")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="per-kernel durations of the timed steps (--steps x layers last dispatches) from a "
                         "rocprofv3 --kernel-trace CSV of this script; runs nothing")
    args = ap.parse_args()
    if args.trace_summary:
        w = WORKLOADS[args.workload]
        layers = args.layers or w["layers"]
        sys.stdout.write(trace_summary(args.trace_summary, args.workload, args.steps * layers, args.command,
                                       w.get("prefill", 0) or w.get("append", 0)))
        return
    if args.pmc_summary:
        sys.stdout.write(pmc_summary(args.pmc_summary, args.workload, args.command, args.title))
        return
    if args.stats_summary:
        sys.stdout.write(stats_summary(args.stats_summary, args.workload, args.command))
        return
    if args.counter_summary:
        w = WORKLOADS[args.workload]
        sys.stdout.write(counter_summary(args.counter_summary[0], args.counter_summary[1], args.workload,
                                         args.copy_mib or 256, args.command,
                                         (args.warmup + args.steps) * (args.layers or w["layers"])))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}), flush=True)
        sys.exit(2)

    import torch

    import compressed_decode_attention_append_amd as tq
    import synth

    w = dict(WORKLOADS[args.workload])
    if args.layers:
        w["layers"] = args.layers
    if args.tokens:
        w["tokens"] = args.tokens
        w["prefill"] = min(w.get("prefill", 0), args.tokens)
    # the oracle's CPU baseline runs first, before anything touches the GPU
    # (its all-cores leg forks worker processes)
    cpu = None if args.no_cpu_baseline else cpu_baseline(w)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    B, Hkv, Hq, d, T, Lyr = w["batch"], w["kv_heads"], w["q_heads"], w["head_dim"], w["tokens"], w["layers"]
    pre = w.get("prefill", 0)
    app = w.get("append", 0)
    n_new = pre or app
    base = T - n_new if n_new else T

    if args.fused_append and (n_new != 1 or args.sparse_v):
        print(json.dumps({"error": "--fused-append needs a one-position append workload and the exact decode"}),
              flush=True)
        sys.exit(2)
    kspec = tq.SideSpec(w["k"][0], w["k"][1])
    vspec = tq.SideSpec(w["v"][0], w["v"][1], w.get("hot", 256))
    layers = []
    t_fill = time.time()
    bsz = args.block_size
    if bsz and (bsz % 32 or T % bsz):
        print(json.dumps({"error": "--block-size must be a multiple of 32 dividing the context"}), flush=True)
        sys.exit(2)
    for li in range(Lyr):
        paging = {}
        if bsz:
            nb = B * (T // bsz)
            perm = torch.randperm(nb, generator=torch.Generator().manual_seed(li)).to(torch.int32)
            paging = dict(block_table=perm.reshape(B, T // bsz), block_size=bsz, num_blocks=nb)
        cache = tq.TQCache(B, Hkv, d, T, kspec, vspec, seed=0, device=dev, **paging)
        q = synth.q_torch(31 + li, B, Hq, d, device=dev)
        peak = w.get("peaked")
        # fill positions [0, base) with the layer's own synthetic rows
        chunk = 4096
        for s in range(0, base, chunk):
            n = min(chunk, base - s)
            k, v = synth.kv_torch(7919 * li + s, B, Hkv, n, d, dist=w["dist"],
                                  outlier_frac=w["outlier_frac"], device=dev)
            if peak:
                synth.peak_keys_torch(k, q, s, *peak)
            cache.quantize_append(k, v, s)
            del k, v
        if n_new:
            kn, vn = synth.kv_torch(104729 + li, B, Hkv, n_new, d, dist=w["dist"],
                                    outlier_frac=w["outlier_frac"], device=dev)
            if peak:
                synth.peak_keys_torch(kn, q, base, *peak)
        else:
            kn = vn = None
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        ws = cache.workspace(Hq, T, args.splits)
        layers.append((cache, kn, vn, q, out, ws))
    torch.cuda.synchronize()
    t_fill = time.time() - t_fill
    print(f"# filled {Lyr} layers in {t_fill:.1f} s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    if args.copy_mib:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)  # reads and writes copy_mib MiB
        torch.cuda.synchronize()
        del src, dst

    # One step = quantize-append for every layer, then decode for every
    # layer.  The layers hold independent synthetic data, so grouping the
    # launches by kind changes no work; it lets one event pair per group time
    # the back-to-back launches of each kernel (per-launch average = group
    # time / layers) without an event between every two kernels.
    # A step whose working set fits the caches (the 256 MB Infinity Cache and
    # the L2s) would be served from them on the next step: such workloads
    # stream-read a 1 GiB scratch buffer (the library's read probe) before
    # every step, outside the event pairs that time the kernels (ms_per_step
    # includes it).  A read leaves the caches holding clean lines; a write
    # flush would leave dirty ones, whose write-back then lands inside the
    # timed decodes.
    working = Lyr * (decode_bytes(w) + (append_bytes(w, n_new) if n_new else 0))
    flush = torch.empty(1 << 28, dtype=torch.int32, device=dev) if working < (1 << 30) else None
    if flush is not None:
        flush.fill_(1)
        flush_sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def step(record):
        if flush is not None:
            tq.read_probe(flush, flush_sink, stream=stream)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)] if record is not None else None
        if ev:
            ev[0].record(stream)
        if n_new and not args.fused_append:
            for cache, kn, vn, q, out, ws in layers:
                cache.quantize_append(kn, vn, base, stream=stream)
        if ev:
            ev[1].record(stream)
        for cache, kn, vn, q, out, ws in layers:
            if args.fused_append:
                cache.decode_attention_append(kn, vn, base, q, T, n_splits=args.splits, out=out, workspace=ws,
                                              stream=stream)
            else:
                cache.decode_attention(q, T, n_splits=args.splits, out=out, workspace=ws, stream=stream,
                                       sparse_v=args.sparse_v)
        if ev:
            ev[2].record(stream)
            record.append(ev)

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    rec = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(rec)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    attain = attainable_read_gbs(stream)

    dec_ms = sum(e[1].elapsed_time(e[2]) for e in rec)
    app_ms = sum(e[0].elapsed_time(e[1]) for e in rec)
    dbytes = decode_bytes(w)
    dec_avg_s = dec_ms / (len(rec) * Lyr) / 1e3
    dec_gbs = dbytes / dec_avg_s / 1e9
    res = {
        "metric": "compressed-KV decode attention GB/s (% of HBM peak) + quantize-append Mtok/s",
        "value": round(dec_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32+fp16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "kv_heads": Hkv, "q_heads": Hq,
                   "head_dim": d, "context": T, "layers": Lyr,
                   "k": f"{w['k'][0]}{w['k'][1] or ''}", "v": f"{w['v'][0]}{w['v'][1] or ''}",
                   "append_per_layer": n_new, "fused_append": bool(args.fused_append),
                   "block_size": bsz, "sparse_v": args.sparse_v,
                   "cache_flush_gib_per_step": 1 if flush is not None else 0},
        "hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4),
        "decode_us_per_layer": round(dec_avg_s * 1e6, 2),
        "decode_bytes_per_layer": dbytes,
        "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     # counters were taken on contiguous caches
                     "traffic": None if (bsz or args.fused_append)
                     else recorded_traffic(traffic_key(args.workload, args.sparse_v))},
        # context for the roofline: what a plain streaming-read kernel attains
        "attainable_read": {"gbs": round(attain, 1), "bytes": 4 << 30,
                            "kernel": "tq_read_probe: 16-byte loads, 256 blocks of 768 threads",
                            "decode_frac": round(dec_gbs / attain, 4)},
    }
    if n_new and not args.fused_append:
        app_avg_s = app_ms / (len(rec) * Lyr) / 1e3
        res["quantize_append_mtok_s"] = round(B * n_new / app_avg_s / 1e6, 2)
        res["quantize_append_us_per_layer"] = round(app_avg_s * 1e6, 2)
        res["quantize_append_gbs"] = round(append_bytes(w, n_new) / app_avg_s / 1e9, 1)
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
