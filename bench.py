#!/usr/bin/env python3
"""Benchmark of the fused rotate + int4 KV-cache quantizer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = quantize K and V, then dequantize K and V, of the Qwen3-8B-shaped
bulk-prefill cache: [36 layers, 262,144 tokens (8 x 32,768), 8 KV heads, 128]
fp16 per tensor, group size 32 (151 M head vectors per tensor, 49.5 GB of
algorithmic traffic per tensor and direction).  Inputs are seeded synthetic
(N(0,1) x per-(layer, head, channel) LogNormal(0,1) scales) and resident in
HBM before the timed region.  The product-VQ encode/decode of the VecInfer-
shaped key cache ([36, 8192, 8, 128], 4096-centroid per-head codebooks) is
timed in the same run and reported under "vq".

Prints ONE JSON line.  `value` is the algorithmic GB/s of a whole step
(bytes the definition must move / wall time of the step);
`roofline` grades the dominant kernel (quantize) with per-launch HIP-event
timings on the stream it runs on; `cpu_baseline` times the fp64 oracle on a
bounded sample on the host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused rotate+int4 quantize GB/s (% of HBM peak) and ns/vector at D=128"
HBM_PEAK_GBPS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_quantize_d128_g32_qwen3-8b.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_vq_encode_vecinfer.json")
# the VQ encoder and its launch configuration
VQ_SOURCES = ["kv_cache_quantization_quantize_amd/csrc/kvq_vq.hip",
              "kv_cache_quantization_quantize_amd/csrc/kvq_device.h",
              "kv_cache_quantization_quantize_amd/csrc/kvq_api.cpp"]
MFMA_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
                 "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]
# MI355X: 8 XCDs of 32 CUs, 4 SIMDs per CU
N_XCD, N_CU, SIMD_PER_CU = 8, 256, 4
# the quantize kernel and its launch configuration (items per wavefront)
KERNEL_SOURCES = ["kv_cache_quantization_quantize_amd/csrc/kvq_int4.hip",
                  "kv_cache_quantization_quantize_amd/csrc/kvq_device.h",
                  "kv_cache_quantization_quantize_amd/csrc/kvq_api.cpp"]


def bytes_per_vector(D: int, G: int) -> int:
    """Algorithmic bytes one quantize or dequantize of a vector must move:
    fp16 vector + packed codes + fp16 scales (lambda/signs amortise to < 0.1%)."""
    return 2 * D + D // 2 + 2 * (D // G)


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def spread(ms):
    """Median, minimum and maximum of a list of launch times (ms)."""
    srt = sorted(ms)
    n = len(srt)
    med = srt[n // 2] if n % 2 else 0.5 * (srt[n // 2 - 1] + srt[n // 2])
    return {"median_ms": round(med, 4), "min_ms": round(srt[0], 4), "max_ms": round(srt[-1], 4)}


def ingest_mfma(csv_path, out_path=None):
    """Turn a rocprofv3 `--pmc <MFMA_COUNTERS>` run of `bench.py --parts vq`
    into per-kernel utilisation figures and write MFMA_FILE.

    rocprofv3 sums each counter over its dimensions (XCDs, shader engines,
    SIMDs), so: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8
    XCDs x 1024 SIMDs) (the MfmaUtil definition with the per-XCD maximum
    taken as the per-XCD mean); VALU busy = SQ_ACTIVE_INST_VALU / (256 CUs x
    GRBM_GUI_ACTIVE / 8) (VALUBusy); executed fp16 MFMA flop =
    SQ_INSTS_VALU_MFMA_MOPS_F16 x 512; clock = GRBM_GUI_ACTIVE / 8 over the
    dispatch's duration."""
    import csv
    vals, dur = {}, {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"].split("(")[0].replace("void ", "")
            if not name.startswith("kvq::"):
                continue
            vals.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
            dur.setdefault(name, {})[r["Dispatch_Id"]] = d
    out = {"source_hash": kernel_source_hash(VQ_SOURCES), "counters": MFMA_COUNTERS,
           "workload": "vecinfer-shaped keys [36, 8192, 8, 128], 4096-centroid fp16 codebooks per head "
                       "(u16 indices); values with 256-centroid codebooks (u8 indices)", "kernels": {}}
    for name, c in vals.items():
        if not all(k in c for k in MFMA_COUNTERS):
            continue
        m = {k: sum(v) / len(v) for k, v in c.items()}
        cyc = m["GRBM_GUI_ACTIVE"] / N_XCD
        secs = sum(dur[name].values()) / len(dur[name])
        k = {"dispatches": len(c["GRBM_GUI_ACTIVE"]), "avg_s": secs,
             "clock_GHz": round(cyc / secs / 1e9, 3) if secs > 0 else None,
             "mfma_busy": round(m["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * N_CU * SIMD_PER_CU), 4),
             "valu_busy": round(m["SQ_ACTIVE_INST_VALU"] / (cyc * N_CU), 4),
             "mfma_instructions": int(m["SQ_INSTS_MFMA"]), "valu_instructions": int(m["SQ_INSTS_VALU"]),
             "executed_fp16_mfma_flop": m["SQ_INSTS_VALU_MFMA_MOPS_F16"] * 512}
        if secs > 0:
            k["executed_fp16_TFLOP_per_s"] = round(k["executed_fp16_mfma_flop"] / secs / 1e12, 2)
        out["kernels"][name] = k
    with open(out_path or MFMA_FILE, "w") as f:
        json.dump(out, f, indent=1)
    return out


def load_mfma(path=None):
    """The committed MFMA counter summary, or None if absent or taken on
    different sources."""
    try:
        with open(path or MFMA_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash(VQ_SOURCES):
        return None
    return t


def load_traffic(per_launch_alg_bytes):
    """HBM bytes per quantize launch from the committed rocprofv3 counter
    summary, or None if absent or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    return t.get("traffic_bytes_per_launch")


def _counter_means(path, counter):
    """Per-kernel mean of one rocprofv3 counter (KiB per dispatch) and the
    per-dispatch values, from a `--pmc <counter> --output-format csv` run."""
    import csv
    vals = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                vals.setdefault(r["Kernel_Name"].split("(")[0].replace("void ", ""), []).append(
                    float(r["Counter_Value"]))
    return vals


def ingest_counters(fetch_csv, write_csv, copy_bytes):
    """Turn the FETCH_SIZE and WRITE_SIZE counter runs of this benchmark into
    HBM bytes per launch for each timed kernel and write TRAFFIC_FILE.

    Both counters are scaled by what they read for the plain-copy reference
    that the same runs time (a device-to-device copy of copy_bytes, which
    must read and write exactly copy_bytes), so that the result is in real
    bytes."""
    fe, wr = _counter_means(fetch_csv, "FETCH_SIZE"), _counter_means(write_csv, "WRITE_SIZE")
    kib = copy_bytes / 1024
    cw = [v for v in wr.get("__amd_rocclr_copyBuffer", []) if abs(v - kib) < 1]
    if not cw:
        raise SystemExit("no %d-byte reference copy in %s" % (copy_bytes, write_csv))
    cf = sorted(fe["__amd_rocclr_copyBuffer"])[-len(cw):]
    f_scale, w_scale = kib / (sum(cf) / len(cf)), kib / (sum(cw) / len(cw))
    L, T, H, D, G = 36, 262144, 8, 128, 32
    nv = L * T * H
    B, R = 8, 4
    att = 2 * L * T * H * (D // 2 + 2 * (D // G)) + 2 * (L * B) * H * R * D * 2
    nk = 36 * 8192 * 8
    kernels = {
        "quantize": ("kvq::quantize_kernel<128, 32, true, 4, false, false>", nv * bytes_per_vector(D, G)),
        "dequantize": ("kvq::dequantize_kernel<128, 32, true, 4, false, false>", nv * bytes_per_vector(D, G)),
        "quantize_int8": ("kvq::quantize_kernel<128, 32, true, 8, false, false>", nv * (3 * D + 2 * (D // G))),
        "dequantize_int8": ("kvq::dequantize_kernel<128, 32, true, 8, false, false>", nv * (3 * D + 2 * (D // G))),
        "quantize_mxfp4": ("kvq::quantize_kernel<128, 32, true, 4, true, false>", nv * (2 * D + D // 2 + D // 32)),
        "dequantize_mxfp4": ("kvq::dequantize_kernel<128, 32, true, 4, true, false>", nv * (2 * D + D // 2 + D // 32)),
        "quantize_srft": ("kvq::quantize_kernel<128, 32, true, 4, false, true>", nv * bytes_per_vector(D, G)),
        "dequantize_srft": ("kvq::dequantize_kernel<128, 32, true, 4, false, true>", nv * bytes_per_vector(D, G)),
        "attend_partial": ("kvq::attend_partial_mfma_kernel<128>", att),
        "attend_combine": ("kvq::attend_combine_kernel<128>", None),
        "vq_encode": ("kvq::vq_encode_kernel<128, false>", nk * (2 * D + 2 * (D // 8))),
        "vq_decode": ("kvq::vq_decode_lds_kernel<128, false>", nk * (2 * D + 2 * (D // 8))),
        "vq_encode_u8": ("kvq::vq_encode_kernel<128, true>", nk * (2 * D + D // 8)),
        "vq_decode_u8": ("kvq::vq_decode_lds_kernel<128, true>", nk * (2 * D + D // 8)),
        # reads the keys and their assignments, writes the 256 (head, range)
        # workspace slots (8 int64 sums and a u32 count per centroid)
        "kmeans_accum": ("kvq::kmeans_accum_kernel<128>", nk * (2 * D + 2 * (D // 8)) + 256 * 4096 * 68),
        "kmeans_finalize": ("kvq::kmeans_finalize_kernel", 256 * 4096 * 68 + 8 * 4096 * (16 + 4)),
    }
    out = {"workload": "qwen3-8b-shaped cache [36, 262144, 8, 128] fp16, group 32, one tensor per launch; "
                       "decode attention over it as 288 sequences of 32768 tokens, 4 query heads per KV head; "
                       "vecinfer-shaped keys and values [36, 8192, 8, 128] for vq (4096 / 256 centroids)",
           "source_hash": kernel_source_hash(), "copy_reference_bytes": copy_bytes,
           "fetch_scale": round(f_scale, 6), "write_scale": round(w_scale, 6)}
    for key, (name, alg) in kernels.items():
        if name not in fe or name not in wr:
            continue
        f, w = sum(fe[name]) / len(fe[name]), sum(wr[name]) / len(wr[name])
        tb = int(f * 1024 * f_scale + w * 1024 * w_scale)
        d = {"kernel": name, "fetch_kib_per_dispatch": round(f, 1), "write_kib_per_dispatch": round(w, 1),
             "dispatches": len(fe[name]), "traffic_bytes_per_launch": tb}
        if alg:
            d["algorithmic_bytes_per_launch"] = alg
            d["traffic_over_algorithmic"] = round(tb / alg, 5)
        out[key] = d
    out["traffic_bytes_per_launch"] = out["quantize"]["traffic_bytes_per_launch"]
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    return out


def cpu_baseline(K, V, lamK, lamV, signs, G, n_tokens: int):
    """Time the fp64 oracle (single thread) on a bounded sample: every layer
    and head, `n_tokens` consecutive tokens, K and V, quantize + dequantize."""
    import numpy as np
    import torch
    import oracle
    oracle.build(force=False)
    L, T, H, D = K.shape
    t0 = (T // 2) // 16 * 16
    xs, ls = [], []
    for x, lam in ((K, lamK), (V, lamV)):
        blk = x[:, t0:t0 + n_tokens].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        xs.append(blk.reshape(-1, D))
        lr = lam.cpu().numpy()[:, None, :, :].repeat(n_tokens, axis=1)
        ls.append(lr.reshape(-1, D))
    x = np.concatenate(xs)
    lam = np.ascontiguousarray(np.concatenate(ls), np.float32)
    s = signs.cpu().numpy()
    # one core: the oracle is single-threaded; pin it so that the figure is a
    # one-core rate whatever the host's load
    try:
        saved = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {min(saved)})
    except (AttributeError, OSError):
        saved = None
    try:
        t = time.perf_counter()
        codes, scales, _, _ = oracle.quantize(x, lam, s, G)
        oracle.dequantize(codes, scales, lam, s, G)
        dt = time.perf_counter() - t
    finally:
        if saved is not None:
            os.sched_setaffinity(0, saved)
    n = x.shape[0]
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(2 * n * bytes_per_vector(D, G) / dt / 1e9, 6), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": "%d vectors (36 layers x 8 heads x %d tokens, K and V) quantize+dequantize, "
                      "single-threaded fp64 pinned to one core, %.1f s" % (n, n_tokens, dt),
            "ns_per_vector": round(dt / n * 1e9, 1),
            "vectors_per_s": round(n / dt, 1),
            "extrapolated_step_s": round(dt / n * 2 * L * T * H, 1),
            "cpu_model": cpu, "host_cpus": os.cpu_count()}


def copy_ceiling(torch, nbytes: int, reps: int = 5):
    """GB/s of a plain device-to-device copy (read + write) of `nbytes`."""
    a = torch.empty(nbytes // 2, dtype=torch.float16, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9


def stream_ceilings(torch, dev, read_bytes: int = 16 << 30, reps: int = 3):
    """Practical HBM bandwidth of this GPU for the read/write mixes of the
    quantizer's kernels, from the hand-written streaming kernels of
    libkvq_stream.so: read only, 80/20 (the quantizer's 256 B in / 72 B out
    is 78/22), 20/80 (the dequantizer's) and 1:1 copy, each with plain and
    nontemporal loads and stores and one or eight units per wavefront.
    GB/s = (bytes read + written) / kernel time (HIP events on the launching
    stream), best of `reps`; the best variant of each mix is its ceiling."""
    import ctypes
    from kv_cache_quantization_quantize_amd import build as kbuild
    lib = ctypes.CDLL(kbuild.STREAM_OUT)
    lib.kvq_stream_run.restype = ctypes.c_int
    lib.kvq_stream_run.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    src = torch.empty(read_bytes, dtype=torch.uint8, device=dev)
    dst = torch.empty(read_bytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(64, dtype=torch.int32, device=dev)
    src.fill_(1)
    stream = torch.cuda.current_stream()
    # (name, mode, chunks read, chunks written per lane and unit)
    mixes = (("read_only", 0, 4, 0), ("read80_write20", 1, 4, 1), ("read20_write80", 2, 1, 4),
             ("copy", 3, 1, 1))
    res = {}
    for name, mode, rd, wr in mixes:
        unit_bytes = 1024 * max(rd, wr)
        n_units = read_bytes // unit_bytes
        moved = n_units * 1024 * (rd + wr)
        variants = {}
        for nt in (0, 1):
            for upw in (1, 8):
                def run():
                    st = lib.kvq_stream_run(mode, ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                            n_units, upw, nt, ctypes.c_void_p(sink.data_ptr()),
                                            ctypes.c_void_p(stream.cuda_stream))
                    if st:
                        raise RuntimeError("kvq_stream_run: hip error %d" % st)
                run()
                ms = []
                for _ in range(reps):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    run()
                    b.record(stream)
                    torch.cuda.synchronize()
                    ms.append(a.elapsed_time(b))
                variants["%s_upw%d" % ("nt" if nt else "plain", upw)] = round(moved / (min(ms) * 1e-3) / 1e9, 1)
        best = max(variants, key=variants.get)
        res[name] = {"GB_per_s": variants[best], "best": best, "variants": variants, "bytes_moved": moved}
    del src, dst, sink
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--tokens", type=int, default=8 * 32768, help="tokens per tensor (default: full size)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-vq", action="store_true")
    ap.add_argument("--no-attend", action="store_true")
    ap.add_argument("--no-int8", action="store_true")
    ap.add_argument("--no-mxfp4", action="store_true")
    ap.add_argument("--no-srft", action="store_true")
    ap.add_argument("--no-small", action="store_true", help="skip the tiny / Qwen2.5 / Gemma cache timings")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-bandwidth ceilings")
    ap.add_argument("--no-d256", action="store_true", help="skip the HBM-scale head_dim-256 cache")
    ap.add_argument("--attend-seqs", type=int, default=8,
                    help="sequences the int4 cache's token axis is split into for the decode-attention leg")
    ap.add_argument("--cpu-tokens", type=int, default=192, help="tokens per (layer, head) in the CPU sample")
    ap.add_argument("--copy-bytes", type=int, default=4 << 30, help="size of the plain-copy reference")
    ap.add_argument("--parts", default="int4,vq",
                    help="comma list of what to run: int4 (the timed step), vq, copy (the plain-copy "
                         "reference of --copy-bytes, used to scale memory counters)")
    ap.add_argument("--ingest-mfma", metavar="PMC_CSV",
                    help="no GPU work: turn the counter_collection.csv of a `rocprofv3 --pmc %s` run of "
                         "`bench.py --parts vq` into the MFMA summary under profiles/ and exit" % " ".join(MFMA_COUNTERS))
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn the counter_collection.csv files of a FETCH_SIZE and a "
                         "WRITE_SIZE rocprofv3 run of this benchmark into the traffic summary under "
                         "profiles/ and exit")
    args = ap.parse_args()

    if args.ingest_mfma:
        t = ingest_mfma(args.ingest_mfma)
        print(json.dumps({k: {kk: v[kk] for kk in ("mfma_busy", "valu_busy", "clock_GHz")}
                          for k, v in t["kernels"].items()}))
        return

    if args.ingest_counters:
        t = ingest_counters(args.ingest_counters[0], args.ingest_counters[1], args.copy_bytes)
        print(json.dumps({k: v.get("traffic_over_algorithmic") for k, v in t.items() if isinstance(v, dict)}))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the quantizer has no cross-GPU step, and this build "
              "runs on a single MI355X (requested --gpus %d, WORLD_SIZE %d)." % (args.gpus, world),
              file=sys.stderr)
        sys.exit(2)

    import torch
    import kv_cache_quantization_quantize_amd as kvq
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    kvq.lib()
    dev = torch.device("cuda:0")
    parts = set(args.parts.split(","))
    if "int4" not in parts:
        # profiling helper runs: only the requested kernels, no JSON line
        if "copy" in parts:
            print("copy reference: %.1f GB/s over %d bytes" % (copy_ceiling(torch, args.copy_bytes), args.copy_bytes))
        if "vq" in parts:
            print(json.dumps({"vq": bench_vq(torch, kvq, synth, dev, args)}))
        return

    cfg = synth.config("qwen3-8b", T=args.tokens)
    L, T, H, D, G = cfg.L, cfg.T, cfg.H, cfg.D, cfg.G
    inp = synth.make_inputs(cfg, dev)
    K, V, lamK, lamV, signs = inp["K"], inp["V"], inp["lam_K"], inp["lam_V"], inp["signs"]
    codes = {n: torch.empty((L, T, H, D // 2), dtype=torch.uint8, device=dev) for n in "KV"}
    scales = {n: torch.empty((L, T, H, D // G), dtype=torch.float16, device=dev) for n in "KV"}
    outs = {n: torch.empty((L, T, H, D), dtype=torch.float16, device=dev) for n in "KV"}
    src = {"K": (K, lamK), "V": (V, lamV)}
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = []

    def step(timed: bool):
        for n in "KV":
            x, lam = src[n]
            if timed:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
            kvq.quantize(x, lam, signs, G, codes=codes[n], scales=scales[n], stream=stream)
            if timed:
                b.record(stream)
                ev.append(("quantize", a, b))
        for n in "KV":
            x, lam = src[n]
            if timed:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
            kvq.dequantize(codes[n], scales[n], lam, signs, G, out=outs[n], stream=stream)
            if timed:
                b.record(stream)
                ev.append(("dequantize", a, b))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    nvec = L * T * H
    bpv = bytes_per_vector(D, G)
    step_bytes = 4 * nvec * bpv
    ms_step = wall / args.steps * 1e3
    value = step_bytes / (wall / args.steps) / 1e9

    kern = {}
    for name in ("quantize", "dequantize"):
        ms = [a.elapsed_time(b) for (k, a, b) in ev if k == name]
        avg = sum(ms) / len(ms)
        gbps = nvec * bpv / (avg * 1e-3) / 1e9
        kern[name] = {"launches": len(ms), "avg_ms": round(avg, 4), **spread(ms), "GB_per_s": round(gbps, 1),
                      "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                      "ns_per_vector": round(avg * 1e6 / nvec, 5),
                      "vectors_per_s": round(nvec / (avg * 1e-3), 1)}

    q = kern["quantize"]
    per_launch = nvec * bpv
    traffic = load_traffic(per_launch)
    roofline = {"bound": "hbm", "achieved": q["GB_per_s"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": q["frac_of_hbm_peak"], "traffic": traffic,
                "kernel": "kvq::quantize_kernel<128, 32>",
                "algorithmic_bytes_per_launch": per_launch,
                "bytes_per_vector": bpv, "vectors_per_launch": nvec}

    del outs
    torch.cuda.empty_cache()

    int8 = None
    if not args.no_int8:
        int8 = bench_variant(torch, kvq, K, lamK, signs, (L, T, H, D, G), args, "int8")
    mxfp4 = None
    if not args.no_mxfp4:
        mxfp4 = bench_variant(torch, kvq, K, lamK, signs, (L, T, H, D, G), args, "mxfp4")
    srft = None
    if not args.no_srft:
        srft = bench_variant(torch, kvq, K, lamK, signs, (L, T, H, D, G), args, "srft")

    attend = None
    if not args.no_attend:
        attend = bench_attend(torch, kvq, codes, scales, lamK, lamV, signs, (L, T, H, D, G), args)

    if "copy" in parts:
        # the plain-copy reference of --copy-bytes that scales the memory
        # counters (not reported)
        copy_ceiling(torch, args.copy_bytes)

    ceil = None
    if not args.no_ceiling:
        ceil = stream_ceilings(torch, dev)
        for name, mix in (("quantize", "read80_write20"), ("dequantize", "read20_write80")):
            kern[name]["frac_of_practical_ceiling"] = round(kern[name]["GB_per_s"] / ceil[mix]["GB_per_s"], 4)
            kern[name]["practical_ceiling_mix"] = mix
        roofline["frac_of_practical_ceiling"] = kern["quantize"]["frac_of_practical_ceiling"]

    d256 = None
    if not args.no_d256:
        d256 = bench_d256(torch, kvq, synth, dev, args, ceil)

    vq = None
    if not args.no_vq:
        vq = bench_vq(torch, kvq, synth, dev, args)

    small = None
    if not args.no_small:
        small = bench_small(torch, kvq, synth, dev, args)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(K, V, lamK, lamV, signs, G, args.cpu_tokens)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "qwen3-8b-shaped bulk prefill KV cache, int4 quantize + dequantize of K and V",
                   "tensor_shape": [L, T, H, D], "head_dim": D, "group": G, "tensors": 2,
                   "vectors_per_tensor": nvec, "step": "quantize K, V then dequantize K, V",
                   "algorithmic_bytes_per_step": step_bytes},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kern,
        "practical_ceiling": ceil,
        "d256": d256,
        "vq": vq,
        "attend": attend,
        "int8": int8,
        "mxfp4": mxfp4,
        "srft": srft,
        "small_workloads": small,
        "frac_of_hbm_peak_step": round(value / HBM_PEAK_GBPS, 4),
    }
    print(json.dumps(out), flush=True)


def bench_small(torch, kvq, synth, dev, args):
    """The pages' smaller caches: quantize + dequantize of the tiny key cache
    (a launch latency), the Qwen2.5-1.5B-shaped K/V caches and the
    Gemma-3-1B-shaped K/V caches at 256-, 1024- and 4096-token prefixes.
    Each is timed warm (10 launches back to back, averaged: the tensors fit
    in the 256 MB Infinity Cache, so this is not an HBM figure) and after a
    1 GB scrub (inputs come from HBM; median of 10 single launches).  Every leg reports
    microseconds, algorithmic GB/s, its fraction of the 8 TB/s HBM peak,
    vectors/s and ns/vector.  Plus, on the 4096-token Gemma cache, the
    decode append (one token per layer, K and V) and a decode-attention
    call."""
    stream = torch.cuda.current_stream()
    scrub = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    res = {}

    def timed(fn, reps, do_scrub):
        """Median kernel time of fn.  Scrubbed: one launch per timed interval,
        behind the scrub (which keeps the GPU busy while the events and the
        launch are queued).  Warm: `reps` launches back to back between two
        events, so that no host launch gap of an idle GPU is timed; the
        interval is divided by the launch count."""
        if not do_scrub:
            fn()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / reps
        ms = []
        for _ in range(reps):
            scrub.zero_()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        ms.sort()
        return ms[len(ms) // 2]

    def leg(ms, nvec, byt):
        gbps = byt / (ms * 1e-3) / 1e9
        return {"us": round(ms * 1e3, 2), "GB_per_s": round(gbps, 1), "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                "vectors_per_s": round(nvec / (ms * 1e-3), 1), "ns_per_vector": round(ms * 1e6 / nvec, 4)}

    for name, T in (("tiny", None), ("qwen2.5-1.5b", None), ("gemma-3-1b", 256), ("gemma-3-1b", 1024),
                    ("gemma-3-1b", 4096)):
        cfg = synth.config(name, T=T) if T else synth.config(name)
        inp = synth.make_inputs(cfg, dev)
        L, T, H, D, G = cfg.L, cfg.T, cfg.H, cfg.D, cfg.G
        nvec = L * T * H
        byt = nvec * bytes_per_vector(D, G)
        r = {"shape": [L, T, H, D], "group": G, "vectors_per_tensor": nvec, "algorithmic_bytes_per_launch": byt}
        for t in ("K", "V"):
            if t not in inp:
                continue
            x, lam = inp[t], inp["lam_" + t]
            codes, scales = kvq.quantize(x, lam, inp["signs"], G, stream=stream)
            out = torch.empty_like(x)
            for mode in ("warm", "scrubbed"):
                qms = timed(lambda: kvq.quantize(x, lam, inp["signs"], G, codes=codes, scales=scales, stream=stream),
                            10, mode == "scrubbed")
                dms = timed(lambda: kvq.dequantize(codes, scales, lam, inp["signs"], G, out=out, stream=stream),
                            10, mode == "scrubbed")
                r["%s_%s" % (t, mode)] = {
                    "residency": "infinity cache (10 launches back to back)" if mode == "warm" else "hbm (after a 1 GB scrub)",
                    "quantize": leg(qms, nvec, byt), "dequantize": leg(dms, nvec, byt)}
        if name == "gemma-3-1b" and T == 4096:
            # decode append: layer by layer, K then V, one token into slot T - 1
            caches = {t: kvq.quantize(inp[t], inp["lam_" + t], inp["signs"], G, stream=stream) for t in ("K", "V")}
            tok = {t: inp[t][:, T - 1:T].contiguous() for t in ("K", "V")}
            lam1 = {t: [inp["lam_" + t][l:l + 1].contiguous() for l in range(L)] for t in ("K", "V")}

            def step(st=stream):
                for l in range(L):
                    for t in ("K", "V"):
                        c, sc = caches[t]
                        kvq.quantize(tok[t][l:l + 1], lam1[t][l], inp["signs"], G, codes=c[l:l + 1, T - 1:T],
                                     scales=sc[l:l + 1, T - 1:T], stream=st)

            def graph_step():
                step(torch.cuda.current_stream())
            step()
            torch.cuda.synchronize()
            sms = timed(step, 10, False)
            # the same launches captured once in a HIP graph and replayed
            # (no Python or per-launch host work in the timed region)
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                graph_step()
            stream.wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                graph_step()
            g.replay()
            torch.cuda.synchronize()
            gms = timed(g.replay, 20, False)
            # K and V in one launch per layer: a cache laid out [L, T, 2H, .]
            # holds K in heads 0..H-1 and V in heads H..2H-1 (attention takes
            # the two halves as strided views), lambda [L, 2H, D] likewise
            kv_codes = torch.empty((L, T, 2 * H, D // 2), dtype=torch.uint8, device=dev)
            kv_scales = torch.empty((L, T, 2 * H, D // G), dtype=torch.float16, device=dev)
            tok_kv = torch.cat([tok["K"], tok["V"]], dim=2).contiguous()
            lam_kv = [torch.cat([lam1["K"][l], lam1["V"][l]], dim=1).contiguous() for l in range(L)]

            def step_kv(st=stream):
                for l in range(L):
                    kvq.quantize(tok_kv[l:l + 1], lam_kv[l], inp["signs"], G, codes=kv_codes[l:l + 1, T - 1:T],
                                 scales=kv_scales[l:l + 1, T - 1:T], stream=st)

            def graph_step_kv():
                step_kv(torch.cuda.current_stream())
            step_kv()
            torch.cuda.synchronize()
            kms = timed(step_kv, 10, False)
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                graph_step_kv()
            stream.wait_stream(side)
            torch.cuda.synchronize()
            g2 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g2):
                graph_step_kv()
            g2.replay()
            torch.cuda.synchronize()
            kgms = timed(g2.replay, 20, False)
            r["decode_append"] = {"us_per_layer_K_and_V": round(sms * 1e3 / L, 2), "us_per_step": round(sms * 1e3, 1),
                                  "layers": L, "note": "two launches per layer; launch-bound",
                                  "hip_graph_us_per_step": round(gms * 1e3, 1),
                                  "hip_graph_us_per_layer_K_and_V": round(gms * 1e3 / L, 2),
                                  "kv_in_one_launch_us_per_step": round(kms * 1e3, 1),
                                  "kv_in_one_launch_hip_graph_us_per_step": round(kgms * 1e3, 1)}
            del g, g2, kv_codes, kv_scales
            # decode attention over the whole cache: 4 query heads on the one
            # KV head, all layers in one call (matrix-core kernel, head_dim 256)
            R = 4
            qg = torch.Generator(device="cpu").manual_seed(2026)
            q = torch.randn((L, H * R, D), generator=qg).to(torch.float16).to(dev)
            kc, ks = caches["K"]
            vc, vs = caches["V"]
            ws = torch.empty(kvq.attend_decode_workspace_bytes(L, T, H, D, R), dtype=torch.uint8, device=dev)
            ao = torch.empty((L, H * R, D), dtype=torch.float16, device=dev)

            def attend():
                kvq.attend_decode(q, kc, ks, vc, vs, inp["lam_K"], inp["lam_V"], inp["signs"], G, out=ao,
                                  workspace=ws, stream=stream)
            attend()
            torch.cuda.synchronize()
            ams = timed(attend, 20, False)
            abytes = 2 * L * T * H * (D // 2 + 2 * (D // G))
            r["decode_attention"] = {"layers": L, "tokens": T, "q_per_kv": R, "ms": round(ams, 4),
                                     "GB_per_s": round(abytes / (ams * 1e-3) / 1e9, 1),
                                     "note": "one call over all layers; small, so launch and tail bound"}
            del ws, ao
        res[name if name != "gemma-3-1b" else "%s_T%d" % (name, T)] = r
        del inp
        torch.cuda.empty_cache()
    del scrub
    torch.cuda.empty_cache()
    return res


def bench_d256(torch, kvq, synth, dev, args, ceil):
    """The head_dim-256 / group-64 kernels at HBM scale: a Gemma-3-1B-shaped
    cache [26 layers, 262,144 tokens (64 sequences x 4,096), 1 KV head, 256],
    K and V (3.49 GB each, far beyond the Infinity Cache), quantize then
    dequantize, HIP events per launch."""
    cfg = synth.config("gemma-3-1b", T=64 * 4096)
    inp = synth.make_inputs(cfg, dev)
    L, T, H, D, G = cfg.L, cfg.T, cfg.H, cfg.D, cfg.G
    stream = torch.cuda.current_stream()
    nvec = L * T * H
    bpv = bytes_per_vector(D, G)
    codes = torch.empty((L, T, H, D // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((L, T, H, D // G), dtype=torch.float16, device=dev)
    out = torch.empty((L, T, H, D), dtype=torch.float16, device=dev)
    ev = {"quantize": [], "dequantize": []}
    for rep in range(1 + max(3, min(args.steps, 10))):
        for t in ("K", "V"):
            x, lam = inp[t], inp["lam_" + t]
            for name, fn in (("quantize", lambda: kvq.quantize(x, lam, inp["signs"], G, codes=codes, scales=scales,
                                                                stream=stream)),
                             ("dequantize", lambda: kvq.dequantize(codes, scales, lam, inp["signs"], G, out=out,
                                                                    stream=stream))):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn()
                b.record(stream)
                if rep:
                    ev[name].append((a, b))
    torch.cuda.synchronize()
    res = {"workload": "gemma-3-1b-shaped cache at HBM scale [%d, %d, %d, %d] (64 sequences x 4096 tokens), "
                       "group %d, K and V" % (L, T, H, D, G), "bytes_per_vector": bpv, "vectors_per_launch": nvec}
    for name, pairs in ev.items():
        ms = [a.elapsed_time(b) for a, b in pairs]
        avg = sum(ms) / len(ms)
        gbps = nvec * bpv / (avg * 1e-3) / 1e9
        r = {"launches": len(ms), "avg_ms": round(avg, 4), **spread(ms), "GB_per_s": round(gbps, 1),
             "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4), "ns_per_vector": round(avg * 1e6 / nvec, 5),
             "vectors_per_s": round(nvec / (avg * 1e-3), 1)}
        if ceil:
            mix = "read80_write20" if name == "quantize" else "read20_write80"
            r["frac_of_practical_ceiling"] = round(gbps / ceil[mix]["GB_per_s"], 4)
        res[name] = r
    del inp, codes, scales, out
    torch.cuda.empty_cache()
    return res


def bench_variant(torch, kvq, K, lamK, signs, dims, args, kind):
    """Time one code variant of the fused quantizer (quantize, then dequantize)
    on the K cache: "int8" (127 levels, fp16 group scales), "mxfp4" (E2M1
    elements, one E8M0 scale byte per 32 coordinates) or "srft" (int4 codes
    on the sign-randomized real Fourier rotation)."""
    L, T, H, D, G = dims
    if kind == "srft":
        codes = torch.empty((L, T, H, D // 2), dtype=torch.uint8, device=K.device)
        scales = torch.empty((L, T, H, D // G), dtype=torch.float16, device=K.device)
        bpv = bytes_per_vector(D, G)
        what = "group %d, int4 codes, SRFT rotation" % G
        qf = lambda: kvq.quantize_srft(K, lamK, signs, G, codes=codes, scales=scales, stream=stream)
        df = lambda: kvq.dequantize_srft(codes, scales, lamK, signs, G, out=out, stream=stream)
    elif kind == "int8":
        codes = torch.empty((L, T, H, D), dtype=torch.int8, device=K.device)
        scales = torch.empty((L, T, H, D // G), dtype=torch.float16, device=K.device)
        bpv = 2 * D + D + 2 * (D // G)
        what = "group %d, int8 codes" % G
        qf = lambda: kvq.quantize_int8(K, lamK, signs, G, codes=codes, scales=scales, stream=stream)
        df = lambda: kvq.dequantize_int8(codes, scales, lamK, signs, G, out=out, stream=stream)
    else:
        codes = torch.empty((L, T, H, D // 2), dtype=torch.uint8, device=K.device)
        scales = torch.empty((L, T, H, D // 32), dtype=torch.uint8, device=K.device)
        bpv = 2 * D + D // 2 + D // 32
        what = "blocks of 32, E2M1 codes, E8M0 scales"
        qf = lambda: kvq.quantize_mxfp4(K, lamK, signs, codes=codes, scales=scales, stream=stream)
        df = lambda: kvq.dequantize_mxfp4(codes, scales, lamK, signs, out=out, stream=stream)
    out = torch.empty_like(K)
    stream = torch.cuda.current_stream()
    qf()
    df()
    torch.cuda.synchronize()
    ev = {"quantize": [], "dequantize": []}
    for _ in range(max(3, min(args.steps, 10))):
        for name, fn in (("quantize", qf), ("dequantize", df)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            ev[name].append((a, b))
    torch.cuda.synchronize()
    nvec = L * T * H
    res = {"workload": "qwen3-8b-shaped K cache [%d, %d, %d, %d], %s" % (L, T, H, D, what),
           "bytes_per_vector": bpv}
    for name, pairs in ev.items():
        ms = [a.elapsed_time(b) for a, b in pairs]
        avg = sum(ms) / len(ms)
        gbps = nvec * bpv / (avg * 1e-3) / 1e9
        res[name] = {"avg_ms": round(avg, 4), **spread(ms), "GB_per_s": round(gbps, 1),
                     "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                     "ns_per_vector": round(avg * 1e6 / nvec, 5)}
    del codes, scales, out
    torch.cuda.empty_cache()
    return res


def bench_attend(torch, kvq, codes, scales, lamK, lamV, signs, dims, args):
    """Time one decode step of attention over the quantized K/V caches: the
    [36, 262144, 8, 128] caches read as 36 layers x B sequences of T/B
    tokens, 4 query heads per KV head (Qwen3-8B: 32 query, 8 KV heads)."""
    L, T, H, D, G = dims
    B, R = args.attend_seqs, 4
    if T % B:
        return None
    Lo, Tq = L * B, T // B
    kc, ks = codes["K"].view(Lo, Tq, H, D // 2), scales["K"].view(Lo, Tq, H, D // G)
    vc, vs = codes["V"].view(Lo, Tq, H, D // 2), scales["V"].view(Lo, Tq, H, D // G)
    lk = lamK.repeat_interleave(B, dim=0).contiguous()
    lv = lamV.repeat_interleave(B, dim=0).contiguous()
    g = torch.Generator(device="cpu").manual_seed(4321)
    q = torch.randn((Lo, H * R, D), generator=g).to(torch.float16).to(kc.device)
    out = torch.empty_like(q)
    ws = torch.empty(max(16, kvq.attend_decode_workspace_bytes(Lo, Tq, H, D, R)), dtype=torch.uint8,
                     device=kc.device)
    stream = torch.cuda.current_stream()

    def call():
        kvq.attend_decode(q, kc, ks, vc, vs, lk, lv, signs, G, out=out, workspace=ws, stream=stream)

    for _ in range(2):
        call()
    torch.cuda.synchronize()
    ms = []
    for _ in range(max(3, min(args.steps, 20))):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        b.record(stream)
        ms.append((a, b))
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ms]
    avg = sum(ms) / len(ms)
    cache_bytes = 2 * Lo * Tq * H * (D // 2 + 2 * (D // G))        # K and V codes + scales
    qo_bytes = 2 * Lo * H * R * D * 2                               # queries in, outputs out
    byt = cache_bytes + qo_bytes
    gbps = byt / (avg * 1e-3) / 1e9
    return {"workload": "qwen3-8b-shaped decode step: %d layers x %d sequences x %d tokens, %d KV heads, "
                        "%d query heads per KV head, head_dim %d, group %d" % (L, B, Tq, H, R, D, G),
            "avg_ms": round(avg, 4), **spread(ms), "GB_per_s": round(gbps, 1),
            "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4), "algorithmic_bytes_per_call": byt,
            "ns_per_token_head": round(avg * 1e6 / (Lo * Tq * H), 5),
            "workspace_bytes": int(ws.numel())}


def bench_vq(torch, kvq, synth, dev, args):
    """Time the product-VQ paths on the VecInfer-shaped caches: key encode and
    decode (4096-centroid codebooks, u16 indices), value encode and decode
    (256-centroid codebooks, one-byte indices) and one k-means codebook
    training step on the keys."""
    cfg = synth.config("vq")
    try:
        inp = synth.make_inputs(cfg, dev)
    except RuntimeError:
        return None
    x, lam, s, cb = inp["K"], inp["lam_K"], inp["signs"], inp["codebook"]
    v, lam_v, cb_v = inp["V"], inp["lam_V"], inp["codebook_V"]
    L, T, H, D = x.shape
    sub = cfg.sub_dim
    idx = torch.empty((L, T, H, D // sub), dtype=torch.int16, device=dev)
    idx8 = torch.empty((L, T, H, D // sub), dtype=torch.uint8, device=dev)
    out = torch.empty_like(x)
    new_cb = torch.empty_like(cb)
    counts = torch.empty((H, cfg.n_centroids), dtype=torch.int32, device=dev)
    ws = torch.empty(kvq.kmeans_step_workspace_bytes(L, T, H, D, cfg.n_centroids, sub), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()
    legs = (
        ("encode", lambda: kvq.vq_encode(x, lam, s, cb, sub, idx=idx, stream=stream)),
        ("decode", lambda: kvq.vq_decode(idx, cb, lam, s, sub, out=out, stream=stream)),
        ("value_encode_u8", lambda: kvq.vq_encode_u8(v, lam_v, s, cb_v, sub, idx=idx8, stream=stream)),
        ("value_decode_u8", lambda: kvq.vq_decode_u8(idx8, cb_v, lam_v, s, sub, out=out, stream=stream)),
        ("kmeans_step", lambda: kvq.kmeans_step(x, lam, s, cb, sub, idx=idx, new_codebook=new_cb, counts=counts,
                                                workspace=ws, stream=stream)),
    )
    try:
        for _, fn in legs:
            fn()
        torch.cuda.synchronize()
    except kvq.KvqError as e:
        return {"status": "unavailable", "error": str(e)}
    res = {}
    reps = max(3, min(args.steps, 10))
    nkeys = L * T * H
    for name, fn in legs:
        fn()
        ms = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        avg = sum(ms) / len(ms)
        r = {"avg_ms": round(avg, 4), **spread(ms), "ns_per_key": round(avg * 1e6 / nkeys, 4)}
        if name in ("encode", "kmeans_step"):
            flop = nkeys * (D // sub) * cfg.n_centroids * sub * 2
            tf = flop / (avg * 1e-3) / 1e12
            r.update({"algorithmic_TFLOP": round(flop / 1e12, 4), "TFLOP_per_s": round(tf, 2),
                      "frac_of_fp16_mfma_peak": round(tf / FP16_MFMA_PEAK_TFLOPS, 4)})
            if name == "encode":
                # per 32-centroid tile and 8 groups of 32 sub-vectors: eight
                # 32x32x16 MFMAs on the fp16 hi/lo split plus one 32x32x8
                # norm MFMA, against 8 x 32 x 32 x 8 algorithmic MACs
                r.update({"executed_mfma_flop_factor": 2.125,
                          "executed_frac_of_fp16_mfma_peak": round(2.125 * tf / FP16_MFMA_PEAK_TFLOPS, 4)})
            else:
                r["includes"] = "assignment (the encoder) + accumulate + finalize"
        else:
            ib = 2 if name == "decode" else 1
            if name == "value_encode_u8":
                # a search against 256 centroids: MFMA contraction plus the
                # VALU argmax, not an HBM stream
                flop = nkeys * (D // sub) * cfg.v_centroids * sub * 2
                tf = flop / (avg * 1e-3) / 1e12
                # one-byte path: 256 centroids = 8 tiles, GPR = 8 groups per norm MFMA
                r.update({"algorithmic_TFLOP": round(flop / 1e12, 4), "TFLOP_per_s": round(tf, 2),
                          "frac_of_fp16_mfma_peak": round(tf / FP16_MFMA_PEAK_TFLOPS, 4),
                          "executed_frac_of_fp16_mfma_peak": round(2.125 * tf / FP16_MFMA_PEAK_TFLOPS, 4)})
            byt = nkeys * (2 * D + ib * (D // sub))
            r.update({"GB_per_s": round(byt / (avg * 1e-3) / 1e9, 1),
                      "frac_of_hbm_peak": round(byt / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)})
        res[name] = r
    res["workload"] = ("vecinfer-shaped keys and values [36, 8192, 8, 128]; key codebooks [8, 4096, 8] fp16, "
                       "value codebooks [8, 256, 8] fp16, sub_dim 8")
    mf = load_mfma()
    for name, kern in (("encode", "kvq::vq_encode_kernel<128, false>"), ("value_encode_u8", "kvq::vq_encode_kernel<128, true>")):
        k = (mf or {}).get("kernels", {}).get(kern)
        if k and name in res:
            res[name]["counters"] = {"source": os.path.relpath(MFMA_FILE, ROOT), "mfma_busy": k["mfma_busy"],
                                     "valu_busy": k["valu_busy"], "clock_GHz": k["clock_GHz"],
                                     "executed_fp16_TFLOP_per_s": k.get("executed_fp16_TFLOP_per_s")}
    return res


if __name__ == "__main__":
    main()
