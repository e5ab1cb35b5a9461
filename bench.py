"""Benchmark of libskipattn on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-sweep] [--no-cpu]
                    [--only LEG] [--prefill-workload prefill_128k|prefill_32k|prefill_8k]

A step is one pass of the whole hot path: a causal GQA prefill at 128K
context (B=1, Hq=8, Hkv=1, N=131072, d=128) followed by a split-K decode
over a 128K KV cache (B=16, Hq=64, Hkv=8, L=131072, d=128), both at
tau = inf, on seeded synthetic bf16 inputs already resident in HBM.

Printed: one JSON line. ``value`` is the prefill's dense-equivalent
TFLOP/s (4 d x unmasked query-key pairs per call) from HIP events recorded on
the launch stream around each call inside the timed region; the decode's KV
GB/s is reported beside it, then a tau sweep (skip fractions, dense and
executed TFLOP/s, dense and actual GB/s) and the fp64 oracle's throughput on
the host cores over a bounded sample of the same workloads. Timed calls
write no skip mask (an optional output); the sweep reads each tau's mask
from one extra call outside its timing.

``--prefill-workload`` puts the 32K (B=1, Hq=64, Hkv=8) or 8K (B=1, Hq=32,
Hkv=8) causal prefill shape in the 128K one's place; the default line is the
128K step.

Beside the step, the same prefill with block-quantised fp8 QK^T
(``prefill_qk8``: time including the quantisers, TFLOP/s dense-equivalent,
fraction of the bf16 peak and of the fp8/bf16 mixed peak, drift from the
exact prefill, tau sweep), likewise with fp8 P.V (``prefill_pv8``), both
products on fp8 (``prefill_qkv8``) and int8 QK^T (``prefill_qki8``), the same
prefill with the SAS exponential of degree
2 and 3 (``prefill_sas2``, ``prefill_sas3``: TFLOP/s dense-equivalent, time
relative to the exact prefill, drift from it, tau sweep), the 8K and 32K
causal prefill workloads are timed alone
(``prefill_8k``, ``prefill_32k``: TFLOP/s, fraction of the bf16 peak, their
tau sweeps), and the same decode workload is run over the 4-bit asymmetric
KV cache (attn_kv_quantize_q4, then attn_decode_q4 timed like the bf16
decode): ``decode_q4`` reports GB/s of the 4-bit bytes read, its fraction of
HBM peak and the bf16-equivalent rate, and the quantiser's time per call
rewriting the cache (``quantise_ms``, ``quantise_gbs`` of bf16 K and V read
plus cache bytes written; ``quantise_first_ms`` for the first call, which
also allocates the cache); likewise ``decode_q2`` and ``decode_hybrid``.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill attn TFLOP/s (dense-equiv) & decode KV GB/s at 128K ctx, per τ"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA (int8: 5000 TOP/s, the same rate)
# the fp8-QK^T prefill does half its dense flops (QK^T) at the fp8 rate and
# half (PV) at the bf16 rate: its MFMA ceiling is the harmonic mix
PEAK_QK8_TFLOPS = 2.0 / (1.0 / PEAK_FP8_TFLOPS + 1.0 / PEAK_BF16_TFLOPS)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE,
# scaled by the same counters on a 1 GiB copy (FETCH x 2.0, WRITE x 1.0).
# Keyed by the SHA-1 of the kernel's source files: once a kernel changes the
# figure no longer applies and is reported as null.
MEASURED_TRAFFIC = {
    "prefill": {"sources": ("prefill.hip", "prefill_steps.inc", "common.hpp", "sas.hpp", "launch.hpp"),
                "sha1": "474d32ae78e620715f0f445753e1bd2f369cdab2",
                "bytes": (2707060.4 * 2.0 + 528520.1) * 1024},
    "prefill_qk8": {"sources": ("prefill.hip", "prefill_steps.inc", "common.hpp", "sas.hpp", "launch.hpp", "fp8.hip"),
                "sha1": "1db5b0e0bc130bbc71659f9eceaefe4bea504230",
                "bytes": (1697532.9 * 2.0 + 528520.1) * 1024},
    "prefill_qki8": {"sources": ("prefill.hip", "prefill_steps.inc", "common.hpp", "sas.hpp", "launch.hpp", "fp8.hip"),
                "sha1": "1db5b0e0bc130bbc71659f9eceaefe4bea504230",
                "bytes": (1701842.8 * 2.0 + 528520.1) * 1024},
    "prefill_pv8": {"sources": ("prefill.hip", "prefill_steps.inc", "common.hpp", "sas.hpp", "launch.hpp", "fp8.hip"),
                "sha1": "1db5b0e0bc130bbc71659f9eceaefe4bea504230",
                "bytes": (1778258.2 * 2.0 + 528520.1) * 1024},
    "prefill_qkv8": {"sources": ("prefill.hip", "prefill_steps.inc", "common.hpp", "sas.hpp", "launch.hpp", "fp8.hip"),
                "sha1": "1db5b0e0bc130bbc71659f9eceaefe4bea504230",
                "bytes": (1162283.7 * 2.0 + 528520.1) * 1024},
    "decode_q4": {"sources": ("kvq4.hip", "kvq_common.hpp", "decode.hip", "common.hpp", "sas.hpp", "lane_max.hpp", "launch.hpp"),
                "sha1": "89f1032dfc320c342979397f4edd240b87cc0c10",
                "bytes": (1148140.6 * 2.0 + 16643.4) * 1024},
    "decode_q2": {"sources": ("kvq2.hip", "kvq_common.hpp", "decode.hip", "common.hpp", "sas.hpp", "lane_max.hpp", "launch.hpp"),
                "sha1": "591dc032bb5f1fe1a42631e99505d3b3911b49fd",
                "bytes": (623809.2 * 2.0 + 16641.0) * 1024},
    "decode_hybrid": {"sources": ("kvq4.hip", "kvq2.hip", "kvq_common.hpp", "decode.hip", "common.hpp", "sas.hpp", "lane_max.hpp", "launch.hpp"),
                "sha1": "63aaf1176aa70d22b48ddec0c0c785fe92a9f75d",
                "bytes": (886084.3 * 2.0 + 16641.0) * 1024},
    "decode": {"sources": ("decode.hip", "common.hpp", "sas.hpp", "lane_max.hpp"),
               "sha1": "333142df1d615caa64770921eb2ebcb71ade361c",
               "bytes": (4195498.3 * 2.0 + 16641.4) * 1024},
}


def _source_sha1(names):
    import hashlib
    h = hashlib.sha1()
    for n in names:
        with open(os.path.join(ROOT, "long_context_tiled_amd", "csrc", n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(leg):
    t = MEASURED_TRAFFIC.get(leg)
    if t is None:
        return None
    return t["bytes"] if _source_sha1(t["sources"]) == t["sha1"] else None


def _dev(bits, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def prefill_dense_flops(B, Hq, N, d, causal=True):
    pairs = N * (N + 1) // 2 if causal else N * N
    return 4.0 * d * B * Hq * pairs


def prefill_exec_flops(mask, d):
    """QK^T on every visited tile, PV on kept tiles (full-tile count)."""
    visited = int((mask != 2).sum())
    kept = int((mask == 0).sum())
    return 2.0 * d * 64 * 64 * (visited + kept), visited, kept


def decode_bytes(B, Hkv, L, d, mask=None, G=1):
    """Dense KV bytes, and the bytes the kernel must read at this mask: all of
    K plus the V tiles that at least one head of the KV group keeps."""
    dense = 2.0 * B * Hkv * L * d * 2
    if mask is None:
        return dense, dense
    Bm, Hq, nt = mask.shape
    keep_any = (mask.reshape(Bm, Hkv, G, nt) == 0).any(axis=2)
    tile_keys = np.full(nt, 64)
    tile_keys[-1] = L - 64 * (nt - 1)
    v_bytes = float((keep_any * tile_keys[None, None, :]).sum()) * d * 2
    return dense, dense / 2 + v_bytes


def qcache_bytes(bits, B, Hkv, L, d, mask=None, G=1):
    """Bytes of a bits-wide cache (4 or 2) the decode must read: K codes
    (d bits / 8 per key) and parameter words (4 per key), and per V tile its
    codes (8 bits d) and parameter words (4 d) when at least one head of the
    KV group keeps it."""
    T = (L + 63) // 64
    k_b = float(B * Hkv * L * (d * bits // 8 + 4))
    v_tile = (8.0 * bits + 4.0) * d
    if mask is None:
        return k_b + B * Hkv * T * v_tile
    Bm, Hq, nt = mask.shape
    keep_any = (mask.reshape(Bm, Hkv, G, nt) == 0).any(axis=2)
    return k_b + float(keep_any.sum()) * v_tile


def q4_bytes(B, Hkv, L, d, mask=None, G=1):
    return qcache_bytes(4, B, Hkv, L, d, mask, G)


def q2_bytes(B, Hkv, L, d, mask=None, G=1):
    return qcache_bytes(2, B, Hkv, L, d, mask, G)


class Timer:
    """HIP events on the current stream around each call."""

    def __init__(self):
        self.pairs = []

    def __enter__(self):
        import torch
        self.s = torch.cuda.Event(enable_timing=True)
        self.e = torch.cuda.Event(enable_timing=True)
        self.s.record()
        return self

    def __exit__(self, *a):
        self.e.record()
        self.pairs.append((self.s, self.e))

    def ms(self):
        return [s.elapsed_time(e) for s, e in self.pairs]


# Extra legs run after seconds of host work (input generation), during which
# the GPU idles and its shader clock falls; a leg timed after two short calls
# runs at that lower clock (measured on prefill_8k: 1.48 GHz after 3 calls,
# 1.92 GHz after 40, with the same cycles per tile). Each extra leg is
# therefore timed after at least WARM_MS of back-to-back untimed calls (and at
# least --warmup calls).
WARM_MS = 100.0


def warm_up(fn, n):
    import torch
    t0 = time.perf_counter()
    i = 0
    while i < n or (time.perf_counter() - t0) * 1e3 < WARM_MS:
        fn()
        i += 1
        if i % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_quantiser(fn, cache_tensors, k, v, steps, warmup):
    """A KV-cache quantiser rewriting a cache it has already written: ms per
    call (HIP events, after warm-up) and GB/s of bytes it must move (bf16 K
    and V read once, every cache byte written once)."""
    import torch
    warm_up(fn, warmup)
    t = Timer()
    torch.cuda.synchronize()
    for _ in range(steps):
        with t:
            fn()
    torch.cuda.synchronize()
    ms = float(np.mean(t.ms()))
    moved = (k.numel() + v.numel()) * 2 + sum(x.numel() * x.element_size() for x in cache_tensors)
    return ms, moved / (ms * 1e-3) / 1e9


# ---------------------------------------------------------------- CPU baseline

_CPU = {}  # arrays shared with forked oracle workers (inherited, never pickled)


def _cpu_prefill_block(qb):
    from threadpoolctl import threadpool_limits
    import oracle
    import synth
    with threadpool_limits(1):
        qrows = synth.bf16_bits_to_f64(_CPU["pq"][qb * 64:(qb + 1) * 64])
        oracle.prefill_blocks(qrows, _CPU["pk"], _CPU["pv"], qb, True, math.inf)


def _cpu_decode_head(job):
    from threadpoolctl import threadpool_limits
    import oracle
    import synth
    i, hh = job
    with threadpool_limits(1):
        k, v, q = _CPU["dkv"][i]
        oracle.decode_head(synth.bf16_bits_to_f64(q[hh]), k, v, math.inf)


def _cpu_decode_q_head(item):
    from threadpoolctl import threadpool_limits
    import oracle
    import synth
    from oracle import kvq2, kvq4
    key, i = item
    with threadpool_limits(1):
        e, q, L, w = _CPU[key][i]
        codec = {4: kvq4, 2: kvq2}[w]
        k = codec.decode_k(e["kq"], e["kp"])
        v = codec.decode_v(e["vq"], e["vp"], L)
        for hh in range(q.shape[0]):
            oracle.decode_head(synth.bf16_bits_to_f64(q[hh]), k, v, math.inf)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(pq, pk, pv, dq, dk, dv, nblocks=768, nkv=32, nkv_q=16, pname="prefill_128k",
                 hybrid_bits=None):
    """The fp64 oracle as it stands, timed on a bounded sample of each
    workload with one process per host core (fp64 widening of the inputs is
    done before the clock starts)."""
    import multiprocessing as mp

    import synth
    cores = min(16, os.cpu_count() or 1)      # worker processes actually used
    N, d = pq.shape[2], pq.shape[3]
    nt = N // 64
    nblocks = min(nblocks, nt)
    qbs = [int(x) for x in np.linspace(0, nt - 1, nblocks).astype(int)]
    _CPU.clear()
    _CPU.update(pq=pq[0, 0], pk=synth.bf16_bits_to_f64(pk[0, 0]),
                pv=synth.bf16_bits_to_f64(pv[0, 0]))
    B, Hq = dq.shape[0], dq.shape[1]
    Hkv, L = dk.shape[1], dk.shape[2]
    G = Hq // Hkv
    picks = [(b, g) for b in range(B) for g in range(Hkv)][:nkv]
    _CPU["dkv"] = [(synth.bf16_bits_to_f64(dk[b, g]), synth.bf16_bits_to_f64(dv[b, g]),
                    dq[b, g * G:(g + 1) * G]) for b, g in picks]
    from oracle import kvq2, kvq4
    pickq = picks[:nkv_q]
    qkeys = [("dq4", lambda g: 4), ("dq2", lambda g: 2)]
    if hybrid_bits is not None:   # each KV head at its width in the hybrid cache
        qkeys.append(("dqh", lambda g: hybrid_bits[g]))
    for key, width in qkeys:
        _CPU[key] = []
        for b, g in pickq:
            codec = {4: kvq4, 2: kvq2}[width(g)]
            _CPU[key].append((codec.encode(synth.bf16_bits_to_f32(dk[b, g]),
                                           synth.bf16_bits_to_f32(dv[b, g])),
                              dq[b, g * G:(g + 1) * G], L, width(g)))
    ctx = mp.get_context("fork")
    qwall = {}
    with ctx.Pool(cores) as pool:
        t0 = time.perf_counter()
        pool.map(_cpu_prefill_block, qbs, chunksize=1)
        pwall = time.perf_counter() - t0
        t0 = time.perf_counter()
        pool.map(_cpu_decode_head, [(i, hh) for i in range(len(picks)) for hh in range(G)],
                 chunksize=1)
        dwall = time.perf_counter() - t0
        for key, _ in qkeys:
            t0 = time.perf_counter()
            pool.map(_cpu_decode_q_head, [(key, i) for i in range(len(pickq))], chunksize=1)
            qwall[key] = time.perf_counter() - t0
    _CPU.clear()
    host = dict(host_cores=os.cpu_count(), host_cpu=_cpu_model())
    pairs = sum(64 * (qb * 64) + 64 * 65 // 2 for qb in qbs)
    pre = dict(value=float(4.0 * d * pairs / pwall / 1e12), unit="TFLOP/s", cores=cores,
               kind="oracle", **host,
               sample=f"{pname} head 0: {nblocks} of {nt} query blocks spread evenly, "
                      f"tau=inf, fp64 numpy, {pwall:.1f} s wall")
    kv_bytes = len(picks) * 2.0 * L * d * 2
    dec = dict(value=float(kv_bytes / dwall / 1e9), unit="GB/s", cores=cores, kind="oracle", **host,
               sample=f"decode_128k: {len(picks)} KV heads x {G} query heads, tau=inf, "
                      f"fp64 numpy, {dwall:.1f} s wall")
    quant = {}
    for key, bits in (("dq4", 4), ("dq2", 2)):
        nb = qcache_bytes(bits, len(pickq), 1, L, d)
        quant[key] = dict(value=float(nb / qwall[key] / 1e9), unit="GB/s", cores=cores,
                          kind="oracle", **host,
                          sample=f"decode_128k over the {bits}-bit cache: {len(pickq)} KV heads "
                                 f"x {G} query heads, dequantise + fp64 decode oracle, tau=inf, "
                                 f"{qwall[key]:.1f} s wall")
    if hybrid_bits is not None:
        nb = sum(qcache_bytes(hybrid_bits[g], 1, 1, L, d) for _, g in pickq)
        quant["dqh"] = dict(value=float(nb / qwall["dqh"] / 1e9), unit="GB/s", cores=cores,
                            kind="oracle", **host,
                            sample=f"decode_128k over the hybrid cache: {len(pickq)} KV heads "
                                   f"(each at its width) x {G} query heads, dequantise + fp64 "
                                   f"decode oracle, tau=inf, {qwall['dqh']:.1f} s wall")
    return pre, dec, quant["dq4"], quant["dq2"], quant.get("dqh")


# ---------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--reading", default="S", choices=["S", "P"])
    ap.add_argument("--only", default="both",
                    choices=["both", "prefill", "decode", "decode_q4", "decode_q2",
                             "decode_hybrid", "prefill_qk8", "prefill_pv8", "prefill_qkv8",
                             "prefill_qki8"],
                    help="profile one leg only (the JSON line then reports that leg)")
    ap.add_argument("--no-q4", action="store_true",
                    help="skip the 4-bit, 2-bit and hybrid KV-cache decodes measured beside "
                         "the step")
    ap.add_argument("--no-sas", action="store_true",
                    help="skip the decodes and the prefill with the SAS exponential measured "
                         "beside the step")
    ap.add_argument("--prefill-workload", default="prefill_128k",
                    choices=["prefill_128k", "prefill_32k", "prefill_8k"],
                    help="prefill shape of the step (default: the 128K one)")
    ap.add_argument("--tau", type=float, default=math.inf,
                    help="tau of the timed prefill calls (default inf: the step); for counter runs")
    ap.add_argument("--no-qk8", action="store_true",
                    help="skip the prefills with 8-bit products (fp8 QK^T, fp8 PV, both; "
                         "int8 QK^T) measured beside the step")
    ap.add_argument("--no-other-prefill", action="store_true",
                    help="skip the 8K and 32K causal prefill workloads timed beside the step")
    ap.add_argument("--copy-ref-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB, a reference "
                         "dispatch of known traffic for hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: --gpus {args.gpus} is not supported "
              "(this attention path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    import torch

    import long_context_tiled_amd as lib
    import synth

    lib.load()
    dev = torch.device("cuda:0")
    pname = args.prefill_workload
    pcfg = synth.workload(pname)
    dcfg = synth.workload("decode_128k")
    t0 = time.perf_counter()
    pq, pk, pv = synth.make_prefill(pcfg, reading=args.reading)
    dq, dk, dv = synth.make_decode(dcfg, reading=args.reading)
    print(f"# inputs generated in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)

    B, Hq, N, d = pq.shape
    Hkv = pk.shape[1]
    tq, tk, tv = _dev(pq, dev), _dev(pk, dev), _dev(pv, dev)
    po = torch.empty((B, Hq, N, d), dtype=torch.float32, device=dev)
    plse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    nt = (N + 63) // 64
    pmask = torch.empty((B, Hq, nt, nt), dtype=torch.uint8, device=dev)
    DB, DHq, Dd = dq.shape
    DHkv, L = dk.shape[1], dk.shape[2]
    uq, uk, uv = _dev(dq, dev), _dev(dk, dev), _dev(dv, dev)
    do = torch.empty((DB, DHq, Dd), dtype=torch.float32, device=dev)
    dlse = torch.empty((DB, DHq), dtype=torch.float32, device=dev)
    dnt = (L + 63) // 64
    dmask = torch.empty((DB, DHq, dnt), dtype=torch.uint8, device=dev)
    ws = torch.empty(lib.attn_decode_workspace_bytes(DB, DHq, L, Dd), dtype=torch.uint8,
                     device=dev)
    torch.cuda.synchronize()

    if args.copy_ref_mib > 0:
        n = args.copy_ref_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# copy reference: {args.copy_ref_mib} MiB read + {args.copy_ref_mib} MiB written",
              file=sys.stderr, flush=True)
        del src, dst

    run_p = args.only in ("both", "prefill")
    run_d = args.only in ("both", "decode")
    # quantised-cache decodes measured beside the step (width in bits)
    widths = [w for w in (4, 2)
              if args.only == f"decode_q{w}" or (args.only == "both" and not args.no_q4)]
    run_hy = args.only == "decode_hybrid" or (args.only == "both" and not args.no_q4)

    # Timed calls pass no skip-mask buffer (the mask is an optional output
    # for analysis); the tau sweep takes one extra masked call per tau to
    # count skipped tiles, outside its timed calls.
    def prefill(tau, mask=None):
        lib.attn_prefill(tq, tk, tv, po, plse, True, tau, mask)

    def decode(tau, mask=None):
        lib.attn_decode(uq, uk, uv, do, dlse, tau, ws, mask)

    for _ in range(args.warmup):
        if run_p:
            prefill(args.tau)
        if run_d:
            decode(math.inf)
    torch.cuda.synchronize()

    tp, td = Timer(), Timer()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for _ in range(args.steps):
        if run_p:
            with tp:
                prefill(args.tau)
        if run_d:
            with td:
                decode(math.inf)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3 / args.steps
    print(f"# timed {args.steps} steps: {wall_ms:.2f} ms/step", file=sys.stderr, flush=True)

    dense_flops = prefill_dense_flops(B, Hq, N, d)
    out = dict(metric=METRIC, n_gpus=1, steps=args.steps, warmup=args.warmup,
               ms_per_step=round(wall_ms, 4), higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype="bf16", data="synthetic")
    cfg = dict(workload=f"{pname} + decode_128k, tau=inf" if math.isinf(args.tau) else
               f"{pname} at tau={args.tau} + decode_128k, tau=inf",
               prefill=dict(B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, causal=True),
               decode=dict(B=DB, Hq=DHq, Hkv=DHkv, L=L, d=Dd, split=4096),
               reading=args.reading, inputs="seeded N(0,1) bf16 + sinks/band/window")
    out["config"] = cfg

    if run_p and not math.isinf(args.tau):
        prefill(args.tau, pmask)
        _, vis, kept = prefill_exec_flops(pmask.cpu().numpy(), d)
        out["tiles_at_tau"] = dict(tau=args.tau, visited=vis, kept=kept)
    if run_p:
        p_ms = float(np.mean(tp.ms()))
        p_tf = dense_flops / (p_ms * 1e-3) / 1e12
        out.update(value=round(p_tf, 3), unit="TFLOP/s")
        out["roofline"] = dict(bound="mfma", achieved=round(p_tf, 3), peak=PEAK_BF16_TFLOPS,
                               unit="TFLOP/s", frac=round(p_tf / PEAK_BF16_TFLOPS, 4),
                               traffic=(measured_traffic("prefill")
                                        if pname == "prefill_128k" else None),
                               kernel="prefill_kernel<128,true,4>",
                               avg_ms=round(p_ms, 4),
                               per_launch_flops=dense_flops)
    if run_d:
        d_ms = float(np.mean(td.ms()))
        dense_b, _ = decode_bytes(DB, DHkv, L, Dd)
        gbs = dense_b / (d_ms * 1e-3) / 1e9
        dec = dict(value=round(gbs, 2), unit="GB/s", ms=round(d_ms, 4),
                   traffic=measured_traffic("decode"),
                   frac_of_hbm=round(gbs / PEAK_HBM_GBS, 4),
                   per_call_kv_bytes=dense_b, kernels="decode_split_kernel<128> + decode_merge_kernel<128>")
        out["decode"] = dec
        if not run_p:
            out.update(value=round(gbs, 2), unit="GB/s")
            out["roofline"] = dict(bound="hbm", achieved=round(gbs, 2), peak=PEAK_HBM_GBS,
                                   unit="GB/s", frac=round(gbs / PEAK_HBM_GBS, 4),
                                   traffic=measured_traffic("decode"),
                                   kernel="decode_split_kernel<128>",
                                   avg_ms=round(d_ms, 4), per_launch_bytes=dense_b)

    if run_d and not args.no_sas:
        # The bf16 decode with the SAS exponential (degree 2 and 3): its time
        # and how far its outputs move from the exact decode's on this input.
        decode(math.inf)
        torch.cuda.synchronize()
        o_ex, l_ex = do.clone(), dlse.clone()
        for deg in (2, 3):
            warm_up(lambda: lib.attn_decode_sas(uq, uk, uv, do, dlse, math.inf, deg, ws),
                    args.warmup)
            ts = Timer()
            torch.cuda.synchronize()
            for _ in range(args.steps):
                with ts:
                    lib.attn_decode_sas(uq, uk, uv, do, dlse, math.inf, deg, ws)
            torch.cuda.synchronize()
            s_ms = float(np.mean(ts.ms()))
            dense_b, _ = decode_bytes(DB, DHkv, L, Dd)
            out[f"decode_sas{deg}"] = dict(
                value=round(dense_b / (s_ms * 1e-3) / 1e9, 2), unit="GB/s", ms=round(s_ms, 4),
                max_abs_o_drift=float((do - o_ex).abs().max()),
                max_abs_lse_drift=float((dlse - l_ex).abs().max()),
                kernels=f"decode_split_kernel<128, {deg}> + decode_merge_kernel<128>")
        del o_ex, l_ex

    # the split kernel each width runs at decode_128k's group size (G = 8):
    # the 2-bit decode packs two KV groups per wave for G <= 8
    qkern = {4: "decode_q4_split_kernel<128>", 2: "decode_q2_pair_kernel<128>"}
    qdecode = {}
    for w in widths:
        # The same decode workload over a w-bit KV cache: quantised (the first
        # call timed on its own, then rewrites of the cache timed warm), then
        # attn_decode_q{w} timed like the bf16 decode.
        quantize = getattr(lib, f"quantize_q{w}")
        tq0 = Timer()
        with tq0:
            cache = quantize(uk, uv)
        torch.cuda.synchronize()
        qb = qcache_bytes(w, DB, DHkv, L, Dd)
        entry = getattr(lib, f"attn_decode_q{w}")

        def decode_q(tau, mask=None, entry=entry, cache=cache):
            entry(uq, cache, L, do, dlse, tau, ws, mask)

        qdecode[w] = decode_q
        requant = getattr(lib, f"attn_kv_quantize_q{w}")
        qz_ms, qz_gbs = time_quantiser(lambda: requant(uk, uv, cache), list(cache.values()), uk, uv,
                                       args.steps, args.warmup)
        warm_up(lambda: decode_q(math.inf), args.warmup)
        tqw = Timer()
        torch.cuda.synchronize()
        for _ in range(args.steps):
            with tqw:
                decode_q(math.inf)
        torch.cuda.synchronize()
        q_ms = float(np.mean(tqw.ms()))
        # the same decode with the SAS exponential (degree 2), timed alike
        dec_sas = getattr(lib, f"decode_q{w}")
        warm_up(lambda: dec_sas(uq, cache, L, math.inf, workspace=ws, sas=2), args.warmup)
        tsw = Timer()
        torch.cuda.synchronize()
        for _ in range(args.steps):
            with tsw:
                dec_sas(uq, cache, L, math.inf, workspace=ws, sas=2)
        torch.cuda.synchronize()
        sas_ms = float(np.mean(tsw.ms()))
        dense_b, _ = decode_bytes(DB, DHkv, L, Dd)
        gbs_q = qb / (q_ms * 1e-3) / 1e9
        leg = f"decode_q{w}"
        out[leg] = dict(value=round(gbs_q, 2), unit="GB/s", ms=round(q_ms, 4),
                        frac_of_hbm=round(gbs_q / PEAK_HBM_GBS, 4), per_call_bytes=qb,
                        gbs_bf16_equivalent=round(dense_b / (q_ms * 1e-3) / 1e9, 2),
                        traffic=measured_traffic(leg),
                        quantise_ms=round(qz_ms, 4), quantise_gbs=round(qz_gbs, 1),
                        quantise_first_ms=round(float(tq0.ms()[0]), 4),
                        sas2_ms=round(sas_ms, 4),
                        kernels=f"{qkern[w]} + decode_merge_kernel<128>")
        if args.only == leg:
            # the step is this leg alone: its per-call time, its workload
            out.update(value=round(gbs_q, 2), unit="GB/s", ms_per_step=round(q_ms, 4))
            out["config"]["workload"] = f"decode_128k over the {w}-bit KV cache, tau=inf"
            out["roofline"] = dict(bound="hbm", achieved=round(gbs_q, 2), peak=PEAK_HBM_GBS,
                                   unit="GB/s", frac=round(gbs_q / PEAK_HBM_GBS, 4),
                                   traffic=measured_traffic(leg),
                                   kernel=qkern[w],
                                   avg_ms=round(q_ms, 4), per_launch_bytes=qb)

    hdecode = None
    if run_hy:
        # The same decode workload over a hybrid cache, its KV heads
        # alternating 4 bits (even heads) and 2 bits (odd heads): quantised
        # (first call and warm rewrites timed), then attn_decode_hybrid timed
        # like the rest.
        hbits = tuple(4 if g % 2 == 0 else 2 for g in range(DHkv))
        tqh = Timer()
        with tqh:
            hcache = lib.quantize_hybrid(uk, uv, hbits)
        torch.cuda.synchronize()
        hb = sum(qcache_bytes(w, DB, hbits.count(w), L, Dd) for w in (4, 2))

        def hdecode(tau, mask=None):
            lib.attn_decode_hybrid(uq, hcache, L, do, dlse, tau, ws, mask)

        htensors = [x for w in ("q4", "q2") if hcache[w] is not None for x in hcache[w].values()]
        hqz_ms, hqz_gbs = time_quantiser(lambda: lib.attn_kv_quantize_hybrid(uk, uv, hcache),
                                         htensors, uk, uv, args.steps, args.warmup)
        warm_up(lambda: hdecode(math.inf), args.warmup)
        th = Timer()
        torch.cuda.synchronize()
        for _ in range(args.steps):
            with th:
                hdecode(math.inf)
        torch.cuda.synchronize()
        h_ms = float(np.mean(th.ms()))
        gbs_h = hb / (h_ms * 1e-3) / 1e9
        dense_b, _ = decode_bytes(DB, DHkv, L, Dd)
        hkern = "decode_q4_split_kernel<128> + decode_q2_pair_kernel<128>"
        out["decode_hybrid"] = dict(value=round(gbs_h, 2), unit="GB/s", ms=round(h_ms, 4),
                                    frac_of_hbm=round(gbs_h / PEAK_HBM_GBS, 4),
                                    per_call_bytes=hb, kv_bits=list(hbits),
                                    gbs_bf16_equivalent=round(dense_b / (h_ms * 1e-3) / 1e9, 2),
                                    quantise_ms=round(hqz_ms, 4), quantise_gbs=round(hqz_gbs, 1),
                                    quantise_first_ms=round(float(tqh.ms()[0]), 4),
                                    traffic=measured_traffic("decode_hybrid"),
                                    kernels=f"{hkern} + decode_merge_kernel<128>")
        if args.only == "decode_hybrid":
            out.update(value=round(gbs_h, 2), unit="GB/s", ms_per_step=round(h_ms, 4))
            out["config"]["workload"] = ("decode_128k over the hybrid cache (KV heads "
                                         "alternating 4 and 2 bits), tau=inf")
            out["roofline"] = dict(bound="hbm", achieved=round(gbs_h, 2), peak=PEAK_HBM_GBS,
                                   unit="GB/s", frac=round(gbs_h / PEAK_HBM_GBS, 4),
                                   traffic=measured_traffic("decode_hybrid"), kernel=hkern,
                                   avg_ms=round(h_ms, 4), per_launch_bytes=hb)

    # The same prefill with 8-bit operands (the quantisers and the prefill
    # kernel, timed per call like the step): fp8 QK^T (attn_prefill_qk8), fp8
    # P.V with bf16 QK^T and with fp8 QK^T (attn_prefill_pv8), int8 QK^T
    # (attn_prefill_qki8; int8 MFMAs run at the fp8 rate).
    lowp = [("prefill_qk8", "fp8 QK^T, bf16 PV", PEAK_QK8_TFLOPS,
             "prefill_kernel<128,true,4,5,false,true,0,false,false>",
             "quant_fp8_kernel<128> x 2 + ",
             "QK^T on fp8 E4M3 codes (64-row tiles, fp32 scales), PV in bf16; time "
             "includes quantising Q and K"),
            ("prefill_pv8", "bf16 QK^T, fp8 PV", PEAK_QK8_TFLOPS,
             "prefill_kernel<128,true,4,5,false,false,0,true,false>",
             "v8_tile_max_kernel<128> + v8_head_scale_kernel + v8_quant_kernel<128> + ",
             "PV on fp8 E4M3 (V with one scale per KV head, probabilities rounded to E4M3 "
             "relative to the reference maximum), QK^T in bf16; time includes quantising V"),
            ("prefill_qkv8", "fp8 QK^T, fp8 PV", PEAK_FP8_TFLOPS,
             "prefill_kernel<128,true,4,5,false,true,0,true,false>",
             "quant_fp8_kernel<128> x 2 + v8 quantisers + ",
             "both products on fp8 E4M3 (QK^T as prefill_qk8, PV as prefill_pv8); time "
             "includes quantising Q, K and V"),
            ("prefill_qki8", "int8 QK^T, bf16 PV", PEAK_QK8_TFLOPS,
             "prefill_kernel<128,true,4,5,false,true,0,false,true>",
             "quant_i8_kernel<128> x 2 + ",
             "QK^T on symmetric int8 codes (64-row tiles, fp32 scales; exact int32 "
             "products), PV in bf16; time includes quantising Q and K")]
    for leg, dtype8, peak8, kern8, quants8, note8 in lowp:
        if not (args.only == leg or (args.only == "both" and not args.no_qk8)):
            continue
        if leg in ("prefill_qk8", "prefill_qki8"):
            qws = torch.empty(lib.attn_prefill_qk8_workspace_bytes(B, Hq, Hkv, N, d),
                              dtype=torch.uint8, device=dev)

            def prefill8(tau, mask=None, qws=qws, i8=leg == "prefill_qki8"):
                lib.attn_prefill_qk8(tq, tk, tv, po, plse, True, tau, qws, mask, int8=i8)
        else:
            both = leg == "prefill_qkv8"
            qws = torch.empty(lib.attn_prefill_pv8_workspace_bytes(B, Hq, Hkv, N, d, both),
                              dtype=torch.uint8, device=dev)

            def prefill8(tau, mask=None, qws=qws, both=both):
                lib.attn_prefill_pv8(tq, tk, tv, po, plse, True, tau, qws, both, mask)

        warm_up(lambda: prefill8(args.tau), args.warmup)
        t8 = Timer()
        torch.cuda.synchronize()
        for _ in range(args.steps):
            with t8:
                prefill8(args.tau)
        torch.cuda.synchronize()
        q8_ms = float(np.mean(t8.ms()))
        q8_tf = dense_flops / (q8_ms * 1e-3) / 1e12
        if not math.isinf(args.tau):
            prefill8(args.tau, pmask)
            _, vis8, kept8 = prefill_exec_flops(pmask.cpu().numpy(), d)
            out[f"tiles_at_tau_{leg[8:]}"] = dict(tau=args.tau, visited=vis8, kept=kept8)
        # drift from the exact bf16 prefill on the same inputs
        prefill(math.inf)
        torch.cuda.synchronize()
        o_ex, l_ex = po.clone(), plse.clone()
        prefill8(math.inf)
        torch.cuda.synchronize()
        drift_o = float((po - o_ex).abs().max())
        drift_l = float((plse - l_ex).abs().max())
        del o_ex, l_ex
        taus8 = []
        if not args.no_sweep:
            for tau in pcfg["taus"][1:]:
                t = Timer()
                for _ in range(3):
                    with t:
                        prefill8(tau)
                torch.cuda.synchronize()
                ms = float(np.median(t.ms()))
                prefill8(tau, pmask)
                ex, vis, kept = prefill_exec_flops(pmask.cpu().numpy(), d)
                taus8.append(dict(tau=str(tau), ms=round(ms, 4),
                                  skip_fraction=round(1 - kept / vis, 4),
                                  tiles_visited=vis, tiles_kept=kept,
                                  tflops_dense=round(dense_flops / ms / 1e9, 3),
                                  tflops_executed=round(ex / ms / 1e9, 3)))
        out[leg] = dict(
            value=round(q8_tf, 3), unit="TFLOP/s", ms=round(q8_ms, 4),
            frac_of_bf16_peak=round(q8_tf / PEAK_BF16_TFLOPS, 4),
            frac_of_mixed_peak=round(q8_tf / peak8, 4),
            mixed_peak=round(peak8, 1),
            max_abs_o_drift=drift_o, max_abs_lse_drift=drift_l, tau_sweep=taus8,
            traffic=measured_traffic(leg),
            kernels=quants8 + kern8, note=note8)
        if args.only == leg:
            out.update(value=round(q8_tf, 3), unit="TFLOP/s", ms_per_step=round(q8_ms, 4),
                       dtype=dtype8)
            out["config"]["workload"] = f"{pname} with {dtype8}, tau=inf"
            out["roofline"] = dict(bound="mfma", achieved=round(q8_tf, 3), peak=peak8,
                                   unit="TFLOP/s", frac=round(q8_tf / peak8, 4),
                                   traffic=measured_traffic(leg),
                                   kernel=kern8 + " + quantisers",
                                   avg_ms=round(q8_ms, 4), per_launch_flops=dense_flops)
        del qws
        torch.cuda.empty_cache()

    if run_p and args.only == "both" and not args.no_sas:
        # The step's prefill with the SAS exponential (degree 2 and 3): time,
        # and how far its outputs move from the exact prefill's on this input.
        prefill(math.inf)
        torch.cuda.synchronize()
        o_ex, l_ex = po.clone(), plse.clone()
        for deg in (2, 3):
            def prefill_sas(tau, mask=None, deg=deg):
                lib.attn_prefill_sas(tq, tk, tv, po, plse, True, tau, deg, mask)

            warm_up(lambda: prefill_sas(math.inf), args.warmup)
            ts = Timer()
            torch.cuda.synchronize()
            for _ in range(args.steps):
                with ts:
                    prefill_sas(math.inf)
            torch.cuda.synchronize()
            s_ms = float(np.mean(ts.ms()))
            drift_o = float((po - o_ex).abs().max())
            drift_l = float((plse - l_ex).abs().max())
            sweep = []
            if not args.no_sweep:
                for tau in pcfg["taus"][1:]:
                    t = Timer()
                    for _ in range(3):
                        with t:
                            prefill_sas(tau)
                    torch.cuda.synchronize()
                    sweep.append(dict(tau=str(tau), ms=round(float(np.median(t.ms())), 4)))
            out[f"prefill_sas{deg}"] = dict(
                value=round(dense_flops / (s_ms * 1e-3) / 1e12, 3), unit="TFLOP/s",
                ms=round(s_ms, 4), vs_exact=round(p_ms / s_ms, 4),
                max_abs_o_drift=drift_o, max_abs_lse_drift=drift_l, tau_sweep=sweep,
                kernel=f"prefill_kernel<128,true,4,5,false,false,{deg},false,false>")
        del o_ex, l_ex

    if run_p and args.only == "both" and not args.no_other_prefill:
        # the other causal prefill workloads, timed alone like the step's
        # prefill (mean of K calls at tau = inf, median of 3 per tau)
        for oname in ("prefill_8k", "prefill_32k"):
            if oname == pname:
                continue
            ocfg = synth.workload(oname)
            oq, ok_, ov = synth.make_prefill(ocfg, reading=args.reading)
            OB, OHq, ON, Od = oq.shape
            xq, xk, xv = _dev(oq, dev), _dev(ok_, dev), _dev(ov, dev)
            xo = torch.empty((OB, OHq, ON, Od), dtype=torch.float32, device=dev)
            xl = torch.empty((OB, OHq, ON), dtype=torch.float32, device=dev)
            ont = (ON + 63) // 64
            xm = torch.empty((OB, OHq, ont, ont), dtype=torch.uint8, device=dev)

            def oprefill(tau, mask=None):
                lib.attn_prefill(xq, xk, xv, xo, xl, True, tau, mask)

            warm_up(lambda: oprefill(math.inf), args.warmup)
            to = Timer()
            torch.cuda.synchronize()
            for _ in range(args.steps):
                with to:
                    oprefill(math.inf)
            torch.cuda.synchronize()
            o_ms = float(np.mean(to.ms()))
            of = prefill_dense_flops(OB, OHq, ON, Od)
            entry = dict(value=round(of / (o_ms * 1e-3) / 1e12, 3), unit="TFLOP/s",
                         ms=round(o_ms, 4),
                         frac_of_peak=round(of / (o_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         per_call_flops=of,
                         shape=dict(B=OB, Hq=OHq, Hkv=ok_.shape[1], N=ON, d=Od, causal=True))
            taus = []
            for tau in ocfg["taus"][1:]:
                t = Timer()
                for _ in range(3):
                    with t:
                        oprefill(tau)
                torch.cuda.synchronize()
                ms = float(np.median(t.ms()))
                oprefill(tau, xm)
                ex, vis, kept = prefill_exec_flops(xm.cpu().numpy(), Od)
                taus.append(dict(tau=str(tau), ms=round(ms, 4), skip_fraction=round(1 - kept / vis, 4),
                                 tflops_dense=round(of / ms / 1e9, 3),
                                 tflops_executed=round(ex / ms / 1e9, 3)))
            entry["tau_sweep"] = taus
            out[oname] = entry
            del xq, xk, xv, xo, xl, xm
            torch.cuda.empty_cache()

    if not args.no_sweep:
        sweep = []
        for tau in pcfg["taus"] if run_p else []:
            t = Timer()
            for _ in range(3):
                with t:
                    prefill(tau)
            torch.cuda.synchronize()
            ms = float(np.median(t.ms()))
            prefill(tau, pmask)
            m = pmask.cpu().numpy()
            ex, vis, kept = prefill_exec_flops(m, d)
            sweep.append(dict(leg=pname, tau=str(tau), ms=round(ms, 4),
                              skip_fraction=round(1 - kept / vis, 4),
                              tiles_visited=vis, tiles_kept=kept,
                              tflops_dense=round(dense_flops / ms / 1e9, 3),
                              tflops_executed=round(ex / ms / 1e9, 3)))
        for tau in dcfg["taus"] if run_d else []:
            t = Timer()
            for _ in range(3):
                with t:
                    decode(tau)
            torch.cuda.synchronize()
            ms = float(np.median(t.ms()))
            decode(tau, dmask)
            m = dmask.cpu().numpy()
            dense_b, act_b = decode_bytes(DB, DHkv, L, Dd, m, DHq // DHkv)
            sweep.append(dict(leg="decode_128k", tau=str(tau), ms=round(ms, 4),
                              skip_fraction=round(float((m == 1).mean()), 4),
                              gbs_dense=round(dense_b / ms / 1e6, 2),
                              gbs_actual=round(act_b / ms / 1e6, 2)))
        for w in widths:
            for tau in dcfg["taus"]:
                t = Timer()
                for _ in range(3):
                    with t:
                        qdecode[w](tau)
                torch.cuda.synchronize()
                ms = float(np.median(t.ms()))
                qdecode[w](tau, dmask)
                m = dmask.cpu().numpy()
                act_b = qcache_bytes(w, DB, DHkv, L, Dd, m, DHq // DHkv)
                sweep.append(dict(leg=f"decode_128k_q{w}", tau=str(tau), ms=round(ms, 4),
                                  skip_fraction=round(float((m == 1).mean()), 4),
                                  gbs_actual=round(act_b / ms / 1e6, 2)))
        if hdecode is not None:
            for tau in dcfg["taus"]:
                t = Timer()
                for _ in range(3):
                    with t:
                        hdecode(tau)
                torch.cuda.synchronize()
                ms = float(np.median(t.ms()))
                hdecode(tau, dmask)
                m = dmask.cpu().numpy()
                G = DHq // DHkv
                act_b = sum(qcache_bytes(w, DB, hbits.count(w), L, Dd,
                                         m.reshape(DB, DHkv, G, -1)[:, [g for g in range(DHkv)
                                                                        if hbits[g] == w]]
                                         .reshape(DB, -1, m.shape[-1]), G)
                            for w in (4, 2))
                sweep.append(dict(leg="decode_128k_hybrid", tau=str(tau), ms=round(ms, 4),
                                  skip_fraction=round(float((m == 1).mean()), 4),
                                  gbs_actual=round(act_b / ms / 1e6, 2)))
        out["tau_sweep"] = sweep

    if not args.no_cpu:
        print("# cpu baseline (fp64 oracle on a bounded sample)", file=sys.stderr, flush=True)
        pre, dec, dq4, dq2, dqh = cpu_baseline(
            pq, pk, pv, dq, dk, dv, pname=pname,
            hybrid_bits=tuple(4 if g % 2 == 0 else 2 for g in range(dk.shape[1])) if run_hy
            else None)
        legs = {"both": pre, "prefill": pre, "decode": dec, "decode_q4": dq4, "decode_q2": dq2,
                "decode_hybrid": dqh}
        # the 8-bit prefill legs report the exact prefill oracle's rate (their
        # oracles are that oracle on quantised operands)
        out["cpu_baseline"] = legs.get(args.only, pre)
        out["cpu_baseline_decode"] = dec
        out["cpu_baseline_decode_q4"] = dq4
        out["cpu_baseline_decode_q2"] = dq2
        if dqh is not None:
            out["cpu_baseline_decode_hybrid"] = dqh
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
