#!/usr/bin/env python3
"""Benchmark of the blockwise low-bit codec on one MI355X.

Workload: one 64 Mi-element binary32 gradient bucket (Student-t with 3
degrees of freedom, times 1e-3, seed 1), block 256, stochastic rounding keyed
by seed 42, bitwidths 1, 2, 4 and 8.  One step is one pass of the whole hot
path over that bucket, as the single-GPU share of a low-bit data-parallel
exchange:

  for b in (1, 2, 4, 8):
      compress the bucket                      (quantize + pack, SR)
      local reduce of this GPU's 8 Mi share:   8 peer chunks (the 8 slices of
                                               the packed bucket) decoded,
                                               summed in peer order, recompressed
      decompress the bucket                    (unpack + dequantize)
  error-feedback compress of the bucket        (b = 4, residual carried over steps)
  weight-difference compress + apply           (64 Mi bfloat16 shard, b = 4, B = 64)

The timed step is issued as a low-bit data-parallel exchange would pipeline
independent buckets: the error-feedback compress alone on the main stream,
then the chains {1-bit, 4-bit, weight difference} on the main stream
concurrently with {2-bit, 8-bit} on a second HIP stream, joined at the
step's end (each chain keeps its own order; chains write no common buffer).
`config.ms_per_step_one_stream` gives the same step with every stage on one
stream, and `kernels` the per-stage durations from that serial form.

`value` counts full-precision (binary32-equivalent) bytes through the step's
15 stage passes -- each stage touches the 64 Mi elements once -- divided by
the step time.  Inputs are resident in HBM before the timed region.

The `roofline` object covers the kernel with the largest share of the step,
timed with HIP events on the stream the kernels run on; `traffic` comes from
the committed rocprofv3 counter summary when it was taken on the current
kernel sources.  `roofline.copy_kernel_GBps` is a plain copy's rate and
`roofline.pattern` times the dominant kernel alone next to a reference
kernel with its memory pattern and none of its arithmetic (for the EF
compress: y += x in place over the bucket).  `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload.

`next_rows` (not part of `value`) times the extension kernels alone on
their own workloads: EF21 compress and Hadamard-smoothed compress /
decompress of the bucket, and the local reduce of 8 peer chunks of 32 Mi with
stage-2 error feedback (b4 B128) and with two-level requantization (8-bit
B512 peers to 4-bit B128).  `roundtrip_4mib` times the 2^20-element
compress + decompress once and over a ring of 256 distinct buffers, issued
eagerly and from a HIP graph (launch-bound at this size).  `configs` times
the kernels of the other workload configurations at full size: EF compress of
128 Mi bfloat16 gradients, the 8 x 32 Mi local reduce (without and with the
binary32 sum written, each also as a fraction of a reference kernel that only
reads the peers' streams with the reduce's access pattern), and weight-difference compress / apply of an 840 Mi
bfloat16 shard.  `size_sweep` gives the latency of one 4-bit compress over
2^10..2^28 elements beside the CPU oracle's, as a latency curve.  Every
per-kernel entry also reports `input_GBps`, the full-precision bytes the
stage handles as stored per second.
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
BITS = (1, 2, 4, 8)
BLOCK = 256
SEED = 42
PEERS = 8
W_BITS, W_BLOCK = 4, 64
EF_BITS = 4
# How the timed step is issued: the chains run alone on the main stream
# first, then the chains of the second list on the main stream concurrently
# with those of the third list on a second stream ("b<bits>": compress ->
# local reduce -> decompress at that width; "wd": weight-difference compress
# -> apply; "ef": the error-feedback compress).
SCHEDULE = (["ef"], ["b1", "b4", "wd"], ["b2", "b8"])
METRIC = "quantize+pack / reduce-requant GB/s of fp32 input on 1 MI355X; % of HBM peak"

# demangled kernel names as rocprofv3 reports them
def kname_quant(bits, log2b, sr, dt, mode, tail=False, stream=False):
    """stream: the non-temporal-input form, taken by a plain or Hadamard-smoothed
    binary32 compress without LOWBIT_HINT_INPUT_REUSED."""
    ntx = str(bool(stream) and mode in (0, 4) and dt == 0 and not tail).lower()
    if bits == 1 and mode != 4:     # 1-bit compress: the coalesced sign kernel
        return f"void lowbit::sign_kernel<{log2b}, {dt}, {mode}, {str(tail).lower()}, {ntx}>" \
               f"(lowbit::QuantArgs, long)"
    if bits in (2, 4) and mode in (1, 3):     # 2- and 4-bit EF / EF21: the row layout
        return f"void lowbit::row_kernel<{bits}, {log2b}, {str(sr).lower()}, {dt}, {mode}, " \
               f"{str(tail).lower()}>(lowbit::QuantArgs, long)"
    return f"void lowbit::quantize_kernel<{bits}, {log2b}, {str(sr).lower()}, {dt}, {mode}, " \
           f"{str(tail).lower()}, {ntx}>(lowbit::QuantArgs, long)"


def kname_reduce(in_bits, bits, log2b, sr, ef=False, tail=False, sum_out=False, stream=True):
    """stream: the form that reads the peers' code words non-temporally (main
    kernel without LOWBIT_HINT_INPUT_REUSED)."""
    st = str(bool(stream) and not tail).lower()
    # 4-bit reduce with a residual or a binary32 sum output: the row layout
    if in_bits == bits == 4 and (ef or sum_out):
        return f"void lowbit::rowr_kernel<{bits}, {log2b}, {str(sr).lower()}, " \
               f"{str(ef).lower()}, {str(tail).lower()}, {st}>(lowbit::ReduceArgs, long)"
    return f"void lowbit::reduce_kernel<{in_bits}, {bits}, {log2b}, {str(sr).lower()}, " \
           f"{str(ef).lower()}, {str(tail).lower()}, {st}>(lowbit::ReduceArgs, long)"


def kname_hadamard_dequant(bits, log2b):
    return f"void lowbit::hadamard_dequant_kernel<{bits}, {log2b}>(lowbit::DequantArgs)"


def kname_dequant(bits, apply, dt):
    return f"void lowbit::dequant_kernel<{bits}, {apply}, {dt}>(lowbit::DequantArgs)"


KNAME_XOR = "lowbit::xor_streams_kernel(lowbit::XorArgs)"
KNAME_COPY = "lowbit::copy_kernel(float const*, float*, long)"
KNAME_ADD = "lowbit::add_inplace_kernel(float const*, float*, long)"


def kname_fold(bits):
    return f"void lowbit::fold_kernel<{bits}>(float const*, long, unsigned int*, long)"


def source_digest() -> str:
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "weight_communication_compression_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "lowbit.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str = None):
    """HBM bytes per launch of `kernel` from the committed counter summaries
    (the line measured on `workload` when there is one, else any line of that
    kernel), or None when there is none for the current sources."""
    digest = source_digest()
    other = None
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            if not line.startswith("traffic:"):
                continue
            parts = line[len("traffic:"):].strip().split(" | ")
            f = dict(kv.split("=", 1) for kv in parts[1:])
            if parts[0] != kernel or f.get("source") != digest:
                continue
            if workload is not None and f.get("workload") == workload:
                return float(f["bytes_per_launch"])
            if other is None:
                other = float(f["bytes_per_launch"])
    return other


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--next-rows", type=int, default=1,
                    help="also time the extension kernels, the configurations, the 4 MiB "
                         "roundtrip and the memory-system comparisons alone (1) or not (0)")
    ap.add_argument("--sweep", type=int, default=1,
                    help="with --next-rows 1, also time the 2^10..2^28 compress latency curve "
                         "(1) or not (0)")
    ap.add_argument("--cpu-sample", type=int, default=64 << 20,
                    help="elements of the bucket the CPU oracle processes (0 = skip)")
    ap.add_argument("--cpu-configs", type=int, default=1,
                    help="with --cpu-sample > 0, also time the CPU oracle on each workload "
                         "configuration, one thread and all threads (1) or not (0)")
    ap.add_argument("--only", default=None,
                    help="run only these measurements, '|'-separated: a group (next_rows, "
                         "configs, compress_pattern, memory_patterns, block_sweep) or one entry of "
                         "next_rows or configs by its "
                         "name; prints them as one JSON line instead of the step (for profiling "
                         "one workload at a time)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the codec shards by block-aligned ranges; collectives are not built)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from weight_communication_compression_amd import lowbit as L
    from weight_communication_compression_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = L.lib()
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)

    # ------------------------------------------------------------ inputs --
    N = synth.BUCKET_N
    share = N // PEERS
    x_host = synth.bucket_input(N)
    w_prev_h, w_new_h = synth.weight_pair(N)
    x = torch.from_numpy(x_host).to(dev)
    w_prev = torch.from_numpy(w_prev_h.view(np.int16)).to(dev).view(torch.bfloat16)
    w_new = torch.from_numpy(w_new_h.view(np.int16)).to(dev).view(torch.bfloat16)
    resid = torch.zeros(N, dtype=torch.float32, device=dev)
    y = torch.empty(N, dtype=torch.float32, device=dev)
    w_out = torch.empty_like(w_prev)
    if args.only:
        return run_only(args.only, L, lib, dev, stream, x, y)

    def qp(bits, block, sr=False, seed=0, off=0, hints=0):
        return L.QParams(bits, block, int(sr), hints, seed, off)

    P = ctypes.c_void_p
    stages = []      # (name, kernel name, algorithmic bytes, callable)
    keep = []        # keep ctypes objects alive
    results = {}     # the step's output buffers, checked against the oracle at the end

    nw, nb = L.num_words(N, EF_BITS), L.num_blocks(N, BLOCK)
    ec = torch.empty(nw, dtype=torch.int32, device=dev)
    es = torch.empty(nb, dtype=torch.float16, device=dev)
    qe = qp(EF_BITS, BLOCK, True, SEED, 0)
    keep += [ec, es, qe]
    a = (P(x.data_ptr()), L.F32, P(resid.data_ptr()), N, ctypes.byref(qe), P(ec.data_ptr()),
         P(es.data_ptr()))
    # the EF compress first, as in the timed schedule (it runs alone at the
    # start of each step); the kernel after it pays for the residual lines it
    # leaves dirty in the Infinity Cache
    stages.append((f"ef_compress b{EF_BITS}", kname_quant(EF_BITS, 8, True, 0, 1),
                   3 * N * 4 + nw * 4 + nb * 2, (lib.lowbit_ef_compress, a)))

    for b in BITS:
        nw, nb = L.num_words(N, b), L.num_blocks(N, BLOCK)
        codes = torch.empty(nw, dtype=torch.int32, device=dev)
        scales = torch.empty(nb, dtype=torch.float16, device=dev)
        # the step compresses the bucket again at the next width (and in the
        # next step), so its compresses keep the input in the caches
        q = qp(b, BLOCK, True, SEED, 0, L.HINT_INPUT_REUSED)
        keep += [codes, scales, q]
        a = (P(x.data_ptr()), L.F32, N, ctypes.byref(q), P(codes.data_ptr()),
             P(scales.data_ptr()))
        stages.append((f"quantize_pack b{b}", kname_quant(b, 8, b > 1, 0, 0),
                       N * 4 + nw * 4 + nb * 2, (lib.lowbit_quantize_pack, a)))

        snw, snb = L.num_words(share, b), L.num_blocks(share, BLOCK)
        cp = (P * PEERS)(*[codes.data_ptr() + p * snw * 4 for p in range(PEERS)])
        spp = (P * PEERS)(*[scales.data_ptr() + p * snb * 2 for p in range(PEERS)])
        rc = torch.empty(snw, dtype=torch.int32, device=dev)
        rs = torch.empty(snb, dtype=torch.float16, device=dev)
        # the decompress reads the same codes right after the reduce
        qi, qo = qp(b, BLOCK, hints=L.HINT_INPUT_REUSED), qp(b, BLOCK)
        keep += [cp, spp, rc, rs, qi, qo]
        a = (ctypes.cast(cp, P), ctypes.cast(spp, P), PEERS, share, ctypes.byref(qi),
             ctypes.byref(qo), P(rc.data_ptr()), P(rs.data_ptr()), None)
        stages.append((f"reduce_requant b{b}", kname_reduce(b, b, 8, False, stream=False),
                       (PEERS + 1) * (snw * 4 + snb * 2), (lib.lowbit_reduce_requant, a)))

        qd = qp(b, BLOCK)
        yb = torch.empty(N, dtype=torch.float32, device=dev)   # this bitwidth's decompressed bucket
        keep += [qd, yb]
        results[f"b{b}"] = (codes, scales, rc, rs, yb)
        a = (P(codes.data_ptr()), P(scales.data_ptr()), N, ctypes.byref(qd), P(yb.data_ptr()))
        stages.append((f"unpack_dequant b{b}", kname_dequant(b, 0, 0),
                       nw * 4 + nb * 2 + N * 4, (lib.lowbit_unpack_dequant, a)))

    nw, nb = L.num_words(N, W_BITS), L.num_blocks(N, W_BLOCK)
    wc = torch.empty(nw, dtype=torch.int32, device=dev)
    ws = torch.empty(nb, dtype=torch.float16, device=dev)
    qw = qp(W_BITS, W_BLOCK)
    keep += [wc, ws, qw]
    results["wd"] = (wc, ws)
    a = (P(w_new.data_ptr()), P(w_prev.data_ptr()), L.BF16, N, ctypes.byref(qw), P(wc.data_ptr()),
         P(ws.data_ptr()))
    stages.append((f"wdiff_compress b{W_BITS}", kname_quant(W_BITS, 6, False, 1, 2),
                   2 * N * 2 + nw * 4 + nb * 2, (lib.lowbit_wdiff_compress, a)))
    a = (P(w_prev.data_ptr()), P(wc.data_ptr()), P(ws.data_ptr()), N, ctypes.byref(qw),
         P(w_out.data_ptr()), L.BF16)
    stages.append((f"wdiff_apply b{W_BITS}", kname_dequant(W_BITS, 1, 1),
                   2 * N * 2 + nw * 4 + nb * 2, (lib.lowbit_wdiff_apply, a)))

    full_precision_bytes = len(stages) * N * 4

    def run(fn_args, h=None):
        fn, a = fn_args
        st = fn(*a) if h is None else fn(*a, h)
        if st != 0:
            raise L.LowbitError(st, fn.__name__)

    def step(timed_index=None, ev=None):
        """The stages in order on one stream (events around one stage)."""
        for i, (_, _, _, fa) in enumerate(stages):
            if i == timed_index:
                ev[0].record(stream)
                run(fa, sh)
                ev[1].record(stream)
            else:
                run(fa, sh)

    # The step as timed: the EF compress alone on the main stream, then the
    # independent chains (per bitwidth: compress -> reduce -> decompress; the
    # weight difference: compress -> apply) split over the main stream and
    # one more stream, so that one chain's launch ramp, tail and short
    # latency-bound reduces overlap the other's streaming kernels; joined at
    # the step's end.  Each chain keeps its own order on its stream, and
    # chains share no written buffer.
    side = torch.cuda.Stream(dev)          # default priority
    side_h = ctypes.c_void_p(side.cuda_stream)
    fork_ev, join_ev = torch.cuda.Event(), torch.cuda.Event()
    chain_of = lambda name: "ef" if name.startswith("ef_") else \
        "wd" if name.startswith("wdiff") else "b" + name.rsplit("b", 1)[1]
    lanes = [[i for c in SCHEDULE[1] for i, st in enumerate(stages) if chain_of(st[0]) == c],
             [i for c in SCHEDULE[2] for i, st in enumerate(stages) if chain_of(st[0]) == c]]
    solo = [i for c in SCHEDULE[0] for i, st in enumerate(stages) if chain_of(st[0]) == c]
    assert sorted(solo + lanes[0] + lanes[1]) == list(range(len(stages)))

    def step_overlapped(timed_index=None, ev=None):
        def go(i, h, st):
            if i == timed_index:
                ev[0].record(st)
                run(stages[i][3], h)
                ev[1].record(st)
            else:
                run(stages[i][3], h)
        for i in solo:
            go(i, sh, stream)
        fork_ev.record(stream)
        side.wait_event(fork_ev)
        for i in lanes[1]:
            go(i, side_h, side)
        for i in lanes[0]:
            go(i, sh, stream)
        join_ev.record(side)
        stream.wait_event(join_ev)

    # ------------------------------------------------------------ warmup --
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()

    # per-stage durations (untimed pass) to find the dominant kernel
    per_stage = []
    for i in range(len(stages)):
        evs = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            step(i, (e0, e1))
            evs.append((e0, e1))
        torch.cuda.synchronize()
        per_stage.append(sorted(e0.elapsed_time(e1) for e0, e1 in evs)[2])
    dom = max(range(len(stages)), key=lambda i: per_stage[i])

    # ------------------------------------------------------------- timed --
    for _ in range(max(1, args.warmup)):
        step_overlapped()
    resid.zero_()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step_overlapped(dom, evs[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    dom_ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / args.steps
    value = full_precision_bytes / (ms_per_step * 1e-3) / 1e9

    # the same step with every stage on one stream, for comparison
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_serial = (time.perf_counter() - t0) * 1e3 / args.steps

    # plain-copy reference on the same box (not part of the step): the copy
    # kernel's rate, each launch after a 1 GiB read that leaves the Infinity
    # Cache clean, and its hardware byte counters when profiled
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    copy_evs = []
    for _ in range(5):
        flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run((lib.lowbit_copy_f32, (P(x.data_ptr()), P(y.data_ptr()), N, sh)))
        e1.record(stream)
        copy_evs.append((e0, e1))
    torch.cuda.synchronize()
    copy_ms = sorted(e0.elapsed_time(e1) for e0, e1 in copy_evs)[2]
    copy_gbs = 2 * N * 4 / (copy_ms * 1e-3) / 1e9

    # the dominant kernel's memory pattern without its arithmetic, and the
    # kernel itself, each alone after the same flush: for the EF compress the
    # reference is y += x in place over the bucket (two binary32 streams read,
    # one rewritten); for any other dominant stage only the kernel is timed
    def alone(fn, reps=11):
        ts = []
        for _ in range(reps):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[reps // 2]

    name, kname, alg_bytes, dom_fa = stages[dom]
    dom_alone_ms = alone(lambda: run(dom_fa, sh))
    pattern = {"dominant_alone_us": round(dom_alone_ms * 1e3, 2),
               "dominant_alone_GBps": round(alg_bytes / (dom_alone_ms * 1e-3) / 1e9, 1)}
    if name.startswith("ef_compress"):
        # the same two buffers as the EF compress (gradient and residual):
        # two streams read at the same offsets are sensitive to where the
        # allocator placed them; the residual's contents are not used after
        # this point
        ref_y = resid
        ref_ms = alone(lambda: run((lib.lowbit_add_inplace_f32,
                                    (P(x.data_ptr()), P(ref_y.data_ptr()), N, sh))))
        ref_gbs = 3 * N * 4 / (ref_ms * 1e-3) / 1e9
        pattern.update({"reference": "y += x in place, 64 Mi binary32 (add_inplace_kernel)",
                        "reference_GBps": round(ref_gbs, 1),
                        "of_reference": round(pattern["dominant_alone_GBps"] / ref_gbs, 3)})
        del ref_y
    del flush

    achieved = alg_bytes / (dom_ms * 1e-3) / 1e9
    traffic = read_traffic(kname, "step")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "kernel": kname, "stage": name,
                "avg_launch_us": round(dom_ms * 1e3, 2), "algorithmic_bytes": alg_bytes,
                "timed_alone_in_step": dom in solo,
                "copy_kernel_GBps": round(copy_gbs, 1), "pattern": pattern}
    # full-precision bytes each stage handles, as stored: the fp32 bucket (the
    # 8 peers' fp32-equivalent share for the reduce), the two bf16 weight
    # tensors read by the weight-difference compress, the bf16 weights read by
    # the apply
    def input_bytes(stage):
        if stage.startswith("reduce_requant"):
            return PEERS * share * 4
        if stage.startswith("wdiff_compress"):
            return 2 * N * 2
        if stage.startswith("wdiff_apply"):
            return N * 2
        return N * 4

    kernels = {s[0]: {"us": round(per_stage[i] * 1e3, 2), "kernel": s[1], "alg_bytes": s[2],
                      "alg_GBps": round(s[2] / (per_stage[i] * 1e-3) / 1e9, 1),
                      "frac": round(s[2] / (per_stage[i] * 1e-3) / 1e9 / HBM_PEAK_GBS, 3),
                      "input_GBps": round(input_bytes(s[0]) / (per_stage[i] * 1e-3) / 1e9, 1)}
               for i, s in enumerate(stages)}

    # ----------------------------------------- extensions beyond the step --
    next_rows = measure_next_rows(L, lib, dev, stream, x) if args.next_rows else None
    roundtrip = measure_roundtrip(L, dev) if args.next_rows else None
    configs = measure_configs(L, dev) if args.next_rows else None
    compress_pattern = measure_compress_pattern(L, dev, x) if args.next_rows else None
    memory_patterns = measure_memory_patterns(L, dev) if args.next_rows else None
    sweep = measure_size_sweep(L, dev, args.cpu_sample > 0) if args.next_rows and args.sweep \
        else None

    # ------------------------------------------------------- CPU oracle --
    cpu = None
    if args.cpu_sample > 0:
        cpu, oracle_out = cpu_baseline(x_host, w_prev_h, w_new_h, min(args.cpu_sample, N),
                                       len(stages))
        # the step's outputs against the oracle's on the same inputs (the
        # EF compress once more from a zero residual, as the oracle ran it)
        n_chk = min(args.cpu_sample, N)
        e0 = torch.zeros(N, dtype=torch.float32, device=dev)
        ec0, es0 = L.ef_compress(x, e0, EF_BITS, BLOCK, True, SEED, 0)
        results["wd"] = results["wd"] + (w_out,)
        results["ef"] = (ec0, es0, e0)
        torch.cuda.synchronize()
        cpu["oracle_check"] = check_against_oracle(results, oracle_out, n_chk, N)
        del e0, ec0, es0
        threads = min(len(os.sched_getaffinity(0)), int(os.environ.get("OMP_NUM_THREADS", "16")))
        if threads > 1:
            cpu["all_cores"] = cpu_baseline_all_cores(x_host, w_prev_h, w_new_h,
                                                      min(args.cpu_sample, N), len(stages), threads)
        if args.cpu_configs:
            cpu["configs"] = cpu_baseline_configs(x_host, threads)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "gradient bucket: 64Mi fp32 Student-t(3) x 1e-3 (seed 1), block 256, "
                        "SR seed 42, bits 1/2/4/8; step = compress + 8-peer local reduce of "
                        "the 8Mi share + decompress per bitwidth, EF compress (b4), weight-diff "
                        "compress+apply (64Mi bf16, b4 B64)",
            "elements": N, "block_size": BLOCK, "bitwidths": list(BITS), "peers": PEERS,
            "value_counts": "binary32-equivalent bytes of the 15 stage passes / step time",
            "step_alg_GBps": round(sum(st[2] for st in stages) / (ms_per_step * 1e-3) / 1e9, 1),
            "step_alg_bytes": int(sum(st[2] for st in stages)),
            "schedule": f"{'+'.join(SCHEDULE[0])} alone on the main stream, then "
                        f"{'+'.join(SCHEDULE[1])} on the main stream concurrently with "
                        f"{'+'.join(SCHEDULE[2])} on a second stream, joined per step",
            "ms_per_step_one_stream": round(ms_serial, 4),
            "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    if next_rows is not None:
        out["next_rows"] = next_rows
    if roundtrip is not None:
        out["roundtrip_4mib"] = roundtrip
    if configs is not None:
        out["configs"] = configs
    if compress_pattern is not None:
        out["compress_pattern"] = compress_pattern
    if memory_patterns is not None:
        out["memory_patterns"] = memory_patterns
    if sweep is not None:
        out["size_sweep"] = sweep
    print(json.dumps(out), flush=True)
    return 0


def run_only(spec, L, lib, dev, stream, x, y):
    """The measurements named in `spec` and nothing else, printed as one JSON
    line: {"only": names, "copy_us", <group>: {entry: ...}}.  A plain copy of
    the 64 Mi binary32 bucket runs first, once, so that a byte-counter run of
    this command holds its own calibration kernel."""
    import torch
    names = [t.strip() for t in spec.split("|") if t.strip()]
    P = ctypes.c_void_p
    sh = ctypes.c_void_p(stream.cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    st = lib.lowbit_copy_f32(P(x.data_ptr()), P(y.data_ptr()), x.numel(), sh)
    e1.record(stream)
    if st != 0:
        raise L.LowbitError(st, "lowbit_copy_f32")
    torch.cuda.synchronize()
    out = {"only": names, "copy_us": round(e0.elapsed_time(e1) * 1e3, 2)}

    def want(group):
        return lambda name: group in names or name in names
    out["next_rows"] = measure_next_rows(L, lib, dev, stream, x, want=want("next_rows"))
    out["configs"] = measure_configs(L, dev, want=want("configs"))
    if "compress_pattern" in names:
        out["compress_pattern"] = measure_compress_pattern(L, dev, x)
    if "memory_patterns" in names:
        out["memory_patterns"] = measure_memory_patterns(L, dev)
    if "block_sweep" in names:
        out["block_sweep"] = measure_block_sweep(L, dev, x)
    print(json.dumps(out), flush=True)
    return 0


def measure_next_rows(L, lib, dev, stream, x, reps=20, want=None):
    """Kernels of the extensions beyond the step (not part of `value`): each
    timed alone with HIP events on `stream`, median of `reps` launches, every
    launch after a 1 GiB read that leaves the Infinity Cache clean.
    `want(name)` false: that entry is skipped.
    Returns {name: {"workload", "us", "alg_bytes", "alg_GBps", "frac"}}."""
    import torch
    from weight_communication_compression_amd import synth

    P = ctypes.c_void_p
    sh = ctypes.c_void_p(stream.cuda_stream)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    N = x.numel()
    out = {}

    def qp(bits, block, sr=False, seed=0, off=0):
        return L.QParams(bits, block, int(sr), 0, seed, off)

    def timed(name, workload, alg_bytes, fn, args, kernel):
        if want is not None and not want(name):
            return
        for _ in range(3):
            st = fn(*args)
            if st != 0:
                raise L.LowbitError(st, fn.__name__)
        ts = []
        for _ in range(reps):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn(*args)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = sorted(ts)[len(ts) // 2]
        gbs = alg_bytes / (ms * 1e-3) / 1e9
        out[name] = {"workload": workload, "us": round(ms * 1e3, 2), "alg_bytes": int(alg_bytes),
                     "alg_GBps": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 3),
                     "kernel": kernel, "traffic": read_traffic(kernel, name)}

    # EF21 compress of the bucket (b4 B256 SR), state carried in place
    state = torch.zeros(N, dtype=torch.float32, device=dev)
    nw, nb = L.num_words(N, 4), L.num_blocks(N, BLOCK)
    c = torch.empty(nw, dtype=torch.int32, device=dev)
    s = torch.empty(nb, dtype=torch.float16, device=dev)
    q = qp(4, BLOCK, True, SEED)
    timed("ef21_compress b4", f"{N} fp32 bucket, b4 B{BLOCK} SR", 3 * N * 4 + nw * 4 + nb * 2,
          lib.lowbit_ef21_compress,
          (P(x.data_ptr()), L.F32, P(state.data_ptr()), N, ctypes.byref(q), P(c.data_ptr()),
           P(s.data_ptr()), sh), kname_quant(4, 8, True, 0, 3))
    del state

    # Hadamard-smoothed compress / decompress of the bucket (b4 B128 SR)
    HB = 128
    nw, nb = L.num_words(N, 4), L.num_blocks(N, HB)
    c = torch.empty(nw, dtype=torch.int32, device=dev)
    s = torch.empty(nb, dtype=torch.float16, device=dev)
    yh = torch.empty(N, dtype=torch.float32, device=dev)
    qh = qp(4, HB, True, SEED)
    hb = N * 4 + nw * 4 + nb * 2
    timed("hadamard_quantize_pack b4", f"{N} fp32 bucket, b4 B{HB} SR", hb,
          lib.lowbit_hadamard_quantize_pack,
          (P(x.data_ptr()), L.F32, N, ctypes.byref(qh), P(c.data_ptr()), P(s.data_ptr()), sh),
          kname_quant(4, 7, True, 0, 4, stream=True))
    timed("hadamard_unpack_dequant b4", f"{N} elements, b4 B{HB}", hb,
          lib.lowbit_hadamard_unpack_dequant,
          (P(c.data_ptr()), P(s.data_ptr()), N, ctypes.byref(qh), P(yh.data_ptr()), sh),
          kname_hadamard_dequant(4, 7))
    del yh, c, s

    # 8 peer chunks of 32 Mi (the local-reduce configuration): stage-2 EF at
    # b4 B128, and the two-level 8-bit B512 -> 4-bit B128 requantization
    NP = synth.PEER_N
    pc8, ps8, pc4, ps4 = [], [], [], []
    for p in range(PEERS):
        xp = torch.from_numpy(synth.peer_input(p)).to(dev)
        a8, b8 = L.quantize_pack(xp, 8, 512)
        a4, b4 = L.quantize_pack(xp, 4, 128)
        pc8.append(a8), ps8.append(b8), pc4.append(a4), ps4.append(b4)
        del xp
    oc = torch.empty(L.num_words(NP, 4), dtype=torch.int32, device=dev)
    os_ = torch.empty(L.num_blocks(NP, 128), dtype=torch.float16, device=dev)
    out_bytes = oc.numel() * 4 + os_.numel() * 2
    resid = torch.zeros(NP, dtype=torch.float32, device=dev)
    cp = (P * PEERS)(*[t.data_ptr() for t in pc4])
    sp = (P * PEERS)(*[t.data_ptr() for t in ps4])
    qi, qo = qp(4, 128), qp(4, 128)
    timed("reduce_requant_ef b4", f"{PEERS} x {NP} peers, b4 B128 -> b4 B128 + fp32 residual",
          (PEERS + 1) * out_bytes + 2 * NP * 4, lib.lowbit_reduce_requant_ef,
          (ctypes.cast(cp, P), ctypes.cast(sp, P), PEERS, NP, ctypes.byref(qi), ctypes.byref(qo),
           P(resid.data_ptr()), P(oc.data_ptr()), P(os_.data_ptr()), None, sh),
          kname_reduce(4, 4, 7, False, True))
    cp8 = (P * PEERS)(*[t.data_ptr() for t in pc8])
    sp8 = (P * PEERS)(*[t.data_ptr() for t in ps8])
    qi8 = qp(8, 512)
    in8 = L.num_words(NP, 8) * 4 + L.num_blocks(NP, 512) * 2
    timed("reduce_requant b8->b4", f"{PEERS} x {NP} peers, b8 B512 -> b4 B128",
          PEERS * in8 + out_bytes, lib.lowbit_reduce_requant,
          (ctypes.cast(cp8, P), ctypes.cast(sp8, P), PEERS, NP, ctypes.byref(qi8),
           ctypes.byref(qo), P(oc.data_ptr()), P(os_.data_ptr()), None, sh),
          kname_reduce(8, 4, 7, False))
    torch.cuda.synchronize()
    return out


def measure_compress_pattern(L, dev, x, reps=20):
    """Each compress and decompress of the step alone on the bucket, and
    beside the compress the reference kernel with its memory volume and none
    of its arithmetic (reads the binary32 bucket, writes the same number of
    code words; the scales' 2/B bytes per element are not written): median of
    `reps`, every launch after a 1 GiB read that leaves the Infinity Cache
    clean."""
    import torch

    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    N = x.numel()

    def alone(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[len(ts) // 2]

    out = {}
    y = torch.empty(N, dtype=torch.float32, device=dev)
    for b in BITS:
        nw, nb = L.num_words(N, b), L.num_blocks(N, BLOCK)
        c = torch.empty(nw, dtype=torch.int32, device=dev)
        s = torch.empty(nb, dtype=torch.float16, device=dev)
        cms = alone(lambda: L.quantize_pack(x, b, BLOCK, b > 1, SEED, 0, c, s))
        dms = alone(lambda: L.unpack_dequant(c, s, N, b, BLOCK, out=y))
        rms = alone(lambda: L.fold_f32(x, b, c))
        alg, ref = N * 4 + nw * 4 + nb * 2, N * 4 + nw * 4
        cg, dg, rg = (alg / (cms * 1e-3) / 1e9, alg / (dms * 1e-3) / 1e9,
                      ref / (rms * 1e-3) / 1e9)
        out[f"b{b}"] = {"workload": f"{N} fp32 bucket, b{b} B{BLOCK}" + (" SR" if b > 1 else ""),
                        "alg_bytes": alg,
                        "kernel": kname_quant(b, 8, b > 1, 0, 0, stream=True),
                        "decompress_kernel": kname_dequant(b, 0, 0),
                        "reference_kernel": kname_fold(b), "reference_bytes": ref,
                        "compress_us": round(cms * 1e3, 2), "compress_GBps": round(cg, 1),
                        "frac": round(cg / HBM_PEAK_GBS, 3),
                        "decompress_us": round(dms * 1e3, 2), "decompress_GBps": round(dg, 1),
                        "decompress_frac": round(dg / HBM_PEAK_GBS, 3),
                        "reference_us": round(rms * 1e3, 2), "reference_GBps": round(rg, 1),
                        "of_reference": round(cg / rg, 3)}
        del c, s
    del y
    return out


KNAME_PROBE = "void lowbit::stream_probe_kernel<{op}, {nt}>(lowbit::ProbeArgs, long)"


def measure_block_sweep(L, dev, x, reps=7):
    """Block sizes 32 .. 4096 at every bitwidth on the 64 Mi bucket (only with
    --only block_sweep): compress (SR above 1 bit), decompress, EF compress,
    Hadamard compress and decompress, and the
    weight-difference compress of a 64 Mi bf16 shard, each alone after a
    1 GiB read that leaves the Infinity Cache clean, median of `reps` (the
    EF residual carries over from launch to launch); the fractions of
    8 TB/s of each kernel's algorithmic bytes."""
    import torch

    N = x.numel()
    gen = torch.Generator(device=dev).manual_seed(3)
    w_old = (torch.randn(N, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
    w_new = (w_old.float() + torch.randn(N, device=dev, generator=gen) * 1e-4).to(torch.bfloat16)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    y = torch.empty(N, dtype=torch.float32, device=dev)
    e = torch.zeros(N, dtype=torch.float32, device=dev)   # the residual carries over

    def median_ms(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[len(ts) // 2]

    def frac(nbytes, ms):
        return round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 3)

    out = {}
    for b in BITS:
        for B in (32, 64, 128, 256, 512, 1024, 2048, 4096):
            nw, nb = L.num_words(N, b), L.num_blocks(N, B)
            c = torch.empty(nw, dtype=torch.int32, device=dev)
            s = torch.empty(nb, dtype=torch.float16, device=dev)
            alg = N * 4 + nw * 4 + nb * 2
            sr = b > 1
            row = {
                "compress": frac(alg, median_ms(lambda: L.quantize_pack(x, b, B, sr, SEED, 0, c, s))),
                "decompress": frac(alg, median_ms(lambda: L.unpack_dequant(c, s, N, b, B, out=y))),
                "ef_compress": frac(alg + 8 * N, median_ms(
                    lambda: L.ef_compress(x, e, b, B, sr, SEED, 0, c, s))),
                "hadamard_compress": frac(alg, median_ms(
                    lambda: L.hadamard_quantize_pack(x, b, B, sr, SEED, 0, codes=c, scales=s))),
                "hadamard_decompress": frac(alg, median_ms(
                    lambda: L.hadamard_unpack_dequant(c, s, N, b, B, out=y))),
                "wdiff_compress": frac(4 * N + nw * 4 + nb * 2, median_ms(
                    lambda: L.wdiff_compress(w_new, w_old, b, B, sr, SEED, 0, codes=c, scales=s))),
            }
            out[f"b{b} B{B}"] = row
            del c, s
    del w_old, w_new, flush, y, e
    return out


def measure_memory_patterns(L, dev, reps=7):
    """The memory-system comparisons behind the codec kernels' launch shape
    and store policy (lowbit_stream_probe_u32 and lowbit_fold_f32; not part of
    `value`), each the median of `reps` launches timed alone, every launch
    after a 1 GiB read that leaves the Infinity Cache clean:
    * grid: 4 GiB read, write and copy of 32-bit words, one trip per wave
      over the whole buffer against persistent grids of 2048 and 8192 waves
      looping over it (streaming stores);
    * drain: a 256 MiB read alone, right after a 256 MiB streaming write,
      and right after a 256 MiB plain write (the write untimed, between the
      flush and the read);
    * write_stream: the same 256 MiB read alone against a pass that reads it
      and writes 32 MiB (the 4-bit compress-volume fold of those bytes as
      64 Mi binary32 values)."""
    import torch

    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)

    def median_ms(fn, pre=None):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            flush.sum()
            if pre is not None:
                pre()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[len(ts) // 2]

    def gbps(nbytes, ms):
        return round(nbytes / (ms * 1e-3) / 1e9, 1)

    NW = 1 << 30                                   # 4 GiB of words
    a = torch.empty(NW, dtype=torch.int32, device=dev)
    b = torch.empty(NW, dtype=torch.int32, device=dev)
    L.stream_probe(L.PROBE_WRITE, a, value=0x9E3779B9)
    rd = torch.empty(NW // 1024, dtype=torch.int32, device=dev)
    grid = {}
    for waves in (0, 2048, 8192):
        r = median_ms(lambda: L.stream_probe(L.PROBE_READ, rd, a, waves=waves))
        w = median_ms(lambda: L.stream_probe(L.PROBE_WRITE, b, waves=waves))
        c = median_ms(lambda: L.stream_probe(L.PROBE_COPY, b, a, waves=waves))
        key = "one_trip_per_wave" if waves == 0 else f"persistent_{waves}_waves"
        grid[key] = {"read_us": round(r * 1e3, 1), "read_GBps": gbps(4 * NW, r),
                     "write_us": round(w * 1e3, 1), "write_GBps": gbps(4 * NW, w),
                     "copy_us": round(c * 1e3, 1), "copy_GBps": gbps(8 * NW, c)}
    S = 1 << 26                                    # 256 MiB of words
    ra, wb = a[:S], b[:S]
    rd2 = rd[:S // 1024]
    read = lambda: L.stream_probe(L.PROBE_READ, rd2, ra)
    alone = median_ms(read)
    after_nt = median_ms(read, pre=lambda: L.stream_probe(L.PROBE_WRITE, wb, nontemporal=True))
    after_plain = median_ms(read, pre=lambda: L.stream_probe(L.PROBE_WRITE, wb, nontemporal=False))
    fold_out = torch.empty(L.num_words(S, 4), dtype=torch.int32, device=dev)
    fold = median_ms(lambda: L.fold_f32(ra.view(torch.float32), 4, fold_out))
    out = {
        "grid": grid,
        "drain": {"read_256MiB_alone_us": round(alone * 1e3, 1),
                  "after_streaming_write_us": round(after_nt * 1e3, 1),
                  "after_plain_write_us": round(after_plain * 1e3, 1)},
        "write_stream": {"read_256MiB_us": round(alone * 1e3, 1),
                         "read_256MiB_write_32MiB_us": round(fold * 1e3, 1)},
        "kernels": {"read": KNAME_PROBE.format(op=0, nt="true"),
                    "write_streaming": KNAME_PROBE.format(op=1, nt="true"),
                    "write_plain": KNAME_PROBE.format(op=1, nt="false"),
                    "copy": KNAME_PROBE.format(op=2, nt="true"),
                    "fold": kname_fold(4)},
    }
    del a, b, rd, fold_out, flush
    return out


def measure_configs(L, dev, reps=20, want=None):
    """The kernels of the other workload configurations at their full sizes,
    each timed alone (median of `reps`, every launch after a 1 GiB read that
    leaves the Infinity Cache clean).  Inputs are drawn on the GPU from seeded
    generators with the configurations' distributions.  Not part of `value`.
    `want(name)` false: that entry is skipped."""
    import torch

    gen = torch.Generator(device=dev).manual_seed(5)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    out = {}

    def timed(name, workload, alg_bytes, fn, input_bytes, kernel):
        if want is not None and not want(name):
            return
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = sorted(ts)[len(ts) // 2]
        gbs = alg_bytes / (ms * 1e-3) / 1e9
        out[name] = {"workload": workload, "us": round(ms * 1e3, 2), "alg_bytes": int(alg_bytes),
                     "alg_GBps": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 3),
                     "input_GBps": round(input_bytes / (ms * 1e-3) / 1e9, 1),
                     "kernel": kernel, "traffic": read_traffic(kernel, name)}

    # error feedback on 128 Mi bfloat16 gradients, b4 B128 SR
    n = 128 << 20
    g = (torch.randn(n, device=dev, generator=gen) * 1e-4).to(torch.bfloat16)
    e = torch.zeros(n, dtype=torch.float32, device=dev)
    c = torch.empty(L.num_words(n, 4), dtype=torch.int32, device=dev)
    s = torch.empty(L.num_blocks(n, 128), dtype=torch.float16, device=dev)
    timed("ef_compress 128Mi bf16", f"{n} bf16 N(0,1e-4), fp32 residual, b4 B128 SR",
          n * (2 + 4 + 4) + c.numel() * 4 + s.numel() * 2,
          lambda: L.ef_compress(g, e, 4, 128, True, 2, 0, c, s), n * 2,
          kname_quant(4, 7, True, 1, 1))
    del g, e, c, s

    # local reduce of 8 peer chunks of 32 Mi, b4 B128 in and out, with the
    # peers in two placements: separately allocated buffers, and the layout an
    # all-to-all exchange delivers (one receive buffer holding each peer's
    # message -- its codes, then its scales -- back to back)
    n = 32 << 20
    nw4, nb4 = L.num_words(n, 4), L.num_blocks(n, 128)
    msg = nw4 * 4 + nb4 * 2                          # bytes of one peer's message
    recv = torch.empty(8 * msg // 4, dtype=torch.int32, device=dev)
    layouts = {
        "": ([torch.empty(nw4, dtype=torch.int32, device=dev) for _ in range(8)],
             [torch.empty(nb4, dtype=torch.float16, device=dev) for _ in range(8)]),
        ", receive buffer": ([recv[p * msg // 4: p * msg // 4 + nw4] for p in range(8)],
                             [recv[(p * msg + nw4 * 4) // 4:(p * msg + nw4 * 4 + nb4 * 2) // 4]
                              .view(torch.float16) for p in range(8)])}
    for p in range(8):
        xp = torch.randn(n, device=dev, generator=gen)
        for pc, ps in layouts.values():
            L.quantize_pack(xp, 4, 128, codes=pc[p], scales=ps[p])
        del xp
    oc = torch.empty(nw4, dtype=torch.int32, device=dev)
    os_ = torch.empty(nb4, dtype=torch.float16, device=dev)
    tot = torch.empty(n, dtype=torch.float32, device=dev)
    for lay, (pc, ps) in layouts.items():
        where = "separate buffers" if not lay else "one receive buffer, messages of codes + scales"
        timed(f"reduce_requant 8x32Mi{lay}", f"8 x {n} peers ({where}), b4 B128 -> b4 B128 "
              "nearest", 9 * (nw4 * 4 + nb4 * 2),
              lambda: L.reduce_requant(pc, ps, n, 4, 128, out_codes=oc, out_scales=os_), 8 * n * 4,
              kname_reduce(4, 4, 7, False))
        timed(f"reduce_requant 8x32Mi +sum{lay}", f"8 x {n} peers ({where}), b4 B128 -> b4 B128 "
              "nearest, fp32 sum written", 9 * (nw4 * 4 + nb4 * 2) + n * 4,
              lambda: L.reduce_requant(pc, ps, n, 4, 128, want_sum=True, out_codes=oc,
                                       out_scales=os_, out_sum=tot), 8 * n * 4,
              kname_reduce(4, 4, 7, False, sum_out=True))
        # bandwidth reference for that access pattern: XOR of the 8 peers' code
        # streams read the way the reduce reads them, one output stream, no
        # arithmetic
        timed(f"xor_streams 8x16MiB reference{lay}", f"XOR of the 8 peers' code streams "
              f"({nw4} words each, {where}) with the reduce's access pattern; not a codec step",
              9 * nw4 * 4, lambda: L.xor_streams(pc, oc), 8 * n * 4, KNAME_XOR)
        ref = out.get(f"xor_streams 8x16MiB reference{lay}")
        for k in (f"reduce_requant 8x32Mi{lay}", f"reduce_requant 8x32Mi +sum{lay}"):
            if ref is not None and k in out:
                out[k]["of_pattern_reference"] = round(out[k]["alg_GBps"] / ref["alg_GBps"], 3)
    # the same bytes as one stream: a 128 MiB read and a 16 MiB write (the
    # compress-volume reference at 4 bits over 32 Mi binary32 values), against
    # which the eight equally long streams read at once are compared
    one = recv[:8 * nw4].view(torch.float32)
    timed("fold 128MiB one-stream reference", "one contiguous 128 MiB read, 16 MiB written "
          "(compress-volume reference kernel); not a codec step", 9 * nw4 * 4,
          lambda: L.fold_f32(one, 4, oc), 8 * n * 4, kname_fold(4))
    one_ref = out.get("fold 128MiB one-stream reference")
    for lay in layouts:
        k = f"xor_streams 8x16MiB reference{lay}"
        if one_ref is not None and k in out:
            out[k]["of_one_stream"] = round(out[k]["alg_GBps"] / one_ref["alg_GBps"], 3)
    del layouts, recv, oc, os_, tot, one

    # weight difference on an 840 Mi bfloat16 shard, b4 B64
    n = 840 << 20
    if want is not None and not (want("wdiff_compress 840Mi bf16") or
                                 want("wdiff_apply 840Mi bf16")):
        return out
    w_prev = (torch.randn(n, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
    w_new = (w_prev.float() + torch.randn(n, device=dev, generator=gen) * 1e-4).to(torch.bfloat16)
    c = torch.empty(L.num_words(n, 4), dtype=torch.int32, device=dev)
    s = torch.empty(L.num_blocks(n, 64), dtype=torch.float16, device=dev)
    w_out = torch.empty_like(w_prev)
    wb = n * 4 + c.numel() * 4 + s.numel() * 2
    timed("wdiff_compress 840Mi bf16", f"{n} bf16 weights, b4 B64", wb,
          lambda: L.wdiff_compress(w_new, w_prev, 4, 64, codes=c, scales=s), n * 4,
          kname_quant(4, 6, False, 1, 2))
    timed("wdiff_apply 840Mi bf16", f"{n} bf16 weights, b4 B64", wb,
          lambda: L.wdiff_apply(w_prev, c, s, 4, 64, out=w_out), n * 2,
          kname_dequant(4, 1, 1))
    del w_prev, w_new, c, s, w_out
    torch.cuda.synchronize()
    return out


def measure_roundtrip(L, dev, reps=20, ring=256):
    """The 2^20-element roundtrip (compress b4 B128 nearest, then decompress):
    one launch of each is launch-bound (4.7 MB of traffic), so it is also
    timed over a ring of `ring` distinct 4 MiB buffers (1 GiB), issued
    eagerly and replayed from a HIP graph.  The graph's output is checked
    against the eager output.  Not part of `value`."""
    import torch

    n, bits, block = 1 << 20, 4, 128
    gen = torch.Generator(device=dev).manual_seed(0)
    xs = [torch.randn(n, device=dev, generator=gen) for _ in range(ring)]
    nw, nb = L.num_words(n, bits), L.num_blocks(n, block)
    cs = [torch.empty(nw, dtype=torch.int32, device=dev) for _ in range(ring)]
    ss = [torch.empty(nb, dtype=torch.float16, device=dev) for _ in range(ring)]
    ys = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(ring)]
    per_pass = 2 * (n * 4 + nw * 4 + nb * 2)            # compress + decompress bytes
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)

    def one(k):
        L.quantize_pack(xs[k], bits, block, codes=cs[k], scales=ss[k])
        L.unpack_dequant(cs[k], ss[k], n, bits, block, out=ys[k])

    def timed(fn):
        ts = []
        for _ in range(reps):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[len(ts) // 2]

    for k in range(ring):
        one(k)
    torch.cuda.synchronize()
    single = timed(lambda: one(0))
    eager = timed(lambda: [one(k) for k in range(ring)])
    want = cs[ring - 1].clone(), ys[ring - 1].clone()
    cs[ring - 1].zero_()
    ys[ring - 1].zero_()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for k in range(ring):
                one(k)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    if not (torch.equal(cs[ring - 1], want[0]) and torch.equal(ys[ring - 1], want[1])):
        raise RuntimeError("graph replay of the roundtrip differs from the eager result")
    replay = timed(graph.replay)
    if not (torch.equal(cs[ring - 1], want[0]) and torch.equal(ys[ring - 1], want[1])):
        raise RuntimeError("a later graph replay of the roundtrip differs from the eager result")
    total = ring * per_pass
    return {"workload": f"{n} fp32 N(0,1), b4 B128 nearest: compress + decompress",
            "single_pass_us": round(single * 1e3, 2),
            "single_pass_GBps": round(per_pass / (single * 1e-3) / 1e9, 1),
            "ring": f"{ring} distinct 4 MiB buffers (1 GiB)",
            "ring_eager_GBps": round(total / (eager * 1e-3) / 1e9, 1),
            "ring_graph_GBps": round(total / (replay * 1e-3) / 1e9, 1),
            "ring_graph_frac": round(total / (replay * 1e-3) / 1e9 / HBM_PEAK_GBS, 3)}


def measure_size_sweep(L, dev, cpu: bool, reps=20, lo=10, hi=28, cpu_hi=23, burst=20):
    """Latency of one compress (b4 B128 nearest, fp32 N(0,1)) over sizes
    2^lo..2^hi, as in the 4-bit quantize latency curve (2^10..2^23 elements,
    CPU path against GPU path) of the bitscom README, 'Quantization CPU vs GPU
    Curve'.  Per size: `call_us`, the caller's wall time of one call through
    the binding plus a synchronize (median of `reps`); `kernel_us`, the GPU
    time per launch of `burst` launches replayed from a HIP graph (warm: the
    same buffers each time; below about 2^20 elements this is the dispatch
    floor, not the kernel); and, up to 2^cpu_hi, the CPU oracle's wall time
    (one thread, median of 3).  Not part of `value`."""
    import torch

    bits, block = 4, 128
    gen = torch.Generator(device=dev).manual_seed(0)
    side = torch.cuda.Stream(device=dev)
    rows = []
    for p in range(lo, hi + 1):
        n = 1 << p
        x = torch.randn(n, device=dev, generator=gen)
        codes = torch.empty(L.num_words(n, bits), dtype=torch.int32, device=dev)
        scales = torch.empty(L.num_blocks(n, block), dtype=torch.float16, device=dev)
        alg = n * 4 + codes.numel() * 4 + scales.numel() * 2
        for _ in range(3):
            L.quantize_pack(x, bits, block, codes=codes, scales=scales)
        torch.cuda.synchronize()
        wall = []
        for _ in range(reps):
            t0 = time.perf_counter()
            L.quantize_pack(x, bits, block, codes=codes, scales=scales)
            torch.cuda.synchronize()
            wall.append(time.perf_counter() - t0)
        graph = torch.cuda.CUDAGraph()
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                for _ in range(burst):
                    L.quantize_pack(x, bits, block, codes=codes, scales=scales)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        kern = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            kern.append(e0.elapsed_time(e1) * 1e-3 / burst)
        k, w = sorted(kern)[2], sorted(wall)[reps // 2]
        row = {"log2_n": p, "kernel_us": round(k * 1e6, 2), "call_us": round(w * 1e6, 2),
               "alg_GBps": round(alg / k / 1e9, 1)}
        if cpu and p <= cpu_hi:
            import oracle as O
            xh = x.cpu().numpy()
            ts = []
            for _ in range(3):
                t0 = time.perf_counter()
                O.quantize_pack(xh, bits, block)
                ts.append(time.perf_counter() - t0)
            row["cpu_oracle_us"] = round(sorted(ts)[1] * 1e6, 1)
            row["cpu_over_call"] = round(sorted(ts)[1] / w, 1)
        rows.append(row)
        del graph, x, codes, scales
    return {"workload": f"fp32 N(0,1), b4 B{block} nearest compress, 2^{lo}..2^{hi} elements",
            "rows": rows}


def _block_ranges(n, align, parts):
    """Split [0, n) into at most `parts` contiguous ranges whose starts are
    multiples of `align`."""
    step = -(-max(1, -(-n // parts)) // align) * align
    return [(lo, min(n, lo + step)) for lo in range(0, n, step)]


def cpu_baseline_all_cores(x, w_prev, w_new, n, nstages, threads):
    """The same oracle calls as `cpu_baseline`, split over `threads` host
    threads by block-aligned element ranges (blocks are independent and the
    SR hash is keyed on the global index, so the outputs are the same bytes);
    the C oracle runs without the interpreter lock."""
    import concurrent.futures as cf
    import numpy as np
    import oracle as O

    xs = np.ascontiguousarray(x[:n])
    wp, wn = np.ascontiguousarray(w_prev[:n]), np.ascontiguousarray(w_new[:n])
    share = n // PEERS
    align = 32 * BLOCK
    ex = cf.ThreadPoolExecutor(threads)

    def par(fn, total):
        return list(ex.map(lambda r: fn(*r), _block_ranges(total, align, threads)))

    t0 = time.perf_counter()
    for b in BITS:
        parts = par(lambda lo, hi: O.quantize_pack(xs[lo:hi], b, BLOCK, True, SEED, lo), n)
        c = np.concatenate([p[0] for p in parts])
        s = np.concatenate([p[1] for p in parts])
        snw, snb = O.num_words(share, b), O.num_blocks(share, BLOCK)

        def red(lo, hi, b=b, c=c, s=s, snw=snw, snb=snb):
            w0, w1 = lo * b // 32, O.num_words(hi, b)
            return O.reduce_requant([c[p * snw + w0:p * snw + w1] for p in range(PEERS)],
                                    [s[p * snb + lo // BLOCK:p * snb + O.num_blocks(hi, BLOCK)]
                                     for p in range(PEERS)], hi - lo, b, BLOCK, b)
        par(red, share)
        par(lambda lo, hi, b=b, c=c, s=s: O.unpack_dequant(
            c[lo * b // 32:O.num_words(hi, b)], s[lo // BLOCK:O.num_blocks(hi, BLOCK)],
            hi - lo, b, BLOCK), n)
    par(lambda lo, hi: O.ef_compress(xs[lo:hi], np.zeros(hi - lo, np.float32), EF_BITS, BLOCK,
                                     True, SEED, lo), n)

    def wd(lo, hi):
        c, s = O.wdiff_compress(wn[lo:hi], wp[lo:hi], W_BITS, W_BLOCK)
        O.wdiff_apply(wp[lo:hi], c, s, W_BITS, W_BLOCK)
    par(wd, n)
    dt = time.perf_counter() - t0
    ex.shutdown()
    return {"value": round(nstages * n * 4 / dt / 1e9, 3), "unit": "GB/s", "cores": threads,
            "seconds": round(dt, 2)}


def cpu_baseline_configs(x_bucket, threads, reps=3):
    """The CPU oracle on each workload configuration's own operation, on the
    host recipes the parity tests use (synth): one thread and `threads`
    threads (block-aligned element ranges; blocks are independent and the SR
    hash is keyed on the global index, so the outputs are the same bytes),
    median wall time of `reps` runs (5 for the small roundtrip), excluding
    input generation.  Sizes are the configurations' own, except the weight
    shard (840 Mi elements), which is timed on a 64 Mi sample drawn with the
    same recipe.  GB/s as in the GPU rows: input = full-precision bytes of the
    operation's input as stored, alg = algorithmic bytes."""
    import concurrent.futures as cf
    import numpy as np
    import oracle as O
    from weight_communication_compression_amd import synth

    ex = cf.ThreadPoolExecutor(threads)

    def median_s(fn, k):
        ts = []
        for _ in range(k):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return sorted(ts)[len(ts) // 2]

    def par(fn, total, align):
        return list(ex.map(lambda r: fn(*r), _block_ranges(total, align, threads)))

    def entry(workload, n, input_bytes, alg_bytes, one, many, k=reps):
        t1, tm = median_s(one, k), median_s(many, k)
        row = lambda t: {"s": round(t, 4), "input_GBps": round(input_bytes / t / 1e9, 3),
                         "alg_GBps": round(alg_bytes / t / 1e9, 3)}
        return {"workload": workload, "elements": n, "reps": k, "stat": "median",
                "one_thread": row(t1), "all_threads": dict(threads=threads, **row(tm))}

    nwb = lambda n, b: O.num_words(n, b) * 4
    nbb = lambda n, B: O.num_blocks(n, B) * 2
    out = {}

    # roundtrip: 2^20 fp32 N(0,1), b4 B128 nearest, compress then decompress
    x = synth.roundtrip_input()
    n = x.size

    def rt(lo, hi):
        c, s = O.quantize_pack(x[lo:hi], 4, 128, False, 0, lo)
        O.unpack_dequant(c, s, hi - lo, 4, 128)
    out["roundtrip 2^20 fp32 b4 B128"] = entry(
        f"{n} fp32 N(0,1), b4 B128 nearest: compress + decompress", n, n * 4,
        2 * (n * 4 + nwb(n, 4) + nbb(n, 128)), lambda: rt(0, n),
        lambda: par(rt, n, 32 * 128), k=5)

    # gradient bucket: 64 Mi fp32 Student-t(3) x 1e-3, B256, SR seed 42, each width
    x = x_bucket
    n = x.size
    for b in BITS:
        out[f"bucket 64Mi fp32 b{b}"] = entry(
            f"{n} fp32 1e-3 Student-t(3), b{b} B256" + (" SR seed 42" if b > 1 else ""), n,
            n * 4, n * 4 + nwb(n, b) + nbb(n, 256),
            lambda b=b: O.quantize_pack(x, b, 256, True, 42, 0),
            lambda b=b: par(lambda lo, hi: O.quantize_pack(x[lo:hi], b, 256, True, 42, lo), n,
                            32 * 256))

    # error feedback, step 0: 128 Mi bf16 1e-4 N(0,1), fp32 residual 0, b4 B128 SR seed 2
    g = synth.ef_gradient(0)
    n = g.size
    e0 = np.zeros(n, np.float32)
    out["ef_compress 128Mi bf16 b4"] = entry(
        f"{n} bf16 1e-4 N(0,1) + fp32 residual, b4 B128 SR seed 2 (step 0)", n, n * 2,
        n * (2 + 4 + 4) + nwb(n, 4) + nbb(n, 128),
        lambda: O.ef_compress(g, e0, 4, 128, True, 2, 0),
        lambda: par(lambda lo, hi: O.ef_compress(g[lo:hi], e0[lo:hi], 4, 128, True, 2, lo), n,
                    32 * 128))
    del g, e0

    # local reduce: 8 peers x 32 Mi, each N(0,1) (seeds 10..17) compressed b4 B128 nearest
    n = synth.PEER_N
    peers = list(ex.map(lambda p: O.quantize_pack(synth.peer_input(p), 4, 128),
                        range(synth.PEERS)))
    pc, ps = [c for c, _ in peers], [s for _, s in peers]

    def red(lo, hi):
        w0, w1 = lo * 4 // 32, O.num_words(hi, 4)
        O.reduce_requant([c[w0:w1] for c in pc],
                         [s[lo // 128:O.num_blocks(hi, 128)] for s in ps], hi - lo, 4, 128, 4)
    out["reduce_requant 8x32Mi b4"] = entry(
        f"8 x {n} peers, b4 B128 -> b4 B128 nearest", n, synth.PEERS * n * 4,
        (synth.PEERS + 1) * (nwb(n, 4) + nbb(n, 128)), lambda: red(0, n),
        lambda: par(red, n, 32 * 128))
    del peers, pc, ps

    # weight difference: 64 Mi sample of the bf16 shard recipe, b4 B64 compress + apply
    n = 64 << 20
    wp, wn = synth.weight_pair(n)

    def wd(lo, hi):
        c, s = O.wdiff_compress(wn[lo:hi], wp[lo:hi], 4, 64)
        O.wdiff_apply(wp[lo:hi], c, s, 4, 64)
    out["wdiff 840Mi bf16 b4 (64Mi sample)"] = entry(
        f"{n}-element sample of the 840 Mi bf16 shard recipe, b4 B64 nearest: "
        "compress + apply", n, 2 * n * 2 + n * 2,
        2 * (2 * n * 2 + nwb(n, 4) + nbb(n, 64)), lambda: wd(0, n),
        lambda: par(wd, n, 32 * 64))
    ex.shutdown()
    return out


def cpu_baseline(x, w_prev, w_new, n, nstages):
    """Time the CPU oracle over the first n elements of the same workload
    (all 15 stage passes), single-threaded; report in the same unit.  Also
    returns the oracle's outputs (held, not copied, inside the timed region)."""
    import numpy as np
    import oracle as O

    xs = np.ascontiguousarray(x[:n])
    wp, wn = np.ascontiguousarray(w_prev[:n]), np.ascontiguousarray(w_new[:n])
    share = n // PEERS
    outs = {}
    t0 = time.perf_counter()
    for b in BITS:
        c, s = O.quantize_pack(xs, b, BLOCK, True, SEED, 0)
        snw, snb = O.num_words(share, b), O.num_blocks(share, BLOCK)
        rc, rs, _ = O.reduce_requant([c[p * snw:(p + 1) * snw] for p in range(PEERS)],
                                     [s[p * snb:(p + 1) * snb] for p in range(PEERS)], share, b,
                                     BLOCK, b)
        y = O.unpack_dequant(c, s, n, b, BLOCK)
        outs[f"b{b}"] = (c, s, rc, rs, y)
    outs["ef"] = O.ef_compress(xs, np.zeros(n, np.float32), EF_BITS, BLOCK, True, SEED, 0)
    c, s = O.wdiff_compress(wn, wp, W_BITS, W_BLOCK)
    outs["wd"] = (c, s, O.wdiff_apply(wp, c, s, W_BITS, W_BLOCK))
    dt = time.perf_counter() - t0
    return {"value": round(nstages * n * 4 / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"first {n} elements of the bucket (and of the weight shard), all "
                      f"{nstages} stage passes, scalar C oracle, one thread",
            "host": host_cpu()}, outs


def host_cpu():
    """The host's CPU model and the threads this process may use."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"model": model, "threads_available": len(os.sched_getaffinity(0)),
            "nproc": os.cpu_count()}


def check_against_oracle(gpu, cpu, n, N):
    """Bit comparison of the step's GPU outputs with the oracle's on the
    first n elements (whole blocks); the local reduce only when the oracle ran
    the full bucket, whose 8 slices are the peers."""
    import numpy as np
    import torch

    def bits(t, m):
        a = t.cpu().numpy()
        return a.view({4: np.uint32, 2: np.uint16}[a.dtype.itemsize])[:m]

    def raw(a):
        return a.view({4: np.uint32, 2: np.uint16}[a.dtype.itemsize])

    checked, bad = [], []

    def cmp(name, g, c):
        c = raw(np.asarray(c))
        (checked if np.array_equal(bits(g, c.size), c) else bad).append(name)

    for b in BITS:
        gc, gs, grc, grs, gy = gpu[f"b{b}"]
        cc, cs, crc, crs, cy = cpu[f"b{b}"]
        cmp(f"quantize_pack b{b} codes", gc, cc)
        cmp(f"quantize_pack b{b} scales", gs, cs)
        if n == N:
            cmp(f"reduce_requant b{b} codes", grc, crc)
            cmp(f"reduce_requant b{b} scales", grs, crs)
        cmp(f"unpack_dequant b{b}", gy, cy)
    for i, what in enumerate(("codes", "scales", "residual")):
        cmp(f"ef_compress b{EF_BITS} {what}", gpu["ef"][i], cpu["ef"][i])
    for i, what in enumerate(("codes", "scales")):
        cmp(f"wdiff_compress b{W_BITS} {what}", gpu["wd"][i], cpu["wd"][i])
    cmp(f"wdiff_apply b{W_BITS}", gpu["wd"][2].view(torch.int16), cpu["wd"][2])
    return {"elements": n, "outputs_bit_identical": len(bad) == 0, "checked": len(checked) +
            len(bad), "mismatched": bad}


if __name__ == "__main__":
    sys.exit(main())
