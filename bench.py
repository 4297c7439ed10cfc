#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One step = one pass of the whole path over resident synthetic inputs:
  * chunked prefill of 1 x 8192 tokens, 96 heads, d_k = d_v = 128, C = 64,
    bf16 q/k/v, fp32 g/beta, zero initial state -> outputs + final state
    (chunk-prep kernel, then chunk-recurrence kernel), and
  * one decode step of 64 sequences x 96 heads, d = 128, fp32 state
    ~N(0, 0.02^2) updated in place, bf16 q/k/v (decode kernel).

Prints ONE JSON line.  `value` is the decode step's state throughput in GB/s
(8 * d^2 bytes per head and token, the fp32 state read and written once:
"Kimi K3: The Manos, The Mythos, The Legendos", section "Complexity
analysis"); the prefill's tokens/s, FLOP and byte rates ride in the same
line.  The prefill runs as its two stages (kda_prefill_varlen_prep, then
kda_prefill_varlen_recur), so that each of the step's three kernels is timed
on its own; `kernels` gives each one's algorithmic HBM rate against the
peak, and `roofline` repeats the one that takes the largest share of the
step.  Kernel durations come from HIP events on the stream the kernels run
on, created without the system-scope fence (see HipEvent).  Decode rotates
three state buffers so that consecutive steps never find the state in the
256 MB Infinity Cache.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from linear_recurrent_attention_kda_amd import counts, inputs  # noqa: E402

METRIC = ("KDA prefill tokens/s + decode state GB/s (H=96,D=128) on 1 MI355X, "
          "% roofline")
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "linear_recurrent_attention_kda_amd", "csrc")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class HipEvent:
    """A timing event created with hipEventDisableSystemFence.  A default
    HIP event performs a system-scope fence when it is recorded (HIP's
    documentation of the flag: a write-back and invalidation of the caches,
    which can slow the work after it).  The library launches its kernels
    back to back with no event between them, so the timing events leave the
    caches alone; elapsed times are read only after a device
    synchronisation.  Measured in kernel traces of this benchmark: the gap
    that an event leaves between two kernels is 4.5-9 us instead of 6-11 us,
    and the kernels' own durations are the same.  Same interface as
    torch.cuda.Event."""
    _lib = None
    DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence

    @classmethod
    def lib(cls):
        if cls._lib is None:
            import ctypes
            # the HIP runtime torch has loaded (it carries this soname)
            lib = ctypes.CDLL("libamdhip64.so.7")
            vp = ctypes.c_void_p
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp),
                                                    ctypes.c_uint]
            lib.hipEventRecord.argtypes = [vp, vp]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                vp, vp]
            lib.hipEventDestroy.argtypes = [vp]
            cls._lib = lib
        return cls._lib

    def __init__(self):
        import ctypes
        self.h = ctypes.c_void_p()
        rc = self.lib().hipEventCreateWithFlags(ctypes.byref(self.h),
                                                self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed: %d" % rc)

    def record(self, stream):
        import ctypes
        rc = self.lib().hipEventRecord(self.h,
                                       ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def elapsed_time(self, end):
        import ctypes
        ms = ctypes.c_float()
        rc = self.lib().hipEventElapsedTime(ctypes.byref(ms), self.h, end.h)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return float(ms.value)

    def __del__(self):
        if self.h and self._lib is not None:
            self._lib.hipEventDestroy(self.h)


def source_hash(name: str) -> str:
    h = hashlib.sha256()
    for f in (name, "kda_device.hpp", "kda_internal.hpp"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_counters(kind: str, kernel_file: str):
    """Per-launch rocprofv3 counter figures stored in
    profiles/<kind>_<name>.txt (key = value lines), as floats, or None when
    no measurement exists or the kernel's source changed since it was
    taken."""
    path = os.path.join(PROFILES, "%s_%s.txt" %
                        (kind, kernel_file.replace(".hip", "")))
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    if kv.pop("source_sha256_16", None) != source_hash(kernel_file):
        return None
    try:
        return {key: float(val) for key, val in kv.items()}
    except ValueError:
        return None


def read_traffic(kernel_file: str):
    """HBM bytes per launch measured with FETCH_SIZE / WRITE_SIZE for the
    current source of `kernel_file`, or None."""
    kv = read_counters("traffic", kernel_file)
    return None if kv is None else kv.get("hbm_bytes_per_launch")


def mfma_figures(kernel_file: str, avg_ms: float):
    """Matrix-core work of one launch from the stored MFMA counters
    (SQ_INSTS_VALU_MFMA_MOPS_* count 512 FLOPs each; SQ_VALU_MFMA_BUSY_CYCLES
    sums over SIMDs), over the live average launch time: achieved TFLOP/s
    against the bf16 peak, and the share of SIMD cycles the matrix cores
    were busy.  None without a measurement for the current source."""
    kv = read_counters("mfma", kernel_file)
    if kv is None:
        return None
    bf16 = kv["bf16_mops"] * 512
    f32 = kv["f32_mops"] * 512
    s = avg_ms * 1e-3
    return {"bf16_flop_per_launch": int(bf16),
            "f32_flop_per_launch": int(f32),
            "achieved_tflops": round((bf16 + f32) / s / 1e12, 2),
            "peak_tflops": counts.BF16_MFMA_PEAK_TFLOPS,
            "frac": round(bf16 / s / 1e12 / counts.BF16_MFMA_PEAK_TFLOPS +
                          f32 / s / 1e12 / counts.FP32_MFMA_PEAK_TFLOPS, 4),
            "busy_frac": round(kv["busy_cycles"] /
                               (s * counts.CLOCK_HZ * counts.SIMDS), 4)}


def kernel_entry(name, src_file, nbytes, ms, traffic=True):
    """Roofline entry of one kernel: its algorithmic bytes per launch over
    its average launch time (HIP events), against the HBM peak.  The stored
    counter figures (traffic, MFMA) were taken on the 8K-token prefill and
    decode workloads, so other workloads pass traffic=False."""
    avg, med = float(np.mean(ms)), float(np.median(ms))
    ach = nbytes / (avg * 1e-3) / 1e9
    return {"kernel": name, "bound": "hbm", "achieved": round(ach, 2),
            "peak": counts.HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(ach / counts.HBM_PEAK_GBPS, 4),
            "traffic": read_traffic(src_file) if traffic else None,
            "algorithmic_bytes_per_launch": nbytes,
            "avg_launch_ms": round(avg, 5),
            "median_launch_ms": round(med, 5),
            "mfma": mfma_figures(src_file, avg) if traffic else None}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--prefill", default="prefill",
                    choices=["prefill", "long", "varlen"],
                    help="prefill workload timed in each step")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the oracle on the host cores")
    ap.add_argument("--ckpt-every", type=int, default=0,
                    help="run the prefill through kda_prefill_varlen_ckpt, "
                         "storing the state every N tokens (a multiple of "
                         "the chunk size)")
    ap.add_argument("--spec-tokens", type=int, default=4,
                    help="time speculative verify, commit and the fused step "
                         "with this many draft tokens per sequence on the "
                         "decode batch (outside the timed steps; 0 skips)")
    ap.add_argument("--no-epilogue", action="store_true",
                    help="skip timing the output epilogue (standalone over "
                         "the prefill output, fused into the prefill's "
                         "recurrence, fused into the decode step), taken "
                         "after the timed steps")
    ap.add_argument("--no-prologue", dest="prologue", action="store_false",
                    help="skip timing the prefill with the input prologue "
                         "fused (outside the timed steps)")
    ap.add_argument("--step-only", action="store_true",
                    help="skip the measurements taken after the timed steps "
                         "(back-to-back decode, reference copy), so that a "
                         "kernel trace sees only the steps")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the legs of the other workloads (the tiny "
                         "prefill's latency, the long-context and the varlen "
                         "prefill), taken after the timed steps")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB per "
                         "step (reference kernel for HBM counter scaling)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: KDA shards over "
              "(sequence, head) with no communication, so a multi-GPU run "
              "is one independent copy of this step per GPU. "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    from linear_recurrent_attention_kda_amd import kda

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kda.load()  # fails loudly if libkda.so is missing

    # ---------------- inputs (seeded, resident in HBM before timing) -------
    t_gen = time.time()
    dp = inputs.make("decode", seed=0)
    pp = inputs.make(args.prefill, seed=0)
    log("inputs generated in %.1fs" % (time.time() - t_gen))

    def to_dev(x, dt):
        t = torch.from_numpy(np.ascontiguousarray(x))
        return (t.to(torch.bfloat16) if dt == "bf16" else t).to(dev)

    dq, dk, dv = (to_dev(x, dp.dtype) for x in (dp.q, dp.k, dp.v))
    dg, dbeta = to_dev(dp.g, "fp32"), to_dev(dp.beta, "fp32")
    states = [to_dev(dp.initial_state, "fp32") for _ in range(3)]
    do = torch.empty((dp.B, dp.H, dp.V), dtype=dq.dtype, device=dev)

    pq, pk, pv = (to_dev(x, pp.dtype) for x in (pp.q, pp.k, pp.v))
    pg, pbeta = to_dev(pp.g, "fp32"), to_dev(pp.beta, "fp32")
    ps0 = None if pp.initial_state is None else to_dev(pp.initial_state,
                                                       "fp32")
    if pp.kind == "varlen":
        cu = torch.from_numpy(pp.cu_seqlens).to(dev)
        nseq, total = len(pp.cu_seqlens) - 1, int(pp.cu_seqlens[-1])
        maxlen = int(pp.seq_lengths.max())
        po = torch.empty((total, pp.H, pp.V), dtype=pq.dtype, device=dev)
    else:
        nseq, total = pp.B, pp.B * pp.T
        po = torch.empty((pp.B, pp.T, pp.H, pp.V), dtype=pq.dtype, device=dev)
    pfs = torch.empty((nseq, pp.H, pp.K, pp.V), dtype=torch.float32,
                      device=dev)
    # the prefill runs as its two stages (chunk prep, then the recurrence)
    # on packed sequences, so that each kernel is timed on its own; for one
    # or more sequences of equal length this is exactly kda_prefill_chunked
    if pp.kind != "varlen":
        cu = torch.arange(nseq + 1, dtype=torch.int32, device=dev) * pp.T
        maxlen = pp.T
    pq_, pk_, pv_ = (x.reshape(total, pp.H, -1) for x in (pq, pk, pv))
    pg_, pbeta_ = pg.reshape(total, pp.H, -1), pbeta.reshape(total, pp.H)
    po_ = po.reshape(total, pp.H, pp.V)
    ck = None
    if args.ckpt_every:
        ck = torch.zeros((total // args.ckpt_every, pp.H, pp.K, pp.V),
                         dtype=torch.float32, device=dev)
    ws = kda.workspace_for(nseq, total, pp.H, pp.K, pp.V, pp.C, dev)
    calib = None
    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        calib = (torch.ones(n, dtype=torch.float32, device=dev),
                 torch.empty(n, dtype=torch.float32, device=dev))
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)

    def prefill(mid=None):
        """The prefill; `mid` (an event) is recorded between its two
        kernels.  With state checkpoints it is one library call."""
        if ck is not None:
            kda.kda_prefill_varlen_ckpt(pq_, pk_, pv_, pg_, pbeta_, cu, maxlen,
                                        ps0, ckpt_every=args.ckpt_every,
                                        chunk_size=pp.C, final_state=pfs,
                                        o=po_, ckpt_states=ck, workspace=ws)
            return
        kda.kda_prefill_varlen_prep(pq_, pk_, pv_, pg_, pbeta_, cu, maxlen,
                                    chunk_size=pp.C, workspace=ws)
        if mid is not None:
            mid.record(stream)
        kda.kda_prefill_varlen_recur(ws, cu, maxlen, total, pp.H, pp.K, pp.V,
                                     pq.dtype, ps0, chunk_size=pp.C,
                                     final_state=pfs, o=po_)

    def decode(i):
        kda.kda_decode_step(dq, dk, dv, dg, dbeta, states[i % 3], o=do)

    ev = HipEvent

    def step(i, rec=None):
        if rec is not None:
            e0, em, e1, e2 = ev(), ev(), ev(), ev()
            e0.record(stream)
        prefill(None if rec is None or ck is not None else em)
        if rec is not None:
            e1.record(stream)
        decode(i)
        if rec is not None:
            e2.record(stream)
            rec.append((e0, None if ck is not None else em, e1, e2))
        if calib is not None:
            calib[1].copy_(calib[0])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log("warmup done (%d steps)" % args.warmup)

    rec = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, rec)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = [a.elapsed_time(b) for a, _, b, _ in rec]
    dec_ms = [b.elapsed_time(c) for _, _, b, c in rec]
    prep_ms = recur_ms = None
    if ck is None:
        prep_ms = [a.elapsed_time(m) for a, m, _, _ in rec]
        recur_ms = [m.elapsed_time(b) for _, m, b, _ in rec]
    ms_step = wall * 1e3 / args.steps

    def busy():  # whole steps (prefill and decode), then wait
        for i in range(3):
            step(i)
        torch.cuda.synchronize()
    # clocks under load, after the timed steps.  Not in profiling runs
    # (--step-only, or any run under rocprofv3): a kernel trace then holds
    # the timed steps only, and no tool is started from a profiled process.
    if args.step_only or any(k.startswith("ROCPROF_") for k in os.environ):
        clocks = {"skipped": "profiling run"}
    else:
        clocks = gpu_clocks(busy)

    # the results of the step's prefill (po, pfs: the same every step) and
    # of one decode step from the initial state, for the oracle leg's
    # parity figures
    gpu_res = None
    if not args.no_cpu_baseline:
        st1 = torch.from_numpy(np.ascontiguousarray(dp.initial_state)).to(dev)
        o1 = kda.kda_decode_step(dq, dk, dv, dg, dbeta, st1)
        torch.cuda.synchronize()
        gpu_res = {"prefill": (po.float().cpu().numpy(), pfs.cpu().numpy()),
                   "decode": (o1.float().cpu().numpy(), st1.cpu().numpy())}
        del st1, o1
    pre_avg = float(np.mean(pre_ms))
    dec_avg = float(np.mean(dec_ms))
    pre_med = float(np.median(pre_ms))
    dec_med = float(np.median(dec_ms))
    log("timed %d steps: %.3f ms/step, prefill %.3f ms, decode %.4f ms"
        % (args.steps, ms_step, pre_avg, dec_avg))
    if prep_ms is not None:
        log("prefill stages: prep %.4f ms, recurrence %.4f ms"
            % (float(np.mean(prep_ms)), float(np.mean(recur_ms))))

    # decode steps back to back (outside the timed region): the state traffic
    # of one step then overlaps the write-back of the previous one, the
    # sustained case of a decode-only server loop
    n_b2b, b2b_ms, copy_ref, pool_ms = 0, None, None, None
    if not args.step_only:
        n_b2b = max(5 * args.steps, 100)  # >= 100 decode iterations
        for i in range(6):
            decode(i)
        b0, b1 = ev(), ev()
        b0.record(stream)
        for i in range(n_b2b):
            decode(i)
        b1.record(stream)
        torch.cuda.synchronize()
        b2b_ms = b0.elapsed_time(b1) / n_b2b
        log("decode back to back: %.4f ms" % b2b_ms)
        # the same from a state pool (kda_decode_step_indexed): the batch's
        # states in 64 scattered rows of a 192-row pool, another third of
        # the pool each launch
        pool = torch.cat(states, 0)
        del states[:]
        perm = torch.randperm(dp.B, generator=torch.Generator().manual_seed(9))
        idxs = [(3 * perm + j).to(torch.int32).to(dev) for j in range(3)]
        states.extend(pool.view(3, dp.B, *pool.shape[1:]).unbind(0))

        def decode_pool(i):
            kda.kda_decode_step_indexed(dq, dk, dv, dg, dbeta, pool,
                                        idxs[i % 3], o=do)
        for i in range(6):
            decode_pool(i)
        b0.record(stream)
        for i in range(n_b2b):
            decode_pool(i)
        b1.record(stream)
        torch.cuda.synchronize()
        pool_ms = b0.elapsed_time(b1) / n_b2b
        log("decode from a state pool, back to back: %.4f ms" % pool_ms)
        # reference: the runtime's device-to-device copy of 1 GiB
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        c0, c1 = ev(), ev()
        c0.record(stream)
        for _ in range(10):
            dst.copy_(src)
        c1.record(stream)
        torch.cuda.synchronize()
        copy_ms = c0.elapsed_time(c1) / 10
        copy_ref = {"bytes_per_copy": 2 << 30, "avg_ms": round(copy_ms, 4),
                    "achieved": round((2 << 30) / (copy_ms * 1e-3) / 1e9, 2)}
        del src, dst
        log("reference copy: %.4f ms" % copy_ms)

    spec = None
    if args.spec_tokens and not args.step_only:
        spec = time_spec(args.spec_tokens, dp, states, dev, stream, ev)
    pro = None
    if args.prologue and not args.step_only:
        pro = time_prologue(pp, nseq, total, ws, dev, stream, ev)
    epi = None
    if not args.no_epilogue and not args.step_only:
        epi = time_epilogue(po, dq, dk, dv, dg, dbeta, states, dev, stream, ev)
        epi["prefill_gated"] = time_gated_prefill(
            (pq_, pk_, pv_, pg_, pbeta_), cu, maxlen, total, pp.H, pp.K,
            pp.V, pp.C, ps0, ws, dev, stream, ev)
    legs, samples = None, {}
    if not args.step_only and not args.no_workloads:
        legs = {"tiny": time_tiny(dev, stream, ev)}
        for name in ("long", "varlen"):
            legs[name], samples[name] = time_prefill_workload(
                name, dev, stream, ev)

    # ---------------- derived figures --------------------------------------
    D, H = dp.K, dp.H
    dec_bytes = counts.decode_bytes_per_head(D) * dp.B * H
    dec_gbps = dec_bytes / (dec_avg * 1e-3) / 1e9
    chunks = int(np.sum((pp.seq_lengths + pp.C - 1) // pp.C)) * pp.H
    pre_flops = counts.prefill_flops_per_chunk(pp.C, D) * chunks
    pre_bytes_pages = (counts.prefill_bytes_per_chunk(pp.C, D) * chunks +
                       counts.decode_bytes_per_head(D) * nseq * pp.H)
    pre_bytes_min = (counts.prefill_min_bytes_per_token_head(pp.K, pp.V) *
                     total * pp.H)
    pre_s = pre_avg * 1e-3
    elt = pq.element_size()
    prep_b = counts.prep_bytes(total * pp.H, chunks, pp.C, pp.K, pp.V, elt)
    recur_b = counts.recur_bytes(total * pp.H, chunks, pp.C, pp.K, pp.V, elt)

    kernels = []
    if prep_ms is not None:
        kernels.append(kernel_entry("prep_kernel (kda_prep.hip)",
                                    "kda_prep.hip", prep_b, prep_ms))
        kernels.append(kernel_entry("chunk recurrence (kda_recur.hip)",
                                    "kda_recur.hip", recur_b, recur_ms))
    dec_entry = kernel_entry("decode_kernel (kda_decode.hip)",
                             "kda_decode.hip", dec_bytes, dec_ms)
    dec_entry.update({
        "copy_reference": copy_ref,
        "vs_copy": None if copy_ref is None else
            round(dec_gbps / copy_ref["achieved"], 4),
        "back_to_back": None if b2b_ms is None else {
            "launches": n_b2b,
            "avg_launch_ms": round(b2b_ms, 5),
            "achieved": round(dec_bytes / (b2b_ms * 1e-3) / 1e9, 2),
            "frac": round(dec_bytes / (b2b_ms * 1e-3) / 1e9 /
                          counts.HBM_PEAK_GBPS, 4),
        },
        "state_pool_back_to_back": None if pool_ms is None else {
            "entry_point": "kda_decode_step_indexed",
            "pool_rows": 3 * dp.B,
            "launches": n_b2b,
            "avg_launch_ms": round(pool_ms, 5),
            "achieved": round(dec_bytes / (pool_ms * 1e-3) / 1e9, 2),
            "frac": round(dec_bytes / (pool_ms * 1e-3) / 1e9 /
                          counts.HBM_PEAK_GBPS, 4),
        }})
    kernels.append(dec_entry)
    # the roofline line is the kernel that takes the largest share of a step
    dominant = max(kernels, key=lambda e: e["avg_launch_ms"])
    # The prefill's place under the roofline by the pages' FLOP count, with
    # the arithmetic intensity taken over the bytes the HBM counters read for
    # its two kernels (when they are current): achieved FLOP/s over
    # min(MFMA peak, intensity x HBM peak).
    pre_traffic = None
    if len(kernels) == 3 and all(e.get("traffic") for e in kernels[:2]):
        pre_traffic = sum(e["traffic"] for e in kernels[:2])
    pages_roof = None
    if pre_traffic:
        ai = pre_flops / pre_traffic
        bound = min(counts.BF16_MFMA_PEAK_TFLOPS,
                    ai * counts.HBM_PEAK_GBPS / 1e3)
        pages_roof = {
            "counter_bytes": int(pre_traffic),
            "ai_flop_per_byte": round(ai, 2),
            "bound_tflops": round(bound, 1),
            "achieved_tflops": round(pre_flops / pre_s / 1e12, 2),
            "frac": round(pre_flops / pre_s / 1e12 / bound, 4),
        }

    result = {
        "metric": METRIC,
        "value": round(dec_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), "
                "g=-5*sigmoid(N(0,1)), beta=sigmoid(N(0,1)), "
                "state N(0,0.02^2))",
        "config": {
            "workload": "KDA decode step: B=64 sequences, H=96, "
                        "d_k=d_v=128, fp32 state in place, bf16 q/k/v; "
                        "each step also runs the chunked prefill below",
            "decode_batch": dp.B, "heads": H, "head_dim": D,
            "prefill_workload": "%s: %d sequence(s), %d tokens, H=%d, d=%d, "
                                "C=%d, %s q/k/v, %s initial state"
                                % (pp.name, nseq, total, pp.H, pp.K, pp.C,
                                   pp.dtype, "zero" if ps0 is None
                                   else "nonzero"),
            "parallelism": "single GPU",
        },
        "roofline": dominant,
        "kernels": kernels,
        "prefill": {
            "tokens_per_s": round(total / pre_s, 1),
            "ms": round(pre_avg, 4),
            "median_ms": round(pre_med, 4),
            "ckpt_every": args.ckpt_every or None,
            "ckpt_slots": None if ck is None else int(ck.shape[0]),
            "unit": "tokens/s",
            "pages_flops": pre_flops,
            "tflops": round(pre_flops / pre_s / 1e12, 2),
            "mfma_util_frac": round(pre_flops / pre_s / 1e12 /
                                    counts.BF16_MFMA_PEAK_TFLOPS, 4),
            "roofline": {
                "kernels": "prep_kernel + recurrence kernel",
                "bound": "hbm",
                "achieved": round(pre_bytes_pages / pre_s / 1e9, 2),
                "peak": counts.HBM_PEAK_GBPS,
                "unit": "GB/s",
                "frac": round(pre_bytes_pages / pre_s / 1e9 /
                              counts.HBM_PEAK_GBPS, 4),
                "algorithmic_bytes": pre_bytes_pages,
                "minimal_bytes": pre_bytes_min,
                "minimal_bytes_frac": round(pre_bytes_min / pre_s / 1e9 /
                                            counts.HBM_PEAK_GBPS, 4),
            },
            "pages_roofline": pages_roof,
        },
        "gpu_clocks": clocks,
    }

    if spec is not None:
        result["spec"] = spec
    if epi is not None:
        result["epilogue"] = epi
    if pro is not None:
        pro["plain_prefill_ms"] = round(pre_avg, 5)
        result["prologue"] = pro
    if legs is not None:
        result["workloads"] = legs

    # ---------------- CPU baseline: the oracle on the host cores -----------
    if not args.no_cpu_baseline:
        cb = cpu_baseline(dp, pp, samples, gpu_res)
        # the GPU's rate over the oracle's on the same workloads
        sp = {"decode": round(dec_gbps / cb["value"], 1),
              "prefill": round(total / pre_s / cb["prefill_tokens_per_s"], 1)}
        for name, leg in (legs or {}).items():
            cw = cb.get("workloads", {}).get(name, {})
            if "tokens_per_s" in leg and cw.get("tokens_per_s"):
                sp[name] = round(leg["tokens_per_s"] / cw["tokens_per_s"], 1)
        cb["gpu_over_cpu"] = sp
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)
    return 0


def _clock_entries(node, path=""):
    """(path, value) leaves of an SMI JSON report whose path names a clock."""
    out = []
    if isinstance(node, dict):
        for k, v in node.items():
            out += _clock_entries(v, path + "/" + str(k))
    elif isinstance(node, list):
        for i, v in enumerate(node):
            out += _clock_entries(v, path + "/" + str(i))
    elif ("clk" in path.lower() or "clock" in path.lower()) and \
            isinstance(node, (int, float, str)):
        out.append((path.strip("/"), node))
    return out


def gpu_clocks(busy=None):
    """The GPU's clocks as its kernel driver reports them (amd-smi, else
    rocm-smi: read-only queries, nothing is pinned or changed), read while
    `busy()` keeps the GPU working, so that the figures are the loaded
    clocks rather than idle ones.  Returns the current gfx clock of each
    XCD, the memory clock, the gfx maximum and whether clocks are locked;
    the raw text when the report is not JSON; or None."""
    import subprocess
    for cmd in (["amd-smi", "metric", "-g", "0", "-c", "--json"],
                ["rocm-smi", "-d", "0", "--showclocks", "--json"]):
        try:
            proc = subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                    stderr=subprocess.DEVNULL, text=True)
        except OSError:
            continue
        t0 = time.perf_counter()
        while proc.poll() is None and time.perf_counter() - t0 < 20:
            if busy is not None:
                busy()
            else:
                time.sleep(0.05)
        if proc.poll() is None:
            proc.kill()
            proc.wait()
            continue
        text = proc.stdout.read()
        if proc.returncode != 0 or not text.strip():
            continue
        try:
            found = _clock_entries(json.loads(text))
        except ValueError:
            return {"tool": cmd[0], "raw": text.strip()[:600]}
        gfx = [v for k, v in found
               if "/gfx_" in k and k.endswith("/clk/value")]
        mem = [v for k, v in found
               if "/mem_" in k and k.endswith("/clk/value")]
        gmax = [v for k, v in found
                if "/gfx_" in k and k.endswith("/max_clk/value")]
        locked = sorted({str(v) for k, v in found if k.endswith("clk_locked")})
        if not gfx:
            return {"tool": cmd[0], "clocks": dict(found[:40])}
        return {"tool": cmd[0], "gfx_reported_mhz": gfx, "mem_mhz": mem,
                "gfx_max_mhz": max(gmax) if gmax else None,
                "clk_locked": locked,
                "read": "while whole steps run; gfx_reported_mhz is the "
                        "driver's sampled figure (it has read 158 to 2,400 "
                        "MHz under the same load), not the kernels' clock"}
    return None


def time_tiny(dev, stream, ev):
    """The tiny fp32 prefill (B=1, H=2, T=64, d=16, C=16) as one
    kda_prefill_chunked call: its device time back to back, and the host's
    latency from the call to its completion."""
    import torch
    from linear_recurrent_attention_kda_amd import kda
    p = inputs.make("tiny", seed=0)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)  # noqa
    q, k, v, g, beta = (t(x) for x in (p.q, p.k, p.v, p.g, p.beta))
    o = torch.empty((p.B, p.T, p.H, p.V), dtype=torch.float32, device=dev)
    fs = torch.empty((p.B, p.H, p.K, p.V), dtype=torch.float32, device=dev)
    ws = kda.workspace_for(p.B, p.B * p.T, p.H, p.K, p.V, p.C, dev)
    run = lambda: kda.kda_prefill_chunked(  # noqa: E731
        q, k, v, g, beta, None, chunk_size=p.C, final_state=fs, o=o,
        workspace=ws)
    for _ in range(10):
        run()
    torch.cuda.synchronize()
    n = 200
    e0, e1 = ev(), ev()
    e0.record(stream)
    for _ in range(n):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    dev_us = e0.elapsed_time(e1) / n * 1e3
    lat = []
    for _ in range(50):
        t0 = time.perf_counter()
        run()
        torch.cuda.synchronize()
        lat.append((time.perf_counter() - t0) * 1e6)
    log("tiny prefill: %.2f us per call back to back, %.1f us call to "
        "completion (median)" % (dev_us, float(np.median(lat))))
    return {"workload": "tiny: B=1, H=2, T=64, d=16, C=16, fp32, zero state",
            "device_us_back_to_back": round(dev_us, 3),
            "latency_us_median": round(float(np.median(lat)), 2),
            "latency_us_min": round(float(np.min(lat)), 2),
            "launches": 2, "tokens": p.B * p.T}


def time_prefill_workload(name, dev, stream, ev, reps=5):
    """One prefill workload (inputs drawn on the device, same recipe as the
    tests' host draws), run as its two stages so that each kernel is timed
    on its own: `reps` launches of each, between events, after two warm-up
    calls.  Returns the leg's figures and a host copy of a head sample for
    the oracle's timing."""
    import torch
    from linear_recurrent_attention_kda_amd import kda
    t_gen = time.time()
    w = inputs.make_device(name, seed=0, device=dev)
    total, H, K, V, C = w["total"], w["H"], w["K"], w["V"], w["C"]
    nseq = len(w["lengths"])
    maxlen = int(w["lengths"].max())
    cu = w["cu_seqlens"]
    o = torch.empty((total, H, V), dtype=w["q"].dtype, device=dev)
    fs = torch.empty((nseq, H, K, V), dtype=torch.float32, device=dev)
    ws = kda.workspace_for(nseq, total, H, K, V, C, dev)
    torch.cuda.synchronize()
    log("%s inputs drawn on the device in %.1fs" % (name, time.time() - t_gen))

    def prep():
        kda.kda_prefill_varlen_prep(w["q"], w["k"], w["v"], w["g"], w["beta"],
                                    cu, maxlen, chunk_size=C, workspace=ws)

    def recur():
        kda.kda_prefill_varlen_recur(ws, cu, maxlen, total, H, K, V,
                                     w["q"].dtype, w["initial_state"],
                                     chunk_size=C, final_state=fs, o=o)
    for _ in range(2):
        prep()
        recur()
    prep_ms, recur_ms = [], []
    for _ in range(reps):
        a, m, b = ev(), ev(), ev()
        a.record(stream)
        prep()
        m.record(stream)
        recur()
        b.record(stream)
        torch.cuda.synchronize()
        prep_ms.append(a.elapsed_time(m))
        recur_ms.append(m.elapsed_time(b))
    tot_ms = float(np.mean(prep_ms)) + float(np.mean(recur_ms))
    chunks = int(np.sum((w["lengths"] + C - 1) // C)) * H
    elt = w["q"].element_size()
    flops = counts.prefill_flops_per_chunk(C, K) * chunks
    log("%s prefill: prep %.4f ms, recurrence %.4f ms"
        % (name, float(np.mean(prep_ms)), float(np.mean(recur_ms))))
    leg = {
        "workload": "%s: %d sequence(s), %d tokens, H=%d, d=%d, C=%d, %s, "
                    "%s initial state" % (name, nseq, total, H, K, C,
                                          w["dtype"], "zero"
                                          if w["initial_state"] is None
                                          else "nonzero"),
        "sequence_lengths": [int(x) for x in w["lengths"]],
        "ms": round(tot_ms, 4),
        "tokens_per_s": round(total / (tot_ms * 1e-3), 1),
        "pages_flops": flops,
        "mfma_util_frac": round(flops / (tot_ms * 1e-3) / 1e12 /
                                counts.BF16_MFMA_PEAK_TFLOPS, 4),
        "kernels": [
            kernel_entry("prep_kernel (kda_prep.hip)", "kda_prep.hip",
                         counts.prep_bytes(total * H, chunks, C, K, V, elt),
                         prep_ms, traffic=False),
            kernel_entry("chunk recurrence (kda_recur.hip)", "kda_recur.hip",
                         counts.recur_bytes(total * H, chunks, C, K, V, elt),
                         recur_ms, traffic=False)],
    }
    leg["gated"] = time_gated_prefill(
        (w["q"], w["k"], w["v"], w["g"], w["beta"]), cu, maxlen, total, H, K,
        V, C, w["initial_state"], ws, dev, stream, ev, n=3)
    # a head sample for the oracle's timing: 16 heads, every token
    nh = min(16, H)
    host = lambda x: x[:, :nh].float().cpu().numpy()  # noqa: E731
    sample = dict(q=host(w["q"]), k=host(w["k"]), v=host(w["v"]),
                  g=host(w["g"]), beta=w["beta"][:, :nh].cpu().numpy(),
                  s0=None if w["initial_state"] is None else
                  w["initial_state"][:, :nh].cpu().numpy(),
                  cu=w["cu_seqlens"].cpu().numpy(), heads=nh, H=H,
                  total=total, C=C,
                  # the plain prefill's results on those heads, for the
                  # oracle leg's parity figures
                  o_gpu=host(o), fs_gpu=fs[:, :nh].cpu().numpy())
    del w, o, fs, ws
    torch.cuda.empty_cache()
    return leg, sample


def time_spec(T, dp, states, dev, stream, ev):
    """Speculative verify of T draft tokens per sequence on the decode
    batch, then commit of all T, against T single decode steps; and the
    fused step (commit of a previous T-token draft, all accepted, then
    verify of the next) against the two calls."""
    import torch
    from linear_recurrent_attention_kda_amd import kda
    sp = inputs.make("varlen", seed=5, H=dp.H, K=dp.K, V=dp.V,
                     lengths=[T] * dp.B)
    B, H = dp.B, dp.H
    shp = lambda x: torch.from_numpy(  # noqa: E731
        np.ascontiguousarray(x.reshape((B, T) + x.shape[1:]))).to(dev)
    q, k, v = (shp(x).to(torch.bfloat16) for x in (sp.q, sp.k, sp.v))
    g, beta = shp(sp.g), shp(sp.beta)
    o = torch.empty((B, T, H, dp.V), dtype=torch.bfloat16, device=dev)
    u = torch.empty((B, T, H, dp.V), dtype=torch.float32, device=dev)
    acc = torch.full((B,), T, dtype=torch.int32, device=dev)
    qs, ks, vs, gs, bs = ([x[:, t].contiguous() for t in range(T)]
                          for x in (q, k, v, g, beta))
    od = torch.empty((B, H, dp.V), dtype=torch.bfloat16, device=dev)
    n = 20

    def timed(fn):
        # n launches back to back between two events (the queue never
        # drains, so host-side gaps do not enter), states rotated so that
        # the 402 MB state is not served from the Infinity Cache
        for i in range(3):
            fn(i)
        e0, e1 = ev(), ev()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ver = timed(lambda i: kda.kda_spec_verify(q, k, v, g, beta, states[i % 3],
                                              o=o, u=u))
    com = timed(lambda i: kda.kda_spec_commit(k, g, u, acc, states[i % 3]))

    def steps(i):
        for t in range(T):
            kda.kda_decode_step(qs[t], ks[t], vs[t], gs[t], bs[t],
                                states[i % 3], o=od)
    dec = timed(steps)
    o2, u2 = torch.empty_like(o), torch.empty_like(u)
    stp = timed(lambda i: kda.kda_spec_step(
        q, k, v, g, beta, states[i % 3], k_prev=k, g_prev=g, u_prev=u,
        accepted_prev=acc, o=o2, u=u2))
    per_head = dp.K * dp.V * 4
    log("spec T=%d: verify %.4f ms, commit %.4f ms, %d decode steps %.4f ms, "
        "fused step %.4f ms" % (T, ver, com, T, dec, stp))
    return {
        "draft_tokens": T, "sequences": B, "heads": H,
        "verify_ms": round(ver, 5), "commit_ms": round(com, 5),
        "verify_commit_ms": round(ver + com, 5),
        "decode_steps_ms": round(dec, 5),
        "verify_state_gbps": round(B * H * per_head / (ver * 1e-3) / 1e9, 1),
        "commit_state_gbps": round(2 * B * H * per_head / (com * 1e-3) / 1e9,
                                   1),
        "speedup_vs_decode_steps": round(dec / (ver + com), 3),
        "step_ms": round(stp, 5),
        "step_state_gbps": round(2 * B * H * per_head / (stp * 1e-3) / 1e9,
                                 1),
        "step_speedup_vs_verify_commit": round((ver + com) / stp, 3),
    }


def time_prologue(pp, nseq, total, ws, dev, stream, ev):
    """Prefill of the same shape with the input prologue fused into the
    chunk-prep kernel (random projected inputs, taps and gate
    pre-activations)."""
    import torch
    from linear_recurrent_attention_kda_amd import kda
    gen = torch.Generator(device=dev).manual_seed(4)
    rn = lambda *shape: torch.randn(shape, generator=gen,  # noqa: E731
                                    device=dev)
    xq, xk = (rn(total, pp.H, pp.K).to(torch.bfloat16) for _ in range(2))
    xv = rn(total, pp.H, pp.V).to(torch.bfloat16)
    w = rn(3, pp.H, pp.K, 4) * 0.5
    a, b = rn(total, pp.H, pp.K), rn(total, pp.H)
    if pp.kind == "varlen":
        cu = torch.from_numpy(pp.cu_seqlens).to(dev)
        maxlen = int(pp.seq_lengths.max())
    else:
        cu = torch.arange(nseq + 1, dtype=torch.int32, device=dev) * pp.T
        maxlen = pp.T
    o = torch.empty((total, pp.H, pp.V), dtype=torch.bfloat16, device=dev)
    fs = torch.empty((nseq, pp.H, pp.K, pp.V), dtype=torch.float32,
                     device=dev)
    run = lambda: kda.kda_prefill_varlen_prologue(  # noqa: E731
        xq, xk, xv, w, a, b, cu, maxlen, None, chunk_size=pp.C,
        final_state=fs, o=o, workspace=ws)
    for _ in range(3):
        run()
    e0, e1 = ev(), ev()
    e0.record(stream)
    n = 10
    for _ in range(n):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    log("prologue-fused prefill: %.4f ms" % ms)
    return {"fused_prefill_ms": round(ms, 5),
            "tokens_per_s": round(total / (ms * 1e-3), 1)}


def time_gated_prefill(ins, cu, maxlen, total, H, K, V, C, s0, ws, dev,
                       stream, ev, n=5):
    """kda_prefill_varlen_gated (the output epilogue fused into the
    recurrence when there are at least two (sequence, head) pairs per
    compute unit, else the plain recurrence then the epilogue kernel),
    against the plain prefill followed by kda_output_norm_gate; each n
    launches back to back between two events, the fastest of four rounds."""
    import torch
    from linear_recurrent_attention_kda_amd import kda
    q, k, v, g, beta = ins
    nseq = len(cu) - 1
    gen = torch.Generator(device=dev).manual_seed(6)
    z = torch.randn((total, H, V), generator=gen, device=dev).to(q.dtype)
    w = 1.0 + 0.3 * torch.randn(V, generator=gen, device=dev)
    y = torch.empty_like(z)
    o = torch.empty_like(z)
    fs = torch.empty((nseq, H, K, V), dtype=torch.float32, device=dev)

    def gated():
        kda.kda_prefill_varlen_gated(q, k, v, g, beta, cu, maxlen, s0, z=z,
                                     w=w, chunk_size=C, final_state=fs, y=y,
                                     workspace=ws)

    def two_pass():
        kda.kda_prefill_varlen(q, k, v, g, beta, cu, maxlen, s0,
                               chunk_size=C, final_state=fs, o=o,
                               workspace=ws)
        kda.kda_output_norm_gate(o, z, w, y=y)

    def timed(fn):
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n
    # Both paths warmed up, then timed alternately in four rounds, each path
    # first in every other round, keeping each path's fastest round:
    # whichever is timed first otherwise pays for the clock and cache state
    # the previous legs left behind (measured up to 12 % on the 8K-token
    # prefill).
    for _ in range(3):
        gated()
        two_pass()
    torch.cuda.synchronize()
    t_g = t_2 = float("inf")
    for r in range(4):
        if r % 2 == 0:
            t_g = min(t_g, timed(gated))
            t_2 = min(t_2, timed(two_pass))
        else:
            t_2 = min(t_2, timed(two_pass))
            t_g = min(t_g, timed(gated))
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    path = "fused" if nseq * H >= 2 * cus else "two-pass"
    log("gated prefill (%s): %.4f ms; plain + epilogue %.4f ms"
        % (path, t_g, t_2))
    return {"gated_ms": round(t_g, 5), "gated_path": path,
            "plain_then_epilogue_ms": round(t_2, 5)}


def time_epilogue(po, dq, dk, dv, dg, dbeta, states, dev, stream, ev):
    """Output epilogue: standalone over the prefill output (HBM GB/s), and
    the decode step with the epilogue fused against the plain decode step."""
    import torch
    from linear_recurrent_attention_kda_amd import kda
    gen = torch.Generator(device=dev).manual_seed(3)
    z = torch.randn(po.shape, generator=gen, device=dev).to(po.dtype)
    w = torch.randn(po.shape[-1], generator=gen, device=dev)
    y = torch.empty_like(po)
    zd = torch.randn(dq.shape[:2] + (dv.shape[-1],), generator=gen,
                     device=dev).to(dq.dtype)
    n = 10
    for _ in range(3):
        kda.kda_output_norm_gate(po, z, w, y=y)
    a0, a1 = ev(), ev()
    a0.record(stream)
    for _ in range(n):
        kda.kda_output_norm_gate(po, z, w, y=y)
    a1.record(stream)
    torch.cuda.synchronize()
    epi_ms = a0.elapsed_time(a1) / n
    nbytes = 3 * po.numel() * po.element_size()

    def timed(fn):
        # back-to-back launches on rotating states (see time_spec)
        for i in range(3):
            fn(i)
        e0, e1 = ev(), ev()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    gated = timed(lambda i: kda.kda_decode_step_gated(
        dq, dk, dv, dg, dbeta, states[i % 3], zd, w))
    plain = timed(lambda i: kda.kda_decode_step(dq, dk, dv, dg, dbeta,
                                                states[i % 3]))
    log("epilogue: standalone %.4f ms; decode gated %.4f ms vs plain %.4f ms"
        % (epi_ms, gated, plain))
    return {
        "standalone_rows": int(po.numel() // po.shape[-1]),
        "standalone_ms": round(epi_ms, 5),
        "standalone_gbps": round(nbytes / (epi_ms * 1e-3) / 1e9, 1),
        "standalone_bytes": nbytes,
        "decode_gated_ms": round(gated, 5),
        "decode_plain_ms": round(plain, 5),
    }


def host_cpus() -> int:
    """CPUs this process may run on (its affinity mask), else the count."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def _rel_per_slice(x, ref, cu=None):
    """Largest max|x - ref| / max|ref| over the (sequence, head) slices of
    [tokens, heads, d] outputs (cu: sequence bounds) or over the leading two
    axes of [sequences, heads, ...] states and decode outputs (cu None)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    if cu is None:
        ax = tuple(range(2, x.ndim))
        num = np.max(np.abs(x - ref), axis=ax)
        den = np.maximum(np.max(np.abs(ref), axis=ax), 1e-30)
        return float(np.max(num / den)) if num.size else 0.0
    worst = 0.0
    for b, e in zip(cu[:-1], cu[1:]):
        if e > b:
            num = np.max(np.abs(x[b:e] - ref[b:e]), axis=(0, 2))
            den = np.maximum(np.max(np.abs(ref[b:e]), axis=(0, 2)), 1e-30)
            worst = max(worst, float(np.max(num / den)))
    return worst


def cpu_baseline(dp, pp, samples=None, gpu=None):
    """Time the fp64 oracle (as it stands) on a bounded sample of the same
    workloads: the whole decode step, the prefill over a head sample of all
    of its tokens (scaled to all heads), and the same for the other
    workloads' legs.  Threads: every CPU the process may use, capped at 16,
    the host-CPU share of one GPU on the machines this runs on."""
    import oracle
    oracle.build(force=False)
    threads = max(1, min(16, host_cpus()))
    oracle.set_threads(threads)
    # each leg repeats (same inputs, results discarded) until it has run
    # for a few seconds, so that the rate is not one short noisy sample
    # The first run of each leg also gives the parity figures: the GPU's
    # results on the same inputs against the oracle's, per (sequence, head),
    # as the tests measure them (bars: 2e-2 for prefill outputs and states,
    # 1e-4 for the fp32 decode state).
    gpu = gpu or {}
    parity = {}
    dec_reps, t = 0, time.perf_counter()
    while dec_reps == 0 or time.perf_counter() - t < 4.0:
        r = oracle.run_decode(dp.q, dp.k, dp.v, dp.g, dp.beta,
                              dp.initial_state)
        if dec_reps == 0 and "decode" in gpu:
            parity["decode_o"] = _rel_per_slice(gpu["decode"][0], r[0])
            parity["decode_state"] = _rel_per_slice(gpu["decode"][1], r[1])
        dec_reps += 1
    dec_s = (time.perf_counter() - t) / dec_reps
    dec_bytes = counts.decode_bytes_per_head(dp.K) * dp.B * dp.H
    # prefill sample: about 96 x 8192 token-heads (the whole 8K-token,
    # 96-head workload; a proportional number of heads of larger ones)
    total_tokens = (int(pp.cu_seqlens[-1]) if pp.kind == "varlen"
                    else pp.B * pp.T)
    nh = max(1, min(pp.H, (96 * 8192) // max(1, total_tokens)))
    heads = list(range(nh))
    sel = lambda x: x[..., heads, :]  # noqa: E731
    s0 = None if pp.initial_state is None else pp.initial_state[:, heads]
    pre_reps, t = 0, time.perf_counter()
    while pre_reps == 0 or time.perf_counter() - t < 6.0:
        if pp.kind == "varlen":
            r = oracle.run_varlen(sel(pp.q), sel(pp.k), sel(pp.v), sel(pp.g),
                                  pp.beta[..., heads], pp.cu_seqlens, s0)
        else:
            r = oracle.run_fixed(sel(pp.q), sel(pp.k), sel(pp.v), sel(pp.g),
                                 pp.beta[..., heads], s0)
        if pre_reps == 0 and "prefill" in gpu:
            go, gs = gpu["prefill"]
            cu = (pp.cu_seqlens if pp.kind == "varlen" else
                  np.arange(pp.B + 1) * pp.T)
            ref_o = np.asarray(r[0]).reshape((-1,) + r[0].shape[-2:])
            parity["prefill_o"] = _rel_per_slice(
                go.reshape((-1,) + go.shape[-2:])[:, heads], ref_o, cu)
            parity["prefill_state"] = _rel_per_slice(gs[:, heads], r[1])
        pre_reps += 1
    pre_s = (time.perf_counter() - t) / pre_reps
    total = int(pp.cu_seqlens[-1]) if pp.kind == "varlen" else pp.B * pp.T
    pre_tps = total / (pre_s * pp.H / len(heads))
    log("oracle: decode %.3fs x %d, prefill sample %.3fs x %d"
        % (dec_s, dec_reps, pre_s, pre_reps))
    legs = {}
    for name, smp in (samples or {}).items():
        reps, t = 0, time.perf_counter()
        while reps == 0 or time.perf_counter() - t < 2.0:
            r = oracle.run_varlen(smp["q"], smp["k"], smp["v"], smp["g"],
                                  smp["beta"], smp["cu"], smp["s0"])
            if reps == 0 and "o_gpu" in smp:
                parity[name + "_o"] = _rel_per_slice(smp["o_gpu"], r[0],
                                                     smp["cu"])
                parity[name + "_state"] = _rel_per_slice(smp["fs_gpu"], r[1])
            reps += 1
        sec = (time.perf_counter() - t) / reps
        legs[name] = {
            "tokens_per_s": round(smp["total"] / (sec * smp["H"] /
                                                  smp["heads"]), 1),
            "sample": "%d of %d heads over all %d tokens, scaled to all "
                      "heads, mean of %d runs" % (smp["heads"], smp["H"],
                                                   smp["total"], reps),
            "sample_seconds": round(sec, 4)}
        log("oracle: %s sample %.3fs x %d" % (name, sec, reps))
    tiny = inputs.make("tiny", seed=0)
    reps, t = 0, time.perf_counter()
    while reps == 0 or time.perf_counter() - t < 0.5:
        oracle.run_fixed(tiny.q, tiny.k, tiny.v, tiny.g, tiny.beta)
        reps += 1
    legs["tiny"] = {"seconds_per_call": round((time.perf_counter() - t) /
                                              reps, 7), "runs": reps}
    return {
        "value": round(dec_bytes / dec_s / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "threads": threads,
        "host_cpus": os.cpu_count(),
        "affinity_cpus": host_cpus(),
        "kind": "oracle",
        "parity": {k: float("%.3e" % v) for k, v in parity.items()},
        "sample": "whole decode step (%dx%d heads, d=%d) in fp64, mean of "
                  "%d runs; prefill: %d of %d heads over all %d tokens, "
                  "scaled to all heads, mean of %d runs"
                  % (dp.B, dp.H, dp.K, dec_reps, len(heads), pp.H, total,
                     pre_reps),
        "prefill_tokens_per_s": round(pre_tps, 1),
        "workloads": legs,
        "decode_seconds": round(dec_s, 4),
        "prefill_sample_seconds": round(pre_s, 4),
        "cpu_model": cpu_model(),
    }


if __name__ == "__main__":
    sys.exit(main())
