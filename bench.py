#!/usr/bin/env python3
"""Benchmark of the A2ATS key-cache hot path on one MI355X.

Headline: the large-codebook H-weighted encode (8 KV heads x 131072 bf16 keys, d = 128,
C = 4096 centroids per head, L from 8192 correlated queries per head, codes + argmin
distances).  One step = one a2ats_encode call: the codebook side (M = L L^T, v = c M,
b = ||c L||^2, fp16 fragments) and the key side (the MFMA pass with its certificate and
fp64 rerank, the rescan of the keys left open).  `value` = keys encoded per second of that
call, inputs resident in HBM.  `roofline` describes the MFMA pass (enc_coarse): 2 N C d
flop per launch over its average launch duration, recorded with HIP events around the
library's own launches on the launch stream.

Also reported (field "extra"): the same encode with the codebook prepared once; the
per-layer cache update of a Llama-3.2-3B-shaped layer (split, plain + H-weighted encode,
bf16 reconstruct; HIP graph replays); the decode step (fp32 reconstruct of 32 x 8 x 16384
tokens, blend of the new keys, far-unrotated update, top-K over codes) and the long-context
pipeline (5% split, C = 2048, W = 1024) with HBM fractions; the sub-vector default
configuration and codebook training.

Modes for the committed counter summaries (rocprofv3 runs these; see profiles/):
  --pmc-probe WORKLOAD     a few calls of one workload plus a 256 MiB reference copy
  --pmc-summarize DIR      turns the --pmc passes under DIR into profiles/*_pmc.{json,md}
  --trace-summarize DIR    turns a --kernel-trace --stats run into profiles/*_trace.md

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2516.6   # MI355X dense fp16/bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector (256 CU x 2.4 GHz x 256 flop/clk with FMA)
PEAK_FP64_TFLOPS = 78.6        # MI355X fp64 vector and matrix (an FMA counted as two operations)
METRIC = "keys encoded/sec (H-weighted VQ, d=128) + % MFMA peak; reconstruct GB/s"
COPY_REF_BYTES = 256 * 2 ** 20
D = 128


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sha_of(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-probe", metavar="WORKLOAD",
                    choices=sorted(PROBES),
                    help="a few calls of one workload and a 256 MiB reference copy, for "
                         "rocprofv3 --pmc")
    ap.add_argument("--pmc-summarize", metavar="DIR",
                    help="turn the rocprofv3 --pmc passes under DIR (subdirectories named "
                         "<workload>_<pass>) into profiles/<kernel>_<workload>_pmc.{json,md}")
    ap.add_argument("--trace-summarize", metavar="DIR",
                    help="turn a rocprofv3 --kernel-trace --stats output under DIR into "
                         "profiles/<name>_trace.md")
    ap.add_argument("--trace-name", default="encode_stress",
                    help="the workload the trace covers, naming its summary file")
    ap.add_argument("--command", default="",
                    help="the command lines that produced the profiler output (recorded in the "
                         "summary); by default they are rebuilt from what the profiler recorded")
    args = ap.parse_args()
    if args.pmc_summarize:
        pmc_summarize(args.pmc_summarize, args.command)
        return
    if args.trace_summarize:
        trace_summarize(args.trace_summarize, args.command, args.trace_name)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py: this build runs on exactly one GPU; --gpus %d (world size %d) is not "
                  "supported" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    import kv_cache_vector_windowed_amd as kv
    from kv_cache_vector_windowed_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ctx = Ctx(torch, kv, synth, dev)
    if args.pmc_probe:
        PROBES[args.pmc_probe](ctx)
        ctx.copy_reference()
        print(json.dumps({"pmc_probe": args.pmc_probe, "copy_ref_bytes": COPY_REF_BYTES}), flush=True)
        return

    head = headline(ctx, args.steps, args.warmup)
    extra = dict(head.pop("extra"))
    if not args.no_extra:
        extra.update(extra_workloads(ctx, args.steps, args.warmup))
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(synth)
    w = synth.WORKLOADS["encode_stress"]
    line = {
        "metric": METRIC, "value": head["value"], "unit": "keys/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "encode_stress: 8 KV heads x 131072 tokens x d=128 bf16 keys, "
                               "C=4096 centroids per head, H-weighted (L from 8192 queries per "
                               "head, ridge 1e-4), codes + argmin distances; step = one "
                               "a2ats_encode call (codebook side + key side)",
                   "heads": w.heads, "tokens": w.n, "centroids": w.c, "head_dim": D,
                   "calibration_queries": w.m, "distances": True},
        "roofline": head["roofline"], "cpu_baseline": cpu, "extra": extra,
    }
    print(json.dumps(line), flush=True)


class Ctx:
    """Device, modules and helpers shared by the workloads."""

    def __init__(self, torch, kv, synth, dev):
        self.torch, self.kv, self.synth, self.dev = torch, kv, synth, dev
        self._flush = None

    def keys_dev(self, k):
        return self.torch.from_numpy(k.bits.view(np.int16)).to(self.dev).view(self.torch.bfloat16)

    def f32(self, a):
        return self.torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(self.dev)

    def profile(self, fn, reps):
        """{kernel: (launches, mean ms)} from the HIP events the library records around each
        of its own launches, on the stream each kernel is launched on."""
        kv = self.kv
        kv.profile_reset()
        kv.profile_enable(True)
        for _ in range(reps):
            fn()
        self.torch.cuda.synchronize()
        prof = kv.profile_read()
        kv.profile_enable(False)
        kv.profile_reset()
        return {k: (c, t / c) for k, (c, t) in prof.items()}

    def flush_buf(self):
        if self._flush is None:
            self._flush = self.torch.ones(2 ** 28, dtype=self.torch.float32, device=self.dev)  # 1 GiB
            self._flush.sum()  # the first reduction launch carries a one-time setup cost
            self.torch.cuda.synchronize()
        return self._flush

    def timed(self, fn, reps, flush=False):
        """ms per call of fn, calls issued back to back on the stream so the host's issue time
        overlaps the GPU's work.  With flush, a read of a 1 GiB buffer (which evicts the
        256 MB last-level cache with clean lines) precedes every call, and the same number of
        reads timed alone is subtracted.  A kernel that follows a large streaming kernel runs
        measurably slower than in a back-to-back steady state on this GPU, so both figures
        are reported for the HBM paths."""
        torch = self.torch
        buf = self.flush_buf() if flush else None

        def run(with_fn):
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                if flush:
                    buf.sum()
                if with_fn:
                    fn()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b)

        fn()
        t = run(True)
        if flush:
            t -= run(False)
        return t / reps

    def fill_rate(self, nbytes):
        """(flushed ms, steady ms) of a plain fill (torch's fill_) of nbytes: the write-only rate
        this GPU reaches under the same timing, the yardstick of a pass whose traffic is almost
        all writes (the reconstruct)."""
        torch = self.torch
        buf = torch.empty(nbytes // 4, dtype=torch.float32, device=self.dev)

        def fill():
            buf.fill_(1.0)

        fill()
        torch.cuda.synchronize()
        out = (self.timed(fill, 5, flush=True), self.timed(fill, 10))
        del buf
        return out

    def copy_reference(self):
        """A plain elementwise kernel that reads and writes COPY_REF_BYTES: the scale of the
        FETCH_SIZE / WRITE_SIZE counters."""
        torch = self.torch
        src = torch.ones(COPY_REF_BYTES // 4, dtype=torch.float32, device=self.dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()


# ---------------------------------------------------------------------------- headline
class EncodeStress:
    """The large-codebook encode inputs, resident on the device, and its one-call step."""

    def __init__(self, ctx):
        torch, kv, synth = ctx.torch, ctx.kv, ctx.synth
        w = synth.WORKLOADS["encode_stress"]
        self.w = w
        log("generating encode_stress inputs")
        self.kd = ctx.keys_dev(synth.keys(w.cfg, w.heads, w.n, "bf16"))
        self.cbd = ctx.f32(synth.codebook(w.cfg, w.heads, w.c))
        self.qd = ctx.f32(synth.queries(w.cfg, w.heads, w.m))
        t0 = time.perf_counter()
        _, self.L = kv.calibrate(self.qd, 1e-4)  # waits: reports a non-positive-definite H
        self.calib_ms = (time.perf_counter() - t0) * 1e3
        self.codes = torch.zeros((w.heads, w.n), dtype=torch.uint16, device=ctx.dev)
        self.dist = torch.zeros((w.heads, w.n), dtype=torch.float32, device=ctx.dev)
        self.stats = torch.zeros(8, dtype=torch.int32, device=ctx.dev)
        self.ws = torch.empty(kv.encode_workspace_bytes(w.heads, w.n, w.c), dtype=torch.uint8,
                              device=ctx.dev)
        self.kv = kv
        self.flops = 2.0 * w.heads * w.n * w.c * D

    def step(self, stats=False):
        self.kv.encode(self.kd, self.cbd, self.L, codes=self.codes, dist=self.dist,
                       stats=self.stats if stats else None, workspace=self.ws)


def headline(ctx, steps, warmup):
    torch, kv = ctx.torch, ctx.kv
    e = EncodeStress(ctx)
    w = e.w
    for _ in range(max(warmup, 1)):
        e.step()
    torch.cuda.synchronize()
    log("timing %d encode calls" % steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        e.step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    keys = w.heads * w.n
    value = keys / (ms * 1e-3)
    log("encode_stress call %.4f ms -> %.4g keys/s" % (ms, value))
    pr = ctx.profile(e.step, min(steps, 10))
    log("kernels: " + ", ".join("%s %.1fus" % (k, v[1] * 1e3) for k, v in pr.items()))
    coarse_ms = pr["encode_coarse_h"][1]
    achieved = e.flops / (coarse_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": "encode_coarse_h (enc_coarse, bf16 keys, H, distances)",
                "achieved": round(achieved, 2), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_MFMA_TFLOPS, 4),
                "traffic": traffic_from_profiles("enc_coarse", "encode_stress"),
                "launch_us": round(coarse_ms * 1e3, 2), "flops_per_launch": e.flops,
                "call_achieved": round(e.flops / (ms * 1e-3) / 1e12, 2),
                "call_frac": round(e.flops / (ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4)}
    # decision statistics of one call; the key side alone with the codebook prepared once
    e.step(stats=True)
    torch.cuda.synchronize()
    st = e.stats.cpu().numpy().tolist()
    prep = kv.encode_prepare(e.cbd, e.L, w.n)

    def prepared():
        kv.encode_prepared(e.kd, prep, codes=e.codes, dist=e.dist)

    ms_p = ctx.timed(prepared, steps)
    pr_p = ctx.profile(lambda: prep.prepare(e.cbd, e.L), 5)
    extra = {
        "encode_stress_kernels_us": {k: round(v[1] * 1e3, 2) for k, v in pr.items()},
        "encode_stress_decided": {"keys": st[0], "direct": st[1], "reranked": st[2],
                                  "rescanned": st[3], "full_scan": st[4]},
        "encode_stress_prepared_ms": round(ms_p, 4),
        "encode_stress_prepared_keys_per_s": round(keys / (ms_p * 1e-3), 1),
        "encode_stress_prepared_mfma_frac": round(e.flops / (ms_p * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
        "encode_stress_prepare_us": round(sum(v[1] for v in pr_p.values()) * 1e3, 2),
        "encode_stress_calibrate_ms_host_clock": round(e.calib_ms, 3),
    }
    log("encode_stress extra %s" % extra)
    del prep
    return {"value": round(value, 1), "ms": round(ms, 5), "roofline": roofline, "extra": extra}


# ---------------------------------------------------------------------------- extra workloads
def layer_step(ctx, steps, warmup):
    """The per-layer cache update of a Llama-3.2-3B-shaped layer: 8 KV heads x 32768 bf16
    keys, C = 1024, H from 4096 queries, W = 512, retrieval fraction 0.1.  One step = split
    (with the codebook side of both encodes on a second stream) -> plain encode of the bulk
    rows and, on the second stream, H-weighted encode of the retrieval rows -> bf16
    reconstruct.  Timed as K replays of the step captured in a HIP graph; the same K steps
    launched one by one are reported too."""
    torch, kv, synth, dev = ctx.torch, ctx.kv, ctx.synth, ctx.dev
    w = synth.WORKLOADS["layer"]
    log("generating layer inputs")
    keys = synth.keys(w.cfg, w.heads, w.n, "bf16")
    kd = ctx.keys_dev(keys)
    cbd = ctx.f32(synth.codebook(w.cfg, w.heads, w.c))
    qd = ctx.f32(synth.queries(w.cfg, w.heads, w.m))
    pos = torch.arange(w.n, dtype=torch.int32, device=dev)[None]
    proxy = kd[:, -1].contiguous()
    H, L = kv.calibrate(qd, 1e-4)
    codes = torch.zeros((w.heads, w.n), dtype=torch.uint16, device=dev)
    out = torch.empty((1, w.heads, w.n, 128), dtype=torch.bfloat16, device=dev)
    # Every step redoes the codebook side of both encodes (it depends on the codebook and L
    # only) on a second stream (default priority) while the split runs; the two key-side
    # passes write disjoint rows (bulk: plain, retrieval: H-weighted), so the small
    # H-weighted one also runs on the second stream beside the plain one.
    aux = torch.cuda.Stream(device=dev)
    main_s = torch.cuda.current_stream(ctx.dev)
    prep_plain = kv.encode_prepare(cbd, None, w.n)
    prep_h = kv.encode_prepare(cbd, L, w.n)

    def step():
        main_s = torch.cuda.current_stream(ctx.dev)  # the capturing stream inside a graph capture
        aux.wait_event(main_s.record_event())
        with torch.cuda.stream(aux):
            prep_plain.prepare(cbd, None)
            plain_ready = aux.record_event()
            prep_h.prepare(cbd, L)
        ret, bulk = kv.select_retrieval(kd, proxy, w.fraction)
        split_done = main_s.record_event()
        main_s.wait_event(plain_ready)
        kv.encode_prepared(kd, prep_plain, idx=bulk, codes=codes)
        aux.wait_event(split_done)
        with torch.cuda.stream(aux):
            kv.encode_prepared(kd, prep_h, idx=ret, codes=codes)
        main_s.wait_event(aux.record_event())
        kv.reconstruct(codes[None], pos, cbd, w.cur_pos, w.window, out=out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_eager = e0.elapsed_time(e1) / steps
    # The same step captured once in a HIP graph (the launches of both streams, replayed as
    # one).  A replay must reproduce the eager step's codes and keys bit for bit.
    ref_codes, ref_out = codes.clone(), out.view(torch.int16).clone()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(main_s)
    with torch.cuda.stream(side):
        step()
    main_s.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    codes.fill_(0)
    graph.replay()
    torch.cuda.synchronize()
    if not (torch.equal(codes, ref_codes) and torch.equal(out.view(torch.int16), ref_out)):
        raise SystemExit("graph replay differs from the eager step")
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # the replays above keep the step's 64 MB of keys in the 256 MB last-level cache; after a
    # cache-evicting read each replay reads them from HBM
    ms_flushed = ctx.timed(graph.replay, 5, flush=True)

    def step_seq():  # the same launches on one stream: per-kernel times without overlap
        prep_plain.prepare(cbd, None)
        prep_h.prepare(cbd, L)
        ret, bulk = kv.select_retrieval(kd, proxy, w.fraction)
        kv.encode_prepared(kd, prep_h, idx=ret, codes=codes)
        kv.encode_prepared(kd, prep_plain, idx=bulk, codes=codes)
        kv.reconstruct(codes[None], pos, cbd, w.cur_pos, w.window, out=out)

    prof = ctx.profile(step_seq, min(steps, 20))
    coarse_ms = prof["encode_coarse_plain"][1]
    n_bulk = w.n - kv.retrieval_count(w.n, w.fraction)  # rows of the plain pass
    flops = 2.0 * w.heads * n_bulk * w.c * 128
    res = {
        "workload": "8 KV heads x 32768 bf16 keys, C=1024, H from 4096 queries, W=512, retrieval "
                    "fraction 0.1; step = split + plain encode of bulk rows || H-weighted encode "
                    "of retrieval rows + bf16 reconstruct",
        "step_ms_graph": round(ms, 5), "keys_per_s_graph": round(w.heads * w.n / (ms * 1e-3), 1),
        "step_ms_graph_flushed": round(ms_flushed, 5),
        "keys_per_s_graph_flushed": round(w.heads * w.n / (ms_flushed * 1e-3), 1),
        "step_ms_eager": round(ms_eager, 5),
        "coarse_plain_us": round(coarse_ms * 1e3, 2),
        "coarse_plain_mfma_frac": round(flops / (coarse_ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
        "kernels_us": {k: round(v[1] * 1e3, 2) for k, v in prof.items()},
    }
    log("layer %s" % res)
    return res


def extra_workloads(ctx, steps, warmup):
    torch, kv, synth = ctx.torch, ctx.kv, ctx.synth
    W = synth.WORKLOADS
    res = {"layer": layer_step(ctx, min(steps, 50), warmup)}
    # decode step
    w = W["decode"]
    log("generating decode inputs")
    cbd = ctx.f32(synth.codebook(w.cfg, w.heads, w.c))
    codes = torch.from_numpy(synth.uniform_codes(w.cfg, (w.batch, w.heads, w.n), w.c).view(np.int16)).to(ctx.dev).view(torch.uint16)
    pos = torch.arange(w.n, dtype=torch.int32, device=ctx.dev)[None].repeat(w.batch, 1).contiguous()
    out = torch.empty((w.batch, w.heads, w.n, 128), dtype=torch.float32, device=ctx.dev)
    newk = ctx.f32(synth.new_keys(w.cfg, w.heads, w.batch))

    def rec():
        kv.reconstruct(codes, pos, cbd, w.cur_pos, w.window, out=out)

    def blend():
        kv.assign_cosine(newk, newk, cbd, w.betas[0])

    rec()
    blend()
    torch.cuda.synchronize()
    ms_r = ctx.timed(rec, 5, flush=True)
    ms_r_steady = ctx.timed(rec, 10)
    ms_b = ctx.timed(blend, 10)
    tokens = w.batch * w.heads * w.n
    alg = tokens * (2 + 128 * 4) + w.batch * w.n * 4 + w.heads * w.c * 128 * 4
    pr = ctx.profile(rec, 3)
    kr = pr["reconstruct"][1]
    res["decode"] = {
        "workload": "32 sequences x 8 heads x 16384 tokens, fp32 out, W=256; blend of 256 new keys",
        "reconstruct_ms": round(ms_r, 4), "reconstruct_GBps": round(alg / (ms_r * 1e-3) / 1e9, 1),
        "reconstruct_call_hbm_frac": round(alg / (ms_r * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "reconstruct_steady_ms": round(ms_r_steady, 4),
        "reconstruct_steady_hbm_frac": round(alg / (ms_r_steady * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "reconstruct_kernel_us": round(kr * 1e3, 2),
        "reconstruct_kernel_GBps": round(alg / (kr * 1e-3) / 1e9, 1),
        "reconstruct_hbm_frac": round(alg / (kr * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "algorithmic_bytes": alg, "blend_us": round(ms_b * 1e3, 2),
    }
    fl_ms, fs_ms = ctx.fill_rate(tokens * 128 * 4)  # a plain fill of the output's bytes
    res["decode"]["fill_output_bytes_flushed_hbm_frac"] = round(
        tokens * 128 * 4 / (fl_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    res["decode"]["fill_output_bytes_steady_hbm_frac"] = round(
        tokens * 128 * 4 / (fs_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    log("decode %s" % res["decode"])
    # Far keys left unrotated (Eq. 12) with R_b on the query (Eq. 11): a decode step then
    # rewrites only the rows that cross the window edge plus the appended token, and rotates
    # the step's queries once.  Same cache; step from cur - 1 to cur, the last token new.
    cur = w.cur_pos
    kv.reconstruct(codes, pos, cbd, cur - 1, w.window, far_mode=kv.FAR_UNROTATED, out=out)

    def upd():
        kv.reconstruct_update(codes, pos, cbd, w.n - 1, cur - 1, cur, w.window, out)

    def full_unrot():
        kv.reconstruct(codes, pos, cbd, cur, w.window, far_mode=kv.FAR_UNROTATED, out=out)

    qh = 24  # query heads of the 8-KV-head layer (grouped-query attention, 3 per KV head)
    qd = torch.randn((w.batch, qh, 128), dtype=torch.float32, device=ctx.dev)
    qo = torch.empty_like(qd)

    def qrope():
        kv.far_query_rope(qd, 2048, out=qo)

    upd()
    torch.cuda.synchronize()
    ms_u = ctx.timed(upd, 20)
    ms_fu = ctx.timed(full_unrot, 5)
    ms_q = ctx.timed(qrope, 20)
    pr_u = ctx.profile(upd, 5)
    rows_step = w.batch * w.heads * 2  # the token leaving the window and the appended token
    res["decode_unrotated"] = {
        "workload": "same cache, far keys unrotated; one decode step (cur-1 -> cur, one token "
                    "appended per sequence); queries 32 x 24 heads",
        "update_us": round(ms_u * 1e3, 2), "update_kernel_us": round(pr_u["reconstruct_update"][1] * 1e3, 2),
        "rows_written": rows_step, "full_reconstruct_us": round(ms_fu * 1e3, 2),
        "speedup_vs_full": round(ms_fu / ms_u, 1),
        "update_bytes": w.batch * w.n * 4 + rows_step * (2 + 512),
        "far_query_rope_us": round(ms_q * 1e3, 2),
    }
    log("decode_unrotated %s" % res["decode_unrotated"])
    del out
    # Top-K retrieval over the same codes: rotate the step's queries by R_b, score every token
    # through the per-query table (q R_b) . c_j gathered by code, keep the best 10%.
    wt = W["topk_decode"]
    kt = int(np.ceil(wt.fraction * wt.n))
    qt = torch.from_numpy(np.ascontiguousarray(
        synth.queries(wt.cfg, wt.q_heads, wt.batch).transpose(1, 0, 2))).to(ctx.dev)
    qtb = torch.empty_like(qt)
    t_idx = torch.empty((wt.batch, wt.q_heads, kt), dtype=torch.int32, device=ctx.dev)

    def topk_step():
        kv.far_query_rope(qt, wt.far_b, out=qtb)
        kv.topk_codes(qtb, codes, cbd, kt)

    topk_step()
    torch.cuda.synchronize()
    ms_t = ctx.timed(topk_step, 20)
    ms_tf = ctx.timed(topk_step, 5, flush=True)
    ms_tc = ctx.timed(lambda: kv.topk_codes(qtb, codes, cbd, kt), 20)  # both launches, no events
    pr_t = ctx.profile(topk_step, 5)
    tab_us = pr_t["topk_table"][1] * 1e3
    sel_us = pr_t["topk_codes"][1] * 1e3
    kt_us = tab_us + sel_us  # both launches of a2ats_topk_codes
    t_bytes = (wt.batch * wt.heads * wt.n * 2 + wt.heads * wt.c * 128 * 4
               + wt.batch * wt.q_heads * (128 * 4 + kt * 8))
    t_flops = 2.0 * wt.batch * wt.q_heads * wt.c * 128  # fp64 table: one fma a term
    res["topk_decode"] = {
        "workload": "32 sequences x 24 query heads over 8 key heads x 16384 codes, C=1024, "
                    "k=%d (10%%); far query rotation + table + top-K" % kt,
        "step_us": round(ms_t * 1e3, 2), "step_flushed_us": round(ms_tf * 1e3, 2),
        "topk_call_us": round(ms_tc * 1e3, 2),
        "topk_kernel_us": round(kt_us, 2),
        "topk_table_us": round(tab_us, 2), "topk_select_us": round(sel_us, 2),
        "far_query_rope_us": round(pr_t["far_query_rope"][1] * 1e3, 2),
        "algorithmic_bytes": t_bytes, "kernel_GBps": round(t_bytes / (kt_us * 1e-6) / 1e9, 1),
        "table_fp64_ops": t_flops,
        # the table kernel on the fp64 matrix cores against their peak
        "table_fp64_frac": round(t_flops / (tab_us * 1e-6) / 1e12 / PEAK_FP64_TFLOPS, 4),
    }
    log("topk_decode %s" % res["topk_decode"])
    # long-context pipeline
    w = W["long_context"]
    log("generating long_context inputs")
    kd = ctx.keys_dev(synth.keys(w.cfg, w.heads, w.n, "bf16"))
    cbd = ctx.f32(synth.codebook(w.cfg, w.heads, w.c))
    _, L = kv.calibrate(ctx.f32(synth.queries(w.cfg, w.heads, w.m)), 1e-4)
    proxy = kd[:, -1].contiguous()
    codes = torch.zeros((w.heads, w.n), dtype=torch.uint16, device=ctx.dev)
    pos = torch.arange(w.n, dtype=torch.int32, device=ctx.dev)[None]
    out = torch.empty((1, w.heads, w.n, 128), dtype=torch.bfloat16, device=ctx.dev)

    def split():
        return kv.select_retrieval(kd, proxy, w.fraction)

    def rec2():
        kv.reconstruct(codes[None], pos, cbd, w.cur_pos, w.window, out=out)

    aux = torch.cuda.Stream(device=ctx.dev)
    main_s = torch.cuda.current_stream(ctx.dev)
    prep_plain = kv.encode_prepare(cbd, None, w.n)
    prep_h = kv.encode_prepare(cbd, L, w.n)

    def pipe():  # as the headline step
        aux.wait_event(main_s.record_event())
        with torch.cuda.stream(aux):
            prep_plain.prepare(cbd, None)
            plain_ready = aux.record_event()
            prep_h.prepare(cbd, L)
        ret, bulk = split()
        split_done = main_s.record_event()
        main_s.wait_event(plain_ready)
        kv.encode_prepared(kd, prep_plain, idx=bulk, codes=codes)
        aux.wait_event(split_done)
        with torch.cuda.stream(aux):
            kv.encode_prepared(kd, prep_h, idx=ret, codes=codes)
        main_s.wait_event(aux.record_event())
        rec2()

    pipe()
    torch.cuda.synchronize()
    ms_s = ctx.timed(split, 10, flush=True)
    ms_r = ctx.timed(rec2, 10, flush=True)
    ms_s_steady = ctx.timed(split, 20)
    ms_r_steady = ctx.timed(rec2, 20)
    ms_p = ctx.timed(pipe, 5)
    split_bytes = w.heads * w.n * (128 * 2 + 4)
    rec_bytes = w.heads * w.n * (2 + 128 * 2) + w.n * 4 + w.heads * w.c * 128 * 4
    pr_s = ctx.profile(split, 5)
    pr_r = ctx.profile(rec2, 5)
    res["long_context"] = {
        "workload": "8 heads x 131072 bf16 keys, 5% split, C=2048, W=1024, bf16 reconstruct",
        "pipeline_ms": round(ms_p, 4), "keys_per_s": round(w.heads * w.n / (ms_p * 1e-3), 1),
        "split_ms": round(ms_s, 4), "split_GBps": round(split_bytes / (ms_s * 1e-3) / 1e9, 1),
        "split_hbm_frac": round(split_bytes / (ms_s * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "split_steady_ms": round(ms_s_steady, 4),
        "split_steady_hbm_frac": round(split_bytes / (ms_s_steady * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "split_kernels_us": {k: round(v[1] * 1e3, 2) for k, v in pr_s.items()},
        "reconstruct_ms": round(ms_r, 4), "reconstruct_GBps": round(rec_bytes / (ms_r * 1e-3) / 1e9, 1),
        "reconstruct_hbm_frac": round(rec_bytes / (ms_r * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "reconstruct_steady_ms": round(ms_r_steady, 4),
        "reconstruct_steady_hbm_frac": round(rec_bytes / (ms_r_steady * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "reconstruct_kernels_us": {k: round(v[1] * 1e3, 2) for k, v in pr_r.items()},
        "pipeline_kernels_us": {k: round(v[1] * 1e3, 2) for k, v in ctx.profile(pipe, 3).items()},
    }
    out_bytes = w.heads * w.n * 128 * 2
    fl_ms, fs_ms = ctx.fill_rate(out_bytes)  # a plain fill of the reconstruct output's bytes
    res["long_context"]["fill_output_bytes_flushed_hbm_frac"] = round(
        out_bytes / (fl_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    res["long_context"]["fill_output_bytes_steady_hbm_frac"] = round(
        out_bytes / (fs_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    log("long_context %s" % res["long_context"])
    del kd, codes, out
    # The pages' default configuration: sub-vector codes (sub_dim 8, one shared 256-entry
    # codebook), keys of the layer shape: split, plain codes for the bulk rows, cosine-blend
    # (beta 0.5; no H) or H-weighted codes for the retrieval rows; values plain; bf16 keys
    # reconstructed with W = 128, values gathered without rotation.
    w = W["pq_layer"]
    log("generating pq_layer inputs")
    kd = ctx.keys_dev(synth.keys(w.cfg, w.heads, w.n, "bf16"))
    vd = ctx.keys_dev(synth.keys(w.cfg, w.heads, w.n, "bf16", stream=8))  # value rows
    cbk = ctx.f32(synth.pq_codebook(w.cfg, w.heads, w.c, 8))
    cbv = ctx.f32(synth.pq_codebook(w.cfg + 100, w.heads, w.c, 8))
    qs = synth.queries(w.cfg, w.heads, w.m)
    _, lq = kv.calibrate(ctx.f32(qs.reshape(1, -1, 8)), 1e-4)
    lq = lq[0].contiguous()
    proxy = kd[:, -1].contiguous()
    ret, bulk = kv.select_retrieval(kd, proxy, w.fraction)
    kc = torch.zeros((w.heads, w.n, 16), dtype=torch.uint8, device=ctx.dev)
    vc = torch.zeros((w.heads, w.n, 16), dtype=torch.uint8, device=ctx.dev)
    pos = torch.arange(w.n, dtype=torch.int32, device=ctx.dev)[None]
    kout = torch.empty((1, w.heads, w.n, 128), dtype=torch.bfloat16, device=ctx.dev)
    vout = torch.empty_like(kout)

    def enc_plain_all():
        kv.pq_encode(kd, cbk, 8, codes=kc)

    def enc_blend():
        kv.pq_encode(kd, cbk, 8, query=proxy[:, None], beta=w.betas[0], idx=ret, codes=kc)

    def enc_h():
        kv.pq_encode(kd, cbk, 8, chol=lq, idx=ret, codes=kc)

    def enc_values():
        kv.pq_encode(vd, cbv, 8, codes=vc)

    def rec_keys():
        kv.pq_reconstruct(kc[None], pos, cbk, w.cur_pos, w.window, out=kout)

    def rec_values():
        kv.pq_reconstruct(vc[None], pos, cbv, w.cur_pos, 0, far_mode=kv.FAR_UNROTATED, out=vout)

    def step():  # split, keys (bulk plain + retrieval blend), values, both reconstructions
        r, b = kv.select_retrieval(kd, proxy, w.fraction)
        kv.pq_encode(kd, cbk, 8, idx=b, codes=kc)
        kv.pq_encode(kd, cbk, 8, query=proxy[:, None], beta=w.betas[0], idx=r, codes=kc)
        enc_values()
        rec_keys()
        rec_values()

    for f in (enc_plain_all, enc_blend, enc_h, enc_values, rec_keys, rec_values, step):
        f()
    torch.cuda.synchronize()
    t_plain = ctx.timed(enc_plain_all, 10)
    t_blend = ctx.timed(enc_blend, 5)
    t_h = ctx.timed(enc_h, 10)
    t_rk = ctx.timed(rec_keys, 10)
    t_rv = ctx.timed(rec_values, 10)
    t_step = ctx.timed(step, 5)
    subvecs = w.heads * w.n * 16
    flops_plain = 2.0 * subvecs * w.c * 8  # the sub-vector contraction, 2 k sub_dim per sub-vector
    acc = kv.pq_accounting(w.n, w.heads, 128, 8, 8)
    res["pq_layer"] = {
        "workload": "8 heads x 32768 bf16 keys and values, sub_dim 8, one 256-entry codebook, "
                    "retrieval fraction 0.2 (beta 0.5 blend or H-weighted), bf16 W=128 keys, "
                    "values unrotated",
        "step_ms": round(t_step, 4), "keys_per_s": round(w.heads * w.n / (t_step * 1e-3), 1),
        "encode_plain_all_us": round(t_plain * 1e3, 2),
        # the matrix cores score 4.2M sub-vectors x 256 centroids; the argmax fold and the
        # per-sub-vector finalisation on the vector ALU set the time
        "encode_plain_subvecs_per_s": round(subvecs / (t_plain * 1e-3), 1),
        "encode_plain_mfma_frac": round(flops_plain / (t_plain * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
        "encode_blend_retrieval_us": round(t_blend * 1e3, 2),
        "encode_h_retrieval_us": round(t_h * 1e3, 2),
        "reconstruct_keys_us": round(t_rk * 1e3, 2),
        "reconstruct_keys_hbm_frac": round(w.heads * w.n * (16 + 256) / (t_rk * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "reconstruct_values_us": round(t_rv * 1e3, 2),
        "accounting": acc,
    }
    log("pq_layer %s" % res["pq_layer"])
    # Codebook training (Lloyd rounds on the device, H-weighted assignment): whole-vector
    # codebooks of the layer workload (8 x 32768 bf16 keys, k = 1024), and the pages' shared
    # sub-vector codebook (k = 256, sub_dim 8) over the same keys pooled as 4.2M sub-vectors.
    wl = W["layer"]
    kl = ctx.keys_dev(synth.keys(wl.cfg, wl.heads, wl.n, "bf16"))
    _, ll = kv.calibrate(ctx.f32(synth.queries(wl.cfg, wl.heads, wl.m)), 1e-4)
    cb_init = kl[:, ::wl.n // wl.c][:, :wl.c].float().contiguous()
    cbw = cb_init.clone()
    sub_x = kd.reshape(-1, 8)
    cbs_init = sub_x[:: sub_x.shape[0] // 256][:256].float().contiguous()
    cbs = cbs_init.clone()

    def train_whole():
        cbw.copy_(cb_init)
        kv.kmeans(kl, cbw, ll, iters=5)

    def train_sub():
        cbs.copy_(cbs_init)
        kv.kmeans(sub_x, cbs, lq, iters=5)

    train_whole()
    train_sub()
    torch.cuda.synchronize()
    t_w = ctx.timed(train_whole, 3)
    t_s = ctx.timed(train_sub, 3)
    pr_w = ctx.profile(train_whole, 1)
    # k-means++ seeding in z-space (the initial codebooks of the same two trainings)
    rd_w = torch.from_numpy(np.random.default_rng(7).integers(0, 2 ** 64, (wl.heads, wl.c), dtype=np.uint64).view(np.int64)).to(ctx.dev)
    rd_s = torch.from_numpy(np.random.default_rng(8).integers(0, 2 ** 64, 256, dtype=np.uint64).view(np.int64)).to(ctx.dev)

    def seed_whole():
        kv.kmeans_init(kl, wl.c, rd_w, ll)

    def seed_sub():
        kv.kmeans_init(sub_x, 256, rd_s, lq)

    seed_whole()
    seed_sub()
    torch.cuda.synchronize()
    t_iw = ctx.timed(seed_whole, 2)
    t_is = ctx.timed(seed_sub, 2)
    res["kmeans"] = {
        "workload": "5 Lloyd rounds + final assignment, H-weighted: 8 heads x 32768 bf16 keys with "
                    "k=1024 per head; 4.2M pooled sub-vectors (sub_dim 8) with one k=256 codebook; "
                    "k-means++ seeding in z-space of the same two",
        "whole_ms_per_round": round(t_w / 6, 4),
        "sub_ms_per_round": round(t_s / 6, 4),
        "whole_update_us": round(sum(v[1] for kk, v in pr_w.items() if kk.startswith("kmeans_")) * 1e3, 2),
        "seed_whole_ms": round(t_iw, 3),
        "seed_sub_ms": round(t_is, 3),
    }
    log("kmeans %s" % res["kmeans"])
    return res




# ---------------------------------------------------------------------------- counter probes
def probe_encode_stress(ctx):
    e = EncodeStress(ctx)
    for _ in range(3):
        e.step()
    ctx.torch.cuda.synchronize()


def probe_long_context(ctx):
    """The long-context split and bf16 reconstruct, three calls each."""
    torch, kv, synth, dev = ctx.torch, ctx.kv, ctx.synth, ctx.dev
    w = synth.WORKLOADS["long_context"]
    kd = ctx.keys_dev(synth.keys(w.cfg, w.heads, w.n, "bf16"))
    cbd = ctx.f32(synth.codebook(w.cfg, w.heads, w.c))
    codes = torch.from_numpy(synth.uniform_codes(w.cfg, (1, w.heads, w.n), w.c).view(np.int16)).to(dev).view(torch.uint16)
    pos = torch.arange(w.n, dtype=torch.int32, device=dev)[None]
    out = torch.empty((1, w.heads, w.n, D), dtype=torch.bfloat16, device=dev)
    proxy = kd[:, -1].contiguous()
    for _ in range(3):
        kv.select_retrieval(kd, proxy, w.fraction)
    for _ in range(3):
        kv.reconstruct(codes, pos, cbd, w.cur_pos, w.window, out=out)
    torch.cuda.synchronize()


def probe_decode(ctx):
    """The decode workload's fp32 reconstruct (32 x 8 x 16384 tokens), three calls."""
    torch, kv, synth, dev = ctx.torch, ctx.kv, ctx.synth, ctx.dev
    w = synth.WORKLOADS["decode"]
    cbd = ctx.f32(synth.codebook(w.cfg, w.heads, w.c))
    codes = torch.from_numpy(synth.uniform_codes(w.cfg, (w.batch, w.heads, w.n), w.c).view(np.int16)).to(dev).view(torch.uint16)
    pos = torch.arange(w.n, dtype=torch.int32, device=dev)[None].repeat(w.batch, 1).contiguous()
    out = torch.empty((w.batch, w.heads, w.n, D), dtype=torch.float32, device=dev)
    for _ in range(3):
        kv.reconstruct(codes, pos, cbd, w.cur_pos, w.window, out=out)
    torch.cuda.synchronize()


PROBES = {"encode_stress": probe_encode_stress, "long_context": probe_long_context,
          "decode": probe_decode}


def _algorithmic():
    """Per kernel and workload: (kernel-name pattern, what it is, algorithmic bytes per launch,
    algorithmic flops per launch or None, source file).  Bytes count what the method must move:
    encode, keys (bf16) + codes + distances + the fp16 codebook fragments and bias of every
    head once; split, keys + one index per key; reconstruct, codes + positions + output + the
    codebook of every head once."""
    enc = 8 * 131072 * (D * 2 + 2 + 4) + 8 * 4096 * (D * 2 + 4)
    split = 8 * 131072 * (D * 2 + 4)
    rec_lc = 8 * 131072 * (2 + D * 2) + 131072 * 4 + 8 * 2048 * D * 4
    rec_dec = 32 * 8 * 16384 * (2 + D * 4) + 32 * 16384 * 4 + 8 * 1024 * D * 4
    return {
        ("encode_stress", "enc_coarse"): ("the MFMA pass of the H-weighted encode with distances",
                                          enc, 2.0 * 8 * 131072 * 4096 * D, "kv_cache_vector_windowed_amd/csrc/encode.hip"),
        ("long_context", "sel_"): ("the four kernels of the retrieval split, per call", split, None,
                                   "kv_cache_vector_windowed_amd/csrc/select.hip"),
        ("long_context", "rope_gather"): ("the bf16 reconstruct gather", rec_lc, None,
                                          "kv_cache_vector_windowed_amd/csrc/reconstruct.hip"),
        ("decode", "rope_gather"): ("the fp32 reconstruct gather", rec_dec, None,
                                    "kv_cache_vector_windowed_amd/csrc/reconstruct.hip"),
    }


def _pmc_dispatches(d):
    """[(kernel name, dispatch id, {counter: value summed over instances})] of one pass."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % d)
    disp = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                k = (f, r["Dispatch_Id"])
                name, vals = disp.setdefault(k, (r["Kernel_Name"], {}))
                vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [(name, k[1], vals) for k, (name, vals) in sorted(disp.items(), key=lambda kv_: int(kv_[0][1]))]


def _median(v):
    v = sorted(v)
    return v[len(v) // 2] if v else None


def pmc_summarize(root, command):
    """Every pass under root/<workload>_<pass>/: per kernel of interest, the median per launch
    of every counter; HBM bytes = FETCH_SIZE and WRITE_SIZE (KiB) scaled by what the same
    counter reads for the reference copy (reads and writes COPY_REF_BYTES)."""
    alg = _algorithmic()
    passes = sorted(p for p in os.listdir(root) if os.path.isdir(os.path.join(root, p)))
    by_wl = {}
    for p in passes:
        wl, _, tag = p.rpartition("_")
        by_wl.setdefault(wl, []).append((tag, os.path.join(root, p)))
    written = []
    absroot = os.path.abspath(root)
    for (wl, pat), (what, abytes, aflops, src) in alg.items():
        if wl not in by_wl:
            continue
        if command:
            cmd = command
        else:
            # one rocprofv3 pass per counter group, as recorded in each pass's own output
            lines = ["cd /tmp && export TMPDIR=/tmp"]
            for tag, d in by_wl[wl]:
                names = []
                for n, _, v in _pmc_dispatches(d):
                    names += [cn for cn in v if cn not in names]
                lines.append("timeout -s KILL 90 rocprofv3 --pmc %s --output-format csv -d %s -o p "
                             "-- python3 %s --pmc-probe %s"
                             % (" ".join(names), os.path.join(absroot, os.path.basename(d)),
                                os.path.join(ROOT, "bench.py"), wl))
            lines.append("python3 %s --pmc-summarize %s" % (os.path.join(ROOT, "bench.py"), absroot))
            cmd = "\n".join(lines)
        counters, scales = {}, {}
        for tag, d in by_wl[wl]:
            rows = _pmc_dispatches(d)
            ref = [v for n, _, v in rows if "neg" in n.lower()]
            # one launch = all dispatches of the pattern between two calls: the split is four
            # kernels, summed per call (calls follow each other, three of them)
            mine = [(n, v) for n, _, v in rows if pat in n]
            if not mine:
                continue
            per_call = {}
            if pat == "sel_":
                names = []
                for n, _ in mine:
                    if n not in names:
                        names.append(n)
                calls = len(mine) // len(names)
                for c in range(calls):
                    chunk = mine[c * len(names):(c + 1) * len(names)]
                    for n, v in chunk:
                        for cn, cv in v.items():
                            per_call.setdefault(cn, [0.0] * calls)[c] += cv
            else:
                for n, v in mine:
                    for cn, cv in v.items():
                        per_call.setdefault(cn, []).append(cv)
            for cn, vals in per_call.items():
                counters[cn] = _median(vals)
                if cn in ("FETCH_SIZE", "WRITE_SIZE") and ref:
                    rv = _median([r[cn] for r in ref if cn in r])
                    if rv:
                        scales[cn] = (COPY_REF_BYTES / 1024.0) / rv
        if not counters:
            continue
        out = {"kernel": pat, "workload": wl, "what": what, "source": src,
               "source_sha": sha_of(os.path.join(ROOT, src)), "counters_per_launch": counters,
               "reference_scale": scales, "algorithmic_bytes_per_launch": abytes,
               "algorithmic_flops_per_launch": aflops, "command": cmd}
        hbm = 0.0
        have = True
        for cn in ("FETCH_SIZE", "WRITE_SIZE"):
            if cn in counters and cn in scales:
                b = counters[cn] * 1024.0 * scales[cn]
                out[cn.lower() + "_bytes"] = round(b)
                hbm += b
            else:
                have = False
        out["hbm_bytes_per_launch"] = round(hbm) if have else None
        if have:
            out["hbm_over_algorithmic"] = round(hbm / abytes, 4)
        if "SQ_INSTS_MFMA" in counters and aflops:
            # v_mfma_f32_32x32x16_f16: 32 x 32 x 16 multiply-adds per wave instruction
            out["mfma_insts_algorithmic"] = aflops / (2 * 32 * 32 * 16)
            out["mfma_insts_over_algorithmic"] = round(counters["SQ_INSTS_MFMA"] / out["mfma_insts_algorithmic"], 4)
        name = "%s_%s_pmc" % (pat.strip("_") if pat != "sel_" else "select", wl)
        base = os.path.join(ROOT, "profiles", name)
        with open(base + ".json", "w") as f:
            json.dump(out, f, indent=1)
        with open(base + ".md", "w") as f:
            f.write("# %s, %s workload: counters per launch\n\n%s.\n\n" % (pat, wl, what))
            f.write("Command (rocprofv3 --pmc passes, one counter group each, then the summary):\n\n"
                    "```\n%s\n```\n\n" % cmd)
            f.write("| counter | median per launch |\n|---|---|\n")
            for cn in sorted(counters):
                f.write("| %s | %.6g |\n" % (cn, counters[cn]))
            if scales:
                f.write("\nReference copy (%d MiB read + %d MiB written): scale per counter %s.\n"
                        % (COPY_REF_BYTES >> 20, COPY_REF_BYTES >> 20,
                           ", ".join("%s %.4f" % kv_ for kv_ in scales.items())))
            if out["hbm_bytes_per_launch"]:
                f.write("\nHBM bytes per launch %.6g (fetch %.6g, write %.6g) against %.6g "
                        "algorithmic: %.3f x.\n" % (out["hbm_bytes_per_launch"], out["fetch_size_bytes"],
                                                   out["write_size_bytes"], abytes,
                                                   out["hbm_over_algorithmic"]))
            if "mfma_insts_over_algorithmic" in out:
                f.write("\nMFMA instructions %.6g against %.6g for the algorithmic 2NCd flop: %.4f x.\n"
                        % (counters["SQ_INSTS_MFMA"], out["mfma_insts_algorithmic"],
                           out["mfma_insts_over_algorithmic"]))
            f.write("\nSource %s @ %s.\n" % (src, out["source_sha"]))
        written.append(base + ".json")
    print(json.dumps({"written": written}))


def trace_summarize(root, command, name="encode_stress"):
    """Kernel statistics of a rocprofv3 --kernel-trace --stats run, read from the rocpd
    database it writes: calls, mean / median / min / max duration and registers per kernel, into
    profiles/<name>_trace.md."""
    import sqlite3

    dbs = glob.glob(os.path.join(root, "**", "*.db"), recursive=True)
    if not dbs:
        raise SystemExit("no rocpd database under %s" % root)
    con = sqlite3.connect(dbs[0])
    rows = con.execute(
        "select name, count(*), avg(duration), min(duration), max(duration), sum(duration), "
        "max(vgpr_count), max(accum_vgpr_count), max(sgpr_count), max(lds_size), "
        "max(grid_x), max(workgroup_x) from kernels group by name").fetchall()
    total = sum(r[5] for r in rows)
    rows.sort(key=lambda r: -r[5])
    med = {}
    for nm, dur in con.execute("select name, duration from kernels"):
        med.setdefault(nm, []).append(dur)
    for nm in med:
        d = sorted(med[nm])
        med[nm] = d[len(d) // 2] if len(d) % 2 else 0.5 * (d[len(d) // 2 - 1] + d[len(d) // 2])

    def short(name):
        for pre in ("void ", "a2ats::(anonymous namespace)::"):
            name = name.replace(pre, "")
        if name.startswith("_ZN5a2ats12_GLOBAL__N_1"):  # mangled: keep the kernel's own name
            rest = name[len("_ZN5a2ats12_GLOBAL__N_1"):]
            k = 0
            while k < len(rest) and rest[k].isdigit():
                k += 1
            ln = int(rest[:k])
            tmpl = rest[k + ln:]
            name = rest[k:k + ln] + ("<" + tmpl[1:tmpl.index("EE") + 1] + ">" if tmpl.startswith("I") else "")
        return name.split("(")[0][:80]

    if not command:
        # the profiled program's command line is in the database; the profiler's own options
        # are those of every trace summarized here
        prog = con.execute("select command from rocpd_info_process").fetchone()
        if not prog or not prog[0]:
            raise SystemExit("the database records no command: pass --command")
        absroot = os.path.abspath(root)
        prefix = os.path.basename(dbs[0])[:-len("_results.db")]
        command = ("cd /tmp && export TMPDIR=/tmp\n"
                   "timeout -k 10 300 rocprofv3 --kernel-trace --stats -d %s -o %s -- %s\n"
                   "python3 %s --trace-summarize %s --trace-name %s"
                   % (absroot, prefix, prog[0], os.path.join(ROOT, "bench.py"), absroot, name))
    path = os.path.join(ROOT, "profiles", "%s_trace.md" % name)
    with open(path, "w") as f:
        f.write("# %s: kernel trace statistics\n\n"
                "Command:\n\n```\n%s\n```\n\n" % (name, command))
        f.write("| kernel | calls | average us | median us | min us | max us | share % | VGPR | AGPR | SGPR | LDS B | grid | block |\n"
                "|---|---|---|---|---|---|---|---|---|---|---|---|---|\n")
        for r in rows:
            f.write("| %s | %d | %.2f | %.2f | %.2f | %.2f | %.2f | %s | %s | %s | %s | %s | %s |\n" % (
                short(r[0]), r[1], r[2] / 1e3, med[r[0]] / 1e3, r[3] / 1e3, r[4] / 1e3,
                100.0 * r[5] / total, r[6], r[7], r[8], r[9], r[10], r[11]))
    print(json.dumps({"written": path}))


def traffic_from_profiles(kernel, workload):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was taken on
    the current kernel source (else None)."""
    p = os.path.join(ROOT, "profiles", "%s_%s_pmc.json" % (kernel, workload))
    if not os.path.exists(p):
        return None
    try:
        with open(p) as f:
            d = json.load(f)
        if sha_of(os.path.join(ROOT, d["source"])) != d["source_sha"]:
            return None
        return d["hbm_bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(synth):
    """The oracle (as it stands) on a bounded sample of the headline workload: the H-weighted
    assignment with distances of the first rows of every head (fp64, z-space form), as many
    1024-row blocks per head as fit in about 15 s."""
    import oracle

    w = synth.WORKLOADS["encode_stress"]
    log("cpu baseline (oracle)")
    rows = 32768
    keys = synth.keys(w.cfg, w.heads, rows, "bf16")  # the first rows of every head
    cb = synth.codebook(w.cfg, w.heads, w.c)
    q = synth.queries(w.cfg, w.heads, w.m)
    _, L = oracle.calibrate(q, 1e-4)
    done = 0
    t0 = time.perf_counter()
    blk = 0
    while blk * 1024 < rows:
        for h in range(w.heads):
            oracle.assign_h(keys.values[h, blk * 1024:(blk + 1) * 1024], cb[h], L[h])
            done += 1024
        blk += 1
        if time.perf_counter() - t0 > 15.0:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done / dt, 1), "unit": "keys/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": "%d keys (the first %d rows of each of the 8 heads) of the encode_stress "
                      "workload: H-weighted assignment with distances against C=4096, fp64; "
                      "%.1f s" % (done, done // w.heads, dt)}


if __name__ == "__main__":
    main()
