#!/usr/bin/env python3
"""Benchmark of the A2ATS key-cache hot path on one MI355X.

Headline: the per-layer cache update of a Llama-3.2-3B-shaped layer (8 KV heads x 32768
tokens x d=128, bf16 keys, C=1024 centroids per head, H from 4096 queries, W=512, retrieval
fraction 0.1).  One step = retrieval split (with the codebook side of both encodes on a
second stream) -> plain encode of the bulk rows and, on the second stream, H-weighted encode
of the retrieval rows (every key gets exactly its pipeline code) -> windowed-RoPE
reconstruct (bf16) of the whole cache.  Calibration
(H and L) is the pages' one-time offline job: it runs once before timing and is reported
separately.  `value` = keys encoded per second.

Also reported (field "extra"): the large-codebook H-weighted encode (8 x 131072 keys,
C=4096, codes + distances) with its MFMA fraction; the decode step (32 x 8 x 16384 tokens,
fp32 reconstruct + cosine-blend of the new keys) and the long-context pipeline (8 x 131072
keys, 5% split, C=2048, W=1024) with HBM fractions.

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
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
PEAK_FP64_TFLOPS = 78.6        # MI355X fp64 vector (an FMA counted as two operations)
METRIC = "keys encoded/sec (H-weighted VQ, d=128) + % MFMA peak; reconstruct GB/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sha_of(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="run 3 layer steps and a 256 MiB reference copy, for rocprofv3 --pmc")
    ap.add_argument("--pmc-summarize", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc outputs (FETCH_SIZE, WRITE_SIZE) of "
                         "--pmc-probe into profiles/encode_coarse_plain_layer_pmc.{json,md}")
    args = ap.parse_args()
    if args.pmc_summarize:
        pmc_summarize(*args.pmc_summarize)
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
    W = synth.WORKLOADS

    def keys_dev(k):
        return torch.from_numpy(k.bits.view(np.int16)).to(dev).view(torch.bfloat16)

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

    # ------------------------------------------------------------------ headline workload
    w = W["layer"]
    log("generating layer inputs")
    keys = synth.keys(w.cfg, w.heads, w.n, "bf16")
    kd = keys_dev(keys)
    cbd = f32(synth.codebook(w.cfg, w.heads, w.c))
    qd = f32(synth.queries(w.cfg, w.heads, w.m))
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
    main_s = torch.cuda.current_stream(dev)
    prep_plain = kv.encode_prepare(cbd, None, w.n)
    prep_h = kv.encode_prepare(cbd, L, w.n)

    def step():
        main_s = torch.cuda.current_stream(dev)  # the capturing stream inside a graph capture
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

    if args.pmc_probe:
        for _ in range(2):
            step()
        torch.cuda.synchronize()
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        src = torch.ones(COPY_REF_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)  # reads and writes COPY_REF_BYTES: the counter scale
        torch.cuda.synchronize()
        print(json.dumps({"pmc_probe": "done", "copy_ref_bytes": COPY_REF_BYTES}), flush=True)
        return

    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("timing %d steps" % args.steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_eager = e0.elapsed_time(e1) / args.steps
    log("layer step, launched one by one: %.4f ms" % ms_eager)
    # The same step captured once in a HIP graph (the launches of both streams, replayed as
    # one): the timed steps are K replays.  A replay must reproduce the eager step's codes
    # and keys bit for bit.
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
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    keys_per_step = w.heads * w.n
    value = keys_per_step / (ms * 1e-3)
    log("layer step %.4f ms (graph replay) -> %.4g keys/s" % (ms, value))

    # per-kernel durations: same step, same launches, with HIP events around every kernel
    def profile(fn, reps):
        kv.profile_reset()
        kv.profile_enable(True)
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        prof = kv.profile_read()
        kv.profile_enable(False)
        kv.profile_reset()
        return {k: (c, t / c) for k, (c, t) in prof.items()}

    def step_seq():  # the same launches on one stream: per-kernel times without overlap
        prep_plain.prepare(cbd, None)
        prep_h.prepare(cbd, L)
        ret, bulk = kv.select_retrieval(kd, proxy, w.fraction)
        kv.encode_prepared(kd, prep_h, idx=ret, codes=codes)
        kv.encode_prepared(kd, prep_plain, idx=bulk, codes=codes)
        kv.reconstruct(codes[None], pos, cbd, w.cur_pos, w.window, out=out)

    prof = profile(step_seq, min(args.steps, 20))
    log("kernels: " + ", ".join("%s %.1fus" % (k, v[1] * 1e3) for k, v in prof.items()))
    coarse_ms = prof["encode_coarse_plain"][1]
    n_bulk = w.n - kv.retrieval_count(w.n, w.fraction)  # rows of the plain pass
    flops = 2.0 * w.heads * n_bulk * w.c * 128
    achieved = flops / (coarse_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": "encode_coarse_plain", "achieved": round(achieved, 2),
                "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_TFLOPS, 4),
                "traffic": traffic_from_profiles("encode_coarse_plain", "layer"),
                "launch_us": round(coarse_ms * 1e3, 2), "flops_per_launch": flops}
    t0 = time.perf_counter()
    kv.calibrate(qd, 1e-4)
    calib_ms = (time.perf_counter() - t0) * 1e3

    extra = {"layer_step_ms_eager": round(ms_eager, 5),
             "layer_kernels_us": {k: round(v[1] * 1e3, 2) for k, v in prof.items()},
             "layer_calibrate_ms_host_clock": round(calib_ms, 3)}
    if not args.no_extra:
        extra.update(extra_workloads(torch, kv, synth, dev, keys_dev, f32, profile))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, keys, synth)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "keys/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "layer: 8 KV heads x 32768 tokens x d=128 bf16 keys, C=1024, "
                               "H from 4096 queries, W=512, retrieval fraction 0.1; step = split + "
                               "plain encode of bulk rows || H-weighted encode of retrieval rows + "
                               "bf16 reconstruct",
                   "heads": w.heads, "tokens": w.n, "centroids": w.c, "window": w.window,
                   "fraction": w.fraction},
        "roofline": roofline, "cpu_baseline": cpu, "extra": extra,
    }
    print(json.dumps(line), flush=True)


COPY_REF_BYTES = 256 * 2 ** 20
COARSE_SOURCE = "kv_cache_vector_windowed_amd/csrc/encode.hip"


def _pmc_rows(d, counter):
    """{dispatch id: (kernel name, grid size, value summed over instances)} for one counter."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % d)
    out = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                k = (f, r["Dispatch_Id"])
                name, grid, v = out.get(k, (r["Kernel_Name"], int(r["Grid_Size"]), 0.0))
                out[k] = (name, grid, v + float(r["Counter_Value"]))
    return out


def pmc_summarize(fetch_dir, write_dir):
    """HBM bytes per launch of the plain coarse encode pass on the layer workload: FETCH_SIZE
    and WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads for a
    reference elementwise kernel that reads and writes COPY_REF_BYTES."""
    # the plain pass of the layer step encodes the bulk rows: 32768 - ceil(0.1 * 32768) a head
    n_bulk = 32768 - 3277
    layer_grid = (8 * ((n_bulk + 255) // 256) + 7) // 8 * 8 * 256  # workgroups x 256 threads
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _pmc_rows(d, counter)
        coarse = sorted(v for n, g, v in rows.values() if "enc_coarse" in n and "Lb0ELb0E" in n
                        and g == layer_grid)
        ref = sorted(v for n, g, v in rows.values() if "neg" in n)
        if not coarse or not ref:
            raise SystemExit("%s: missing dispatches (coarse %d, reference %d)" % (counter, len(coarse), len(ref)))
        kib = coarse[len(coarse) // 2]
        ref_kib = ref[len(ref) // 2]
        scale = (COPY_REF_BYTES / 1024.0) / ref_kib
        res[counter] = {"kib_per_dispatch": kib, "reference_kib": ref_kib, "scale": scale,
                        "bytes": kib * 1024.0 * scale}
    total = res["FETCH_SIZE"]["bytes"] + res["WRITE_SIZE"]["bytes"]
    # bf16 keys, fp16 codebook fragments, fp32 bias, int32 row indices, uint16 codes
    algorithmic = 8 * n_bulk * (128 * 2 + 4 + 2) + 8 * 1024 * (128 * 2 + 4)
    cmd = ["cd /tmp && export TMPDIR=/tmp",
           "rocprofv3 --pmc FETCH_SIZE --output-format csv -d %s -o p -- "
           "python <repo>/bench.py --pmc-probe" % fetch_dir,
           "rocprofv3 --pmc WRITE_SIZE --output-format csv -d %s -o p -- "
           "python <repo>/bench.py --pmc-probe" % write_dir,
           "python bench.py --pmc-summarize %s %s" % (fetch_dir, write_dir)]
    d = {"kernel": "encode_coarse_plain", "workload": "layer", "source": COARSE_SOURCE,
         "source_sha": sha_of(os.path.join(ROOT, COARSE_SOURCE)),
         "hbm_bytes_per_launch": round(total), "algorithmic_bytes_per_launch": algorithmic,
         "counters": res, "commands": cmd}
    base = os.path.join(ROOT, "profiles", "encode_coarse_plain_layer_pmc")
    with open(base + ".json", "w") as f:
        json.dump(d, f, indent=1)
    with open(base + ".md", "w") as f:
        f.write("# encode_coarse_plain, layer workload: HBM traffic per launch\n\n")
        f.write("Commands:\n\n```\n%s\n```\n\n" % "\n".join(cmd))
        f.write("| counter | KiB / dispatch | reference KiB (%d MiB read + write) | scale | bytes |\n"
                "|---|---|---|---|---|\n" % (COPY_REF_BYTES >> 20))
        for k, v in res.items():
            f.write("| %s | %.0f | %.0f | %.4f | %.4g |\n" % (k, v["kib_per_dispatch"], v["reference_kib"],
                                                         v["scale"], v["bytes"]))
        f.write("\nTotal %.4g bytes per launch; algorithmic %.4g (bulk keys, fp16 codebook, bias, "
                "row indices, codes); "
                "source %s @ %s\n" % (total, algorithmic, COARSE_SOURCE, d["source_sha"]))
    print(json.dumps(d))


def traffic_from_profiles(kernel, workload):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was taken on
    the current kernel source (else None)."""
    p = os.path.join(ROOT, "profiles", "%s_%s_pmc.json" % (kernel, workload))
    if not os.path.exists(p):
        return None
    try:
        with open(p) as f:
            d = json.load(f)
        src = os.path.join(ROOT, d["source"])
        if sha_of(src) != d["source_sha"]:
            return None
        return d["hbm_bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def extra_workloads(torch, kv, synth, dev, keys_dev, f32, profile):
    W = synth.WORKLOADS
    res = {}
    flush_buf = torch.ones(2 ** 28, dtype=torch.float32, device=dev)  # 1 GiB, finite values
    flush_buf.sum()  # the first reduction launch carries a one-time setup cost of ~20 ms
    torch.cuda.synchronize()

    def timed(fn, reps, flush=False):
        """ms per call of fn, calls issued back to back on the stream so the host's issue time
        overlaps the GPU's work.  With flush, a read of a 1 GiB buffer (which evicts the
        256 MB last-level cache with clean lines) precedes every call, and the same number of
        reads timed alone is subtracted.  A kernel that follows a large streaming kernel runs
        measurably slower than in a back-to-back steady state on this GPU (the gap does not
        come from cache contents: it appears after a read of 256 MB as after a write of the
        kernel's own output), so both figures are reported."""
        def run(with_fn):
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                if flush:
                    flush_buf.sum()
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

    # large-codebook encode
    w = W["encode_stress"]
    log("generating encode_stress inputs")
    kd = keys_dev(synth.keys(w.cfg, w.heads, w.n, "bf16"))
    cbd = f32(synth.codebook(w.cfg, w.heads, w.c))
    _, L = kv.calibrate(f32(synth.queries(w.cfg, w.heads, w.m)), 1e-4)
    stats = torch.zeros(8, dtype=torch.int32, device=dev)

    def enc():
        kv.encode(kd, cbd, L, want_dist=True, stats=stats)

    enc()
    torch.cuda.synchronize()
    ms = timed(enc, 5)
    pr = profile(enc, 3)
    flops = 2.0 * w.heads * w.n * w.c * 128
    cms = pr["encode_coarse_h"][1]
    st = stats.cpu().numpy().tolist()
    res["encode_stress"] = {
        "workload": "8 heads x 131072 bf16 keys, C=4096, H-weighted, codes + distances",
        "ms_per_call": round(ms, 4), "keys_per_s": round(w.heads * w.n / (ms * 1e-3), 1),
        "mfma_frac_call": round(flops / (ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
        "coarse_us": round(cms * 1e3, 2),
        "mfma_frac_coarse": round(flops / (cms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
        "kernels_us": {k: round(v[1] * 1e3, 2) for k, v in pr.items()},
        "decided": {"direct": st[1], "reranked": st[2], "rescanned": st[3], "full_scan": st[4]},
    }
    log("encode_stress %s" % res["encode_stress"])
    del kd
    # decode step
    w = W["decode"]
    log("generating decode inputs")
    cbd = f32(synth.codebook(w.cfg, w.heads, w.c))
    codes = torch.from_numpy(synth.uniform_codes(w.cfg, (w.batch, w.heads, w.n), w.c).view(np.int16)).to(dev).view(torch.uint16)
    pos = torch.arange(w.n, dtype=torch.int32, device=dev)[None].repeat(w.batch, 1).contiguous()
    out = torch.empty((w.batch, w.heads, w.n, 128), dtype=torch.float32, device=dev)
    newk = f32(synth.new_keys(w.cfg, w.heads, w.batch))

    def rec():
        kv.reconstruct(codes, pos, cbd, w.cur_pos, w.window, out=out)

    def blend():
        kv.assign_cosine(newk, newk, cbd, w.betas[0])

    rec()
    blend()
    torch.cuda.synchronize()
    ms_r = timed(rec, 5, flush=True)
    ms_r_steady = timed(rec, 10)
    ms_b = timed(blend, 10)
    tokens = w.batch * w.heads * w.n
    alg = tokens * (2 + 128 * 4) + w.batch * w.n * 4 + w.heads * w.c * 128 * 4
    pr = profile(rec, 3)
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
    qd = torch.randn((w.batch, qh, 128), dtype=torch.float32, device=dev)
    qo = torch.empty_like(qd)

    def qrope():
        kv.far_query_rope(qd, 2048, out=qo)

    upd()
    torch.cuda.synchronize()
    ms_u = timed(upd, 20)
    ms_fu = timed(full_unrot, 5)
    ms_q = timed(qrope, 20)
    pr_u = profile(upd, 5)
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
        synth.queries(wt.cfg, wt.q_heads, wt.batch).transpose(1, 0, 2))).to(dev)
    qtb = torch.empty_like(qt)
    t_idx = torch.empty((wt.batch, wt.q_heads, kt), dtype=torch.int32, device=dev)

    def topk_step():
        kv.far_query_rope(qt, wt.far_b, out=qtb)
        kv.topk_codes(qtb, codes, cbd, kt)

    topk_step()
    torch.cuda.synchronize()
    ms_t = timed(topk_step, 20)
    ms_tf = timed(topk_step, 5, flush=True)
    pr_t = profile(topk_step, 5)
    kt_us = pr_t["topk_codes"][1] * 1e3
    t_bytes = (wt.batch * wt.heads * wt.n * 2 + wt.heads * wt.c * 128 * 4
               + wt.batch * wt.q_heads * (128 * 4 + kt * 8))
    t_flops = 2.0 * wt.batch * wt.q_heads * wt.c * 128  # fp64 table: one mul + one add a term
    res["topk_decode"] = {
        "workload": "32 sequences x 24 query heads over 8 key heads x 16384 codes, C=1024, "
                    "k=%d (10%%); far query rotation + table + top-K" % kt,
        "step_us": round(ms_t * 1e3, 2), "step_flushed_us": round(ms_tf * 1e3, 2),
        "topk_kernel_us": round(kt_us, 2),
        "far_query_rope_us": round(pr_t["far_query_rope"][1] * 1e3, 2),
        "algorithmic_bytes": t_bytes, "kernel_GBps": round(t_bytes / (kt_us * 1e-6) / 1e9, 1),
        "table_fp64_ops": t_flops,
        "table_fp64_frac": round(t_flops / (kt_us * 1e-6) / 1e12 / (PEAK_FP64_TFLOPS / 2), 4),
    }
    log("topk_decode %s" % res["topk_decode"])
    # long-context pipeline
    w = W["long_context"]
    log("generating long_context inputs")
    kd = keys_dev(synth.keys(w.cfg, w.heads, w.n, "bf16"))
    cbd = f32(synth.codebook(w.cfg, w.heads, w.c))
    _, L = kv.calibrate(f32(synth.queries(w.cfg, w.heads, w.m)), 1e-4)
    proxy = kd[:, -1].contiguous()
    codes = torch.zeros((w.heads, w.n), dtype=torch.uint16, device=dev)
    pos = torch.arange(w.n, dtype=torch.int32, device=dev)[None]
    out = torch.empty((1, w.heads, w.n, 128), dtype=torch.bfloat16, device=dev)

    def split():
        return kv.select_retrieval(kd, proxy, w.fraction)

    def rec2():
        kv.reconstruct(codes[None], pos, cbd, w.cur_pos, w.window, out=out)

    aux = torch.cuda.Stream(device=dev)
    main_s = torch.cuda.current_stream(dev)
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
    ms_s = timed(split, 10, flush=True)
    ms_r = timed(rec2, 10, flush=True)
    ms_s_steady = timed(split, 20)
    ms_r_steady = timed(rec2, 20)
    ms_p = timed(pipe, 5)
    split_bytes = w.heads * w.n * (128 * 2 + 4)
    rec_bytes = w.heads * w.n * (2 + 128 * 2) + w.n * 4 + w.heads * w.c * 128 * 4
    pr_s = profile(split, 5)
    pr_r = profile(rec2, 5)
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
        "pipeline_kernels_us": {k: round(v[1] * 1e3, 2) for k, v in profile(pipe, 3).items()},
    }
    log("long_context %s" % res["long_context"])
    del kd, codes, out
    # The pages' default configuration: sub-vector codes (sub_dim 8, one shared 256-entry
    # codebook), keys of the layer shape: split, plain codes for the bulk rows, cosine-blend
    # (beta 0.5; no H) or H-weighted codes for the retrieval rows; values plain; bf16 keys
    # reconstructed with W = 128, values gathered without rotation.
    w = W["pq_layer"]
    log("generating pq_layer inputs")
    kd = keys_dev(synth.keys(w.cfg, w.heads, w.n, "bf16"))
    vd = keys_dev(synth.keys(w.cfg, w.heads, w.n, "bf16", stream=8))  # value rows
    cbk = f32(synth.pq_codebook(w.cfg, w.heads, w.c, 8))
    cbv = f32(synth.pq_codebook(w.cfg + 100, w.heads, w.c, 8))
    qs = synth.queries(w.cfg, w.heads, w.m)
    _, lq = kv.calibrate(f32(qs.reshape(1, -1, 8)), 1e-4)
    lq = lq[0].contiguous()
    proxy = kd[:, -1].contiguous()
    ret, bulk = kv.select_retrieval(kd, proxy, w.fraction)
    kc = torch.zeros((w.heads, w.n, 16), dtype=torch.uint8, device=dev)
    vc = torch.zeros((w.heads, w.n, 16), dtype=torch.uint8, device=dev)
    pos = torch.arange(w.n, dtype=torch.int32, device=dev)[None]
    kout = torch.empty((1, w.heads, w.n, 128), dtype=torch.bfloat16, device=dev)
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
    t_plain = timed(enc_plain_all, 10)
    t_blend = timed(enc_blend, 5)
    t_h = timed(enc_h, 10)
    t_rk = timed(rec_keys, 10)
    t_rv = timed(rec_values, 10)
    t_step = timed(step, 5)
    subvecs = w.heads * w.n * 16
    flops_plain = 2.0 * subvecs * w.c * 8  # the sub-vector contraction, 2 k sub_dim per sub-vector
    acc = kv.pq_accounting(w.n, w.heads, 128, 8, 8)
    res["pq_layer"] = {
        "workload": "8 heads x 32768 bf16 keys and values, sub_dim 8, one 256-entry codebook, "
                    "retrieval fraction 0.2 (beta 0.5 blend or H-weighted), bf16 W=128 keys, "
                    "values unrotated",
        "step_ms": round(t_step, 4), "keys_per_s": round(w.heads * w.n / (t_step * 1e-3), 1),
        "encode_plain_all_us": round(t_plain * 1e3, 2),
        "encode_plain_alu_frac": round(flops_plain / (t_plain * 1e-3) / 1e12 / PEAK_FP32_VALU_TFLOPS, 4),
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
    kl = keys_dev(synth.keys(wl.cfg, wl.heads, wl.n, "bf16"))
    _, ll = kv.calibrate(f32(synth.queries(wl.cfg, wl.heads, wl.m)), 1e-4)
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
    t_w = timed(train_whole, 3)
    t_s = timed(train_sub, 3)
    pr_w = profile(train_whole, 1)
    res["kmeans"] = {
        "workload": "5 Lloyd rounds + final assignment, H-weighted: 8 heads x 32768 bf16 keys with "
                    "k=1024 per head; 4.2M pooled sub-vectors (sub_dim 8) with one k=256 codebook",
        "whole_ms_per_round": round(t_w / 6, 4),
        "sub_ms_per_round": round(t_s / 6, 4),
        "whole_update_us": round(sum(v[1] for kk, v in pr_w.items() if kk.startswith("kmeans_")) * 1e3, 2),
    }
    log("kmeans %s" % res["kmeans"])
    return res


def cpu_baseline(w, keys, synth):
    """The oracle (as it stands) on a bounded sample of the headline step: whole heads of the
    layer workload, each running split, plain encode of the bulk rows, H-weighted encode of
    the retrieval rows and the fp64 reconstruct; as many heads as fit in about 15 s."""
    import oracle

    log("cpu baseline (oracle)")
    cb = synth.codebook(w.cfg, w.heads, w.c)
    q = synth.queries(w.cfg, w.heads, w.m)
    _, L = oracle.calibrate(q, 1e-4)
    done = 0
    t0 = time.perf_counter()
    for h in range(w.heads):
        x = keys.values[h]
        ret, bulk, _ = oracle.select_retrieval(x, x[-1], w.fraction)
        code = np.zeros(w.n, dtype=np.int32)
        code[bulk], _, _ = oracle.assign_h(x[bulk], cb[h], None)
        code[ret], _, _ = oracle.assign_h(x[ret], cb[h], L[h])
        oracle.reconstruct(code.astype(np.uint16), np.arange(w.n, dtype=np.int32), cb[h],
                           w.cur_pos, w.window)
        done += 1
        if time.perf_counter() - t0 > 15.0:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done * w.n / dt, 1), "unit": "keys/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": "%d of %d heads of the layer step (%d keys each): split, plain encode of "
                      "bulk rows, H-weighted encode of retrieval rows, reconstruct; %.1f s"
                      % (done, w.heads, w.n, dt)}


if __name__ == "__main__":
    main()
