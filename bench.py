"""Benchmark of the Token Radius Attention (TRA) hot path on one MI355X.

One step = the whole hot path over one batch of synthetic activations already
resident in HBM:
    tile-major permute of q, k, v
    dense warm-up attention with fused per-query entropy (all N keys)
    entropy -> budget -> radius -> block-sparse mask
    the order the sparse workgroups take the rows in (computed once per mask, like it)
    block-sparse attention over that mask (the reused-mask call of later steps)
    unpermute of the output
Every stage is timed with HIP events on the stream the kernels run on.  The
headline value is the effective throughput of the block-sparse attention:
4 * D FLOPs per retained (query, key) token pair (real tokens only) divided by its
average call time.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ms/call + effective TFLOP/s (% bf16 MFMA peak), TRA block-sparse attn at Wan-14B"
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", type=int, default=3)
    p.add_argument("--tau", type=float, default=None)
    p.add_argument("--density", type=float, default=None,
                   help="use the oracle-calibrated tau for this retained density (0.09, 0.15, 0.19 at workload 3)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--headline-only", action="store_true",
                   help="only the timed steps: no extra calls after them (so a profiler's per-kernel statistics cover "
                        "the steps' kernels alone)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB (3 times), to calibrate HBM counters")
    return p.parse_args()


def profiled_traffic(workload: str, kernel_source: str):
    """HBM bytes per launch of the sparse attention kernel from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE scaled by a plain copy's readings), or None when the
    summary was taken on another workload or on a different kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "attn_sparse_hbm_traffic.md")
    try:
        with open(kernel_source, "rb") as fh:
            sha = hashlib.sha256(fh.read()).hexdigest()
        with open(path) as fh:
            for line in fh:
                if line.startswith("traffic:"):
                    f = dict(kv.split("=", 1) for kv in line[len("traffic:"):].split())
                    if f.get("workload") == workload and f.get("attention_hip_sha256") == sha:
                        return int(f["bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        pass
    return None


def copy_calibration(mib: int) -> None:
    """A plain copy kernel of known size: its FETCH_SIZE / WRITE_SIZE counters per dispatch
    should read mib MiB each; the ratio scales the counters of the TRA kernels."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_mib": mib, "bytes_read": n * 4, "bytes_written": n * 4}), flush=True)


def retained_pairs(torch, cnt, idx, N, bq, bk):
    """Exact number of retained (query, key) token pairs, ragged blocks counted by their real size."""
    outer, nqb = cnt.shape
    nkb = idx.shape[2]
    qsize = torch.full((nqb,), bq, dtype=torch.float64, device=cnt.device)
    qsize[-1] = N - (nqb - 1) * bq
    ksz_last = N - (nkb - 1) * bk
    c = cnt.to(torch.int64)
    last = torch.gather(idx, 2, (c - 1).clamp(min=0).unsqueeze(2)).squeeze(2)
    has_last = (c > 0) & (last == nkb - 1)
    keys = c.to(torch.float64) * bk - has_last.to(torch.float64) * (bk - ksz_last)
    return float((keys * qsize[None, :]).sum().item())


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(wl, q, k, v, mask_rows, blocks, head, budget_s, perm, sparse_flops, mask_s):
    """The oracle's masked attention on seeded q-blocks of one head, timed on the host cores, with
    the time one whole sparse call (sparse_flops) and one whole mask call would take at the
    measured rates (mask_s: the oracle's brute-force mask of the same q-blocks)."""
    import numpy as np
    import oracle

    threads = oracle.default_threads()
    qp, kp, vp = (oracle.permute(x[head].float().numpy().astype(np.float64), perm) for x in (q, k, v))
    full = np.zeros((wl.nqb, wl.nkb), dtype=np.uint8)
    full[blocks] = mask_rows
    done_rows, done_pairs, elapsed, passes = 0, 0.0, 0.0, 0
    ksz = np.array([min(wl.N, (kb + 1) * wl.block_k) - kb * wl.block_k for kb in range(wl.nkb)])
    while elapsed < budget_s:  # whole passes over the sampled q-blocks until the budget is spent
        for b in blocks:
            rows = np.arange(b * wl.block_q, min(wl.N, b * wl.block_q + wl.block_q), dtype=np.int32)
            t0 = time.perf_counter()
            oracle.attention(qp, kp, vp, wl.sm_scale, rows=rows, block_mask=full, bq=wl.block_q, bk=wl.block_k,
                             nthreads=threads)
            elapsed += time.perf_counter() - t0
            done_rows += len(rows)
            done_pairs += float(len(rows) * (ksz * full[b]).sum())
        passes += 1
    flops = 4.0 * wl.D * done_pairs
    rate = flops / elapsed
    return {
        "value": rate / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "fp64 masked attention of %d seeded q-blocks of head %d (N=%d keys, each q-block's retained "
                  "k-blocks from the oracle's mask) x %d passes: %d query rows, %.3g retained pairs, %.1f s"
                  % (len(blocks), head, wl.N, passes, done_rows, done_pairs, elapsed),
        "cpu": cpu_model(),
        "extrapolated_ms_per_call": round(1e3 * sparse_flops / rate, 1),
        "mask": {"ms_per_qblock": round(1e3 * mask_s / len(blocks), 3),
                 "extrapolated_ms_per_call": round(1e3 * mask_s / len(blocks) * wl.outer * wl.nqb, 1),
                 "sample": "the oracle's brute-force mask rows (every query against every key) of the same %d "
                           "q-blocks, scaled to %d heads x %d q-blocks" % (len(blocks), wl.outer, wl.nqb)},
    }


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus %d requested). "
              "Sharding by (batch, head) needs no exchange inside TRA; see the design notes." % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import entropy_adaptive_sparse_amd as tra
    from entropy_adaptive_sparse_amd import synth, workloads

    tra.load()
    dev = torch.device("cuda:0")
    wl = workloads.get(args.workload)
    tau = wl.tau if args.tau is None else args.tau
    if args.density is not None:
        if args.density not in workloads.DENSITY_TAU.get(wl.wid, {}):
            sys.exit("no calibrated tau for density %g at workload %d (have %s)"
                     % (args.density, wl.wid, sorted(workloads.DENSITY_TAU.get(wl.wid, {}))))
        tau = workloads.DENSITY_TAU[wl.wid][args.density]
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32

    t0 = time.time()
    qn, kn, vn = synth.qkv(wl.wid, wl.outer, wl.F, wl.H, wl.W, wl.D, wl.t_lo, wl.t_hi)
    q, k, v = (torch.from_numpy(x).to(dt) for x in (qn, kn, vn))
    del qn, kn, vn
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    print("# inputs ready in %.1f s: %s outer=%d N=%d D=%d" % (time.time() - t0, wl.name, wl.outer, wl.N, wl.D),
          file=sys.stderr, flush=True)

    qp, kp, vp = (torch.empty_like(qd) for _ in range(3))
    od = torch.empty_like(qd)
    osp = torch.empty_like(qd)
    onat = torch.empty_like(qd)
    ent = torch.empty((wl.outer, wl.N), dtype=torch.float32, device=dev)
    cnt = torch.empty((wl.outer, wl.nqb), dtype=torch.int32, device=dev)
    idx = torch.empty((wl.outer, wl.nqb, wl.nkb), dtype=torch.int32, device=dev)
    order = torch.empty((wl.outer * wl.nqb,), dtype=torch.int32, device=dev)
    tra.mask_prepare(wl.F, wl.H, wl.W, tau, wl.gamma, wl.block_q, wl.block_k)
    if wl.W % 4 == 0 and wl.tile_w % 4 == 0:
        tra.natural_prepare(wl.F, wl.H, wl.W, wl.tile_h, wl.tile_w)
    # static radial-style mask: head h's queries all take the entropy c_h (the warm-up pass still runs)
    ent_mask = ent
    if wl.static_mask:
        ent_mask = torch.tensor(wl.static_entropy, dtype=torch.float32, device=dev).view(wl.outer, 1).expand(
            wl.outer, wl.N).contiguous()
    stages = ["permute_qkv", "dense_entropy", "build_mask", "schedule", "sparse_attn", "unpermute"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        for src, dst in ((qd, qp), (kd, kp), (vd, vp)):
            tra.tile_major_permute(src, wl.F, wl.H, wl.W, out=dst)
        mark(1)
        tra.dense_attn_entropy(qp, kp, vp, wl.sm_scale, entropy=True, out=od, ent_out=ent)
        mark(2)
        tra.build_block_mask(ent_mask, wl.F, wl.H, wl.W, tau, wl.gamma, wl.block_q, wl.block_k, wl.vote_threshold,
                             kv_count=cnt, kv_index=idx)
        mark(3)
        tra.sparse_schedule(cnt, wl.F, wl.H, wl.W, wl.block_q, wl.block_k, wl.tile_h, wl.tile_w, out=order)
        mark(4)
        tra.block_sparse_attn_scheduled(qp, kp, vp, cnt, idx, order, wl.block_q, wl.block_k, wl.sm_scale, out=osp)
        mark(5)
        tra.tile_major_unpermute(osp, wl.F, wl.H, wl.W, out=onat)
        mark(6)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("# warmup done", file=sys.stderr, flush=True)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    per_stage = {name: [] for name in stages}
    for s in range(args.steps):
        for i, name in enumerate(stages):
            per_stage[name].append(evs[s][i].elapsed_time(evs[s][i + 1]))
    ms = {name: float(np.mean(v)) for name, v in per_stage.items()}
    ms_step = wall * 1e3 / args.steps

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        fn()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    reps = max(3, args.steps)
    ms_dense_plain = ms_reuse_b2b = ms_sparse_b2b = ms_sparse_default = ms_sparse_cold = ms_copy = None
    ms_fused = ms_reuse_nat = ms_dense_nat = ms_fused_nat = None
    if not args.headline_only:
        # the library's dense path without the entropy: the speed-up reference (outside the steps)
        tra.dense_attn_entropy(qp, kp, vp, wl.sm_scale, entropy=False, out=od)
        e0.record()
        for _ in range(2):
            tra.dense_attn_entropy(qp, kp, vp, wl.sm_scale, entropy=False, out=od)
        e1.record()
        torch.cuda.synchronize()
        ms_dense_plain = e0.elapsed_time(e1) / 2
        # later denoising steps reuse the mask and its schedule: reuse steps back to back (permute, sparse,
        # unpermute), the sparse call alone back to back, and the sparse call in the default order
        def reuse_step():
            for src, dst in ((qd, qp), (kd, kp), (vd, vp)):
                tra.tile_major_permute(src, wl.F, wl.H, wl.W, out=dst)
            tra.block_sparse_attn_scheduled(qp, kp, vp, cnt, idx, order, wl.block_q, wl.block_k, wl.sm_scale, out=osp)
            tra.tile_major_unpermute(osp, wl.F, wl.H, wl.W, out=onat)
        reps = max(3, args.steps)
        ms_reuse_b2b = timed(reuse_step, reps)
        ms_sparse_b2b = timed(lambda: tra.block_sparse_attn_scheduled(qp, kp, vp, cnt, idx, order, wl.block_q,
                                                                      wl.block_k, wl.sm_scale, out=osp), reps)
        ms_sparse_default = timed(lambda: tra.block_sparse_attn(qp, kp, vp, cnt, idx, wl.block_q, wl.block_k,
                                                                wl.sm_scale, out=osp), reps)
        # cold variant of the sparse call: 512 MB written between calls (the last-level cache is 256 MB)
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cold = []
        for _ in range(3):
            scratch.fill_(1)
            e0.record()
            tra.block_sparse_attn_scheduled(qp, kp, vp, cnt, idx, order, wl.block_q, wl.block_k, wl.sm_scale, out=osp)
            e1.record()
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        del scratch
        ms_sparse_cold = float(np.mean(cold))
        # the runtime's own device-to-device copy of one q-sized tensor: the reference the
        # permutations are compared with beside the HBM peak
        ms_copy = timed(lambda: osp.copy_(qp), reps)
        # the warm-up pass with the mask builder fused in (same outputs as dense_entropy + build_mask)
        ms_fused = None
        if wl.dtype == "bf16" and wl.D == 128 and wl.block_q == 128 and not wl.static_mask:
            def fused():
                tra.dense_attn_entropy_mask(qp, kp, vp, wl.F, wl.H, wl.W, tau, wl.gamma, wl.sm_scale, wl.block_q,
                                            wl.block_k, wl.vote_threshold, out=od, ent_out=ent, kv_count=cnt,
                                            kv_index=idx)
            fused()
            e0.record()
            for _ in range(2):
                fused()
            e1.record()
            torch.cuda.synchronize()
            ms_fused = e0.elapsed_time(e1) / 2

        # the permutation folded into the attention kernels (natural-order q, k, v, o): a reuse step
        # is then one call, a warm-up one dense call plus the mask
        ms_reuse_nat = ms_dense_nat = ms_fused_nat = None
        if wl.dtype == "bf16" and wl.D == 128 and wl.block_q == 128 and wl.W % 4 == 0 and wl.tile_w % 4 == 0:
            def sparse_nat():
                tra.block_sparse_attn_natural(qd, kd, vd, cnt, idx, wl.F, wl.H, wl.W, wl.block_q, wl.block_k,
                                              wl.sm_scale, tile_h=wl.tile_h, tile_w=wl.tile_w, out=onat)

            def dense_nat():
                tra.dense_attn_entropy_natural(qd, kd, vd, wl.F, wl.H, wl.W, wl.sm_scale, entropy=True, out=onat,
                                               ent_out=ent, tile_h=wl.tile_h, tile_w=wl.tile_w)
            for fn in (sparse_nat, dense_nat):
                fn()
            reps = max(2, args.steps)
            e0.record()
            for _ in range(reps):
                sparse_nat()
            e1.record()
            torch.cuda.synchronize()
            ms_reuse_nat = e0.elapsed_time(e1) / reps
            e0.record()
            for _ in range(2):
                dense_nat()
            e1.record()
            torch.cuda.synchronize()
            ms_dense_nat = e0.elapsed_time(e1) / 2
            if not wl.static_mask:
                def fused_nat():
                    tra.dense_attn_entropy_mask_natural(qd, kd, vd, wl.F, wl.H, wl.W, tau, wl.gamma, wl.sm_scale,
                                                        wl.block_q, wl.block_k, wl.vote_threshold, wl.tile_h, wl.tile_w,
                                                        out=onat, ent_out=ent, kv_count=cnt, kv_index=idx)
                fused_nat()
                e0.record()
                for _ in range(2):
                    fused_nat()
                e1.record()
                torch.cuda.synchronize()
                ms_fused_nat = e0.elapsed_time(e1) / 2
    pairs = retained_pairs(torch, cnt, idx, wl.N, wl.block_q, wl.block_k)
    density = pairs / (wl.outer * float(wl.N) ** 2)

    # fp8 queries and keys (OCP E4M3, rounded once from the bf16 values, outside the timing) with bf16
    # values: the sparse call over the same mask and schedule
    fp8 = None
    if wl.dtype == "bf16" and wl.D == 128 and wl.block_q == 128 and not args.headline_only:
        q8 = qp.to(torch.float8_e4m3fn)
        k8 = kp.to(torch.float8_e4m3fn)
        ms_fp8 = timed(lambda: tra.block_sparse_attn_fp8(q8, k8, vp, cnt, idx, wl.block_q, wl.block_k, wl.sm_scale,
                                                         out=osp, order=order), reps)
        del q8, k8
        tf8 = 4.0 * wl.D * pairs / (ms_fp8 * 1e-3) / 1e12
        # half the work (q.k) at the fp8 rate, half (p.v) at the bf16 rate
        blended = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
        fp8 = {"ms": round(ms_fp8, 4), "achieved": round(tf8, 2), "unit": "TFLOP/s", "peak_blended": round(blended, 1),
               "frac_blended": round(tf8 / blended, 4), "frac_bf16_peak": round(tf8 / PEAK_BF16_TFLOPS, 4),
               "speedup_vs_bf16": round(ms_sparse_b2b / ms_fp8, 3),
               "note": "q, k fp8 E4M3 (scores on the fp8 matrix cores), v, o bf16; same mask and schedule; "
                       "back to back, as the bf16 ms_sparse_back_to_back"}

    # the 1D-distance variant of the mask (the ablation of the radius mask), from the same warm-up
    # entropies and tau, and the sparse call over its lists
    mask1d = None
    if not wl.static_mask and not args.headline_only:
        cnt1 = torch.empty_like(cnt)
        idx1 = torch.empty_like(idx)
        tra.mask_prepare_1d(wl.F, wl.H, wl.W, tau, wl.block_q, wl.block_k, wl.tile_h, wl.tile_w)
        ms_m1 = timed(lambda: tra.build_block_mask_1d(ent, wl.F, wl.H, wl.W, tau, wl.block_q, wl.block_k,
                                                      wl.vote_threshold, wl.tile_h, wl.tile_w, kv_count=cnt1,
                                                      kv_index=idx1), reps)
        order1 = tra.sparse_schedule(cnt1, wl.F, wl.H, wl.W, wl.block_q, wl.block_k, wl.tile_h, wl.tile_w)
        ms_s1 = timed(lambda: tra.block_sparse_attn_scheduled(qp, kp, vp, cnt1, idx1, order1, wl.block_q, wl.block_k,
                                                              wl.sm_scale, out=osp), reps)
        pairs1 = retained_pairs(torch, cnt1, idx1, wl.N, wl.block_q, wl.block_k)
        mask1d = {"ms_mask": round(ms_m1, 4), "density": round(pairs1 / (wl.outer * float(wl.N) ** 2), 5),
                  "ms_sparse": round(ms_s1, 4),
                  "sparse_tflops": round(4.0 * wl.D * pairs1 / (ms_s1 * 1e-3) / 1e12, 2),
                  "note": "same tau and entropies as the disk mask; sparse call back to back with its own schedule"}
        del cnt1, idx1, order1
    sparse_flops = 4.0 * wl.D * pairs
    dense_flops = wl.dense_flops
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    sparse_tf = sparse_flops / (ms["sparse_attn"] * 1e-3) / 1e12
    dense_tf = dense_flops / (ms["dense_entropy"] * 1e-3) / 1e12
    elem = 2 if wl.dtype == "bf16" else 4
    tensor_bytes = wl.outer * wl.N * wl.D * elem
    perm_gbs = 3 * 2 * tensor_bytes / (ms["permute_qkv"] * 1e-3) / 1e9
    unperm_gbs = 2 * tensor_bytes / (ms["unpermute"] * 1e-3) / 1e9
    copy_gbs = None if ms_copy is None else 2 * tensor_bytes / (ms_copy * 1e-3) / 1e9
    nnz = int(cnt.to(torch.int64).sum().item())
    mask_bytes = 4 * wl.outer * wl.N + 4 * nnz + 4 * wl.outer * wl.nqb
    mask_gbs = mask_bytes / (ms["build_mask"] * 1e-3) / 1e9

    def r4(x):
        return None if x is None else round(x, 4)

    result = {
        "metric": METRIC,
        "value": round(sparse_tf, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded q/k/v with 3D sinusoidal positions and log-uniform query temperatures)",
        "config": {
            "workload": wl.name, "batch": wl.batch, "heads": wl.heads, "N": wl.N, "D": wl.D,
            "grid": [wl.F, wl.H, wl.W], "block_q": wl.block_q, "block_k": wl.block_k, "tau": tau,
            "gamma": wl.gamma, "vote_threshold": wl.vote_threshold, "tile": [wl.tile_h, wl.tile_w],
            "retained_density": round(density, 5), "static_mask": wl.static_mask,
        },
        "ms_per_call": {k2: round(v2, 4) for k2, v2 in ms.items()},
        "ms_dense_no_entropy": r4(ms_dense_plain),
        "ms_sparse_cold": r4(ms_sparse_cold),
        "ms_warmup_separate": round(ms["dense_entropy"] + ms["build_mask"], 4),
        "ms_warmup_fused": None if ms_fused is None else round(ms_fused, 4),
        "ms_reuse_step": round(ms["permute_qkv"] + ms["sparse_attn"] + ms["unpermute"], 4),
        "ms_reuse_step_back_to_back": r4(ms_reuse_b2b),
        "ms_sparse_back_to_back": r4(ms_sparse_b2b),
        "ms_sparse_default_order": r4(ms_sparse_default),
        "ms_reuse_step_natural": None if ms_reuse_nat is None else round(ms_reuse_nat, 4),
        "ms_dense_entropy_natural": None if ms_dense_nat is None else round(ms_dense_nat, 4),
        "ms_warmup_fused_natural": None if ms_fused_nat is None else round(ms_fused_nat, 4),
        "roofline": {
            "bound": "mfma", "achieved": round(sparse_tf, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(sparse_tf / peak, 4),
            "traffic": profiled_traffic(wl.name, os.path.join(ROOT, "entropy_adaptive_sparse_amd", "csrc",
                                                              "attention.hip")),
            "kernel": "attn_bf16_kernel (sparse)" if wl.dtype == "bf16" else "attn_f32_kernel (sparse)",
            "flops_per_launch": sparse_flops,
        },
        "rooflines": {
            "dense_entropy": {"bound": "mfma", "achieved": round(dense_tf, 2), "peak": peak, "unit": "TFLOP/s",
                              "frac": round(dense_tf / peak, 4), "flops_per_launch": dense_flops},
            "permute_qkv": {"bound": "hbm", "achieved": round(perm_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(perm_gbs / PEAK_HBM_GBS, 4), "bytes": 6 * tensor_bytes,
                            "vs_device_copy": None if copy_gbs is None else round(perm_gbs / copy_gbs, 3)},
            "unpermute": {"bound": "hbm", "achieved": round(unperm_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": round(unperm_gbs / PEAK_HBM_GBS, 4), "bytes": 2 * tensor_bytes,
                          "vs_device_copy": None if copy_gbs is None else round(unperm_gbs / copy_gbs, 3)},
            "device_copy": None if copy_gbs is None else {
                "achieved": round(copy_gbs, 1), "unit": "GB/s", "bytes": 2 * tensor_bytes,
                "note": "the runtime's device-to-device copy of one q-sized tensor, back to back"},
            "build_mask": {"bound": "alu", "achieved_hbm": round(mask_gbs, 2), "unit": "GB/s", "bytes": mask_bytes,
                           "pct_of_sparse_time": round(100.0 * ms["build_mask"] / ms["sparse_attn"], 2)},
        },
        "fp8_sparse": fp8,
        "mask_1d": mask1d,
        "speedup_sparse_vs_dense": None if ms_dense_plain is None else round(ms_dense_plain / ms["sparse_attn"], 3),
        "speedup_target": round(0.6 / density, 3) if density > 0 else None,
    }

    if not args.no_cpu:
        import oracle
        oracle.build(force=False)
        perm = oracle.tile_major_order(wl.F, wl.H, wl.W)
        head = 0
        blocks = synth.uniform_ints(7, 64, 0, wl.nqb)
        ent_h = synth.entropy_like(900 + wl.wid, 1, wl.N)[0]
        t0 = time.perf_counter()
        mask_rows, _ = oracle.block_mask(ent_h, wl.F, wl.H, wl.W, tau, wl.gamma, wl.block_q, wl.block_k,
                                         wl.vote_threshold, qblocks=blocks)
        mask_s = time.perf_counter() - t0
        print("# cpu baseline ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, q, k, v, mask_rows, blocks, head, args.cpu_seconds, perm,
                                              sparse_flops, mask_s)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
