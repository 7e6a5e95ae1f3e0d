"""Benchmark of the draft-block verification step on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--config block16] [--no-extra] [--no-cpu] [--no-peaks]

A step is one call of the whole verification path (MLP, shared LM head over the target
and draft rows, statistics, acceptance, residual/bonus sampling, tau) on one batch of
synthetic inputs already resident in HBM.  Every point rotates R seeded input sets
(hidden rows, drafts, coins; the weights stay fixed) through its loops, so tau and the
accepted-token rate are averages over R draws rather than one draw.  Before the W warmup
steps each point runs its step untimed for --settle seconds (the GPU clock ramps up over
the first ~0.1-0.3 s of work); then exactly K steps are timed with events on the call's
stream.

The headline workload is the 16-token block (B=1, K=15, d=4096, d_ff=12288, V=151936,
T=1 sampled); `value` is verified positions per second (B*(K+1) target rows per step).
Rank 0 prints one JSON line.  Extra points (greedy at B=1; FP8 weights; the greedy batch
sweep at B=1, 8, 32, 128 with K=7; the confidence-scheduled step, literal and
budget-binding; the block as a candidate tree; the drafter step; commit; the wide model) are reported under
"extra", each with its own roofline.  The fp64 oracle is timed on the host cores for the
headline and for the B=128, scheduled and wide points (`cpu_baseline`), and gives the
closed-form expected tau of the sampled points' input sets beside the measured one.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "verified positions/sec + accepted tokens/sec @B=1,128; % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure
RIDGE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)  # FLOP per byte where the two bounds meet


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps before each timed loop (after --settle)")
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed steps before the warmup steps of each point (GPU clock ramp)")
    ap.add_argument("--config", default="block16", choices=["block16", "sweep", "sched", "sched_stress", "wide"])
    ap.add_argument("--batch", type=int, default=0, help="override B (sweep)")
    ap.add_argument("--sets", type=int, default=0, help="input sets rotated through the loops (0: 16 at B=1, else 8)")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--mode", default="", choices=["", "sample", "greedy", "scheduled"])
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy 1 GiB device-to-device once (a copy kernel of known size for counter scaling)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def t_quantile_975(n: int) -> float:
    """Two-sided 95% Student-t quantile for n-1 degrees of freedom (small table, normal beyond)."""
    table = {1: 12.706, 2: 4.303, 3: 3.182, 4: 2.776, 5: 2.571, 6: 2.447, 7: 2.365, 8: 2.306, 9: 2.262, 10: 2.228,
             11: 2.201, 12: 2.179, 13: 2.160, 14: 2.145, 15: 2.131, 16: 2.120, 20: 2.086, 30: 2.042}
    df = n - 1
    if df < 1:
        return float("nan")
    for k in sorted(table):
        if df <= k:
            return table[k]
    return 1.96


def roofline(bytes_, flops, ms, peaks_m, kernel):
    """Roofline of one launch of `ms` milliseconds moving `bytes_` and computing `flops`."""
    ai = flops / bytes_ if bytes_ else float("inf")
    if ai < RIDGE:
        r = {"bound": "hbm", "achieved": bytes_ / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        ach = peaks_m.get("hbm_read_GBps") if peaks_m else None
    else:
        r = {"bound": "mfma", "achieved": flops / (ms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
        ach = peaks_m.get("mfma_bf16_TFLOPs") if peaks_m else None
    r["frac"] = r["achieved"] / r["peak"]
    if ach:
        r["frac_of_measured_peak"] = r["achieved"] / ach
    r["kernel"] = kernel
    r["launch_ms"] = ms
    return r


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark measures one GPU (one process per GPU); --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    from draft_block_verification_spec_amd import binding as bd
    from draft_block_verification_spec_amd import workload as wl

    bd.load()  # fail loudly without the HIP library
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def to_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def to_i32(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev)

    def to_f32(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)

    peaks_m = None
    if not args.no_peaks:
        from draft_block_verification_spec_amd import peaks
        peaks_m = peaks.measure(dev)
        log(f"measured peaks: {peaks_m['hbm_read_GBps']:.0f} GB/s read, {peaks_m['mfma_bf16_TFLOPs']:.0f} TFLOP/s bf16")

    def n_sets(wk):
        return args.sets if args.sets else (16 if wk.B == 1 else 8)

    def input_sets(wk, data0, R):
        """Input set 0 is data0 (which also holds the weights); sets 1..R-1 are fresh draws of
        the activations, noise and coins with the next seeds (same weights)."""
        return [data0] + [wl.generate(wk, r, weights=False) for r in range(1, R)]

    def weights(datac, wkc):
        return bd.Weights(to_bf16(datac["w_lm"]), to_bf16(datac["w_gate"]) if wkc.d_ff else None,
                          to_bf16(datac["w_up"]) if wkc.d_ff else None, to_bf16(datac["w_down"]) if wkc.d_ff else None)

    def prepare(wkc, sets, modec, w):
        """Per input set: device inputs, drafts from the library's own drafter step, outputs;
        one workspace shared by the sets (the calls run in order on one stream)."""
        T = 0.0 if modec == "greedy" else wkc.T
        B, K = wkc.B, wkc.K
        mcode = {"greedy": bd.SV_MODE_GREEDY, "sample": bd.SV_MODE_SAMPLE, "scheduled": bd.SV_MODE_SCHEDULED}[modec]
        ws = bd.workspace(mcode, B, K, w, dev)
        calls, outs = [], []
        for datac in sets:
            h = to_bf16(datac["h"])
            hd = to_bf16(datac["h_draft"])
            u = to_f32(datac["coins"])
            draft, _ = bd.spec_draft_propose(w, hd, to_f32(datac["draft_coins"]), T)
            draft = draft.contiguous()
            out = bd.make_outputs(B, K, dev, mode=mcode, V=wkc.V, d=wkc.d)

            def call(h=h, hd=hd, u=u, draft=draft, out=out):
                if modec == "greedy":
                    bd.spec_verify_greedy(w, h, draft, out=out, ws=ws)
                elif modec == "sample":
                    bd.spec_verify_sample(w, h, hd, draft, u, T, out=out, ws=ws)
                else:
                    bd.spec_verify_scheduled(w, h, hd, draft, u, T, wkc.threshold, wkc.budget, out=out, ws=ws)
            calls.append(call)
            outs.append(out)
        return calls, outs

    def run_n(calls, n, start=0):
        for i in range(n):
            calls[(start + i) % len(calls)]()

    def timed(calls, outs, steps, warmup):
        """Settle, warm up, then time exactly `steps` steps rotating the input sets; then the
        same steps with events around the dominant GEMM, then with an event between steps."""
        R = len(calls)
        t0 = time.time()
        n = 0
        while time.time() - t0 < args.settle:
            run_n(calls, 16, n)
            n += 16
            torch.cuda.synchronize()
        run_n(calls, warmup, n)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run_n(calls, steps)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in evs:  # materialise the HIP events; the library re-records them around the GEMM
            a.record()
            b.record()
        torch.cuda.synchronize()
        for i in range(steps):
            outs[i % R].ev_lm = evs[i]
            calls[i % R]()
            outs[i % R].ev_lm = None
        torch.cuda.synchronize()
        lm_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        sev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        sev[0].record()
        for i in range(steps):
            calls[i % R]()
            sev[i + 1].record()
        torch.cuda.synchronize()
        per = np.array([sev[i].elapsed_time(sev[i + 1]) for i in range(steps)])
        spread = {"median": float(np.median(per)), "min": float(per.min()), "max": float(per.max())}
        return ms, lm_ms, spread

    def tau_stats(outs, steps, B):
        """Per input set: tau (mean of A+1 over its requests), emitted and accepted tokens;
        their averages over the timed steps (set i of step i % R); a 95% interval of the mean
        tau over the R sets.  A flagged request (device status) aborts the run."""
        R = len(outs)
        taus, emitted, accepted, verified = [], [], [], []
        for o in outs:
            st = int(o.dev_status.item())
            if st != 0:
                raise SystemExit(f"device status {st}")
            c = o.counters.cpu().numpy()
            accepted.append(float(c[0]))
            verified.append(float(c[1]))
            emitted.append(float(c[2]))
            taus.append(float(c[2]) / B)
        use = [i % R for i in range(steps)]
        em_step = float(np.mean([emitted[i] for i in use]))
        ac_step = float(np.mean([accepted[i] for i in use]))
        taus = np.array(taus)
        half = t_quantile_975(R) * taus.std(ddof=1) / math.sqrt(R) if R > 1 else float("nan")
        return {"tau": float(taus.mean()), "tau_ci95": [float(taus.mean() - half), float(taus.mean() + half)],
                "tau_sets": [round(float(t), 4) for t in taus], "input_sets": R,
                "emitted_per_step": em_step, "accepted_per_step": ac_step,
                "verified_per_step": float(np.mean([verified[i] for i in use]))}

    def point(wkc, modec, sets, w, label, fp8=False):
        calls, outs = prepare(wkc, sets, modec, w)
        ms, lm_ms, spread = timed(calls, outs, args.steps, args.warmup)
        ts = tau_stats(outs, args.steps, wkc.B)
        B, K, V, d, d_ff = wkc.B, wkc.K, wkc.V, wkc.d, wkc.d_ff
        if modec == "scheduled":
            vl = [o.verify_len.cpu().numpy() for o in outs]
            M_t = float(np.mean([int((v + 1).sum()) for v in (vl[i % len(vl)] for i in range(args.steps))]))
        else:
            M_t = B * (K + 1)
        pt = {"workload": label, "ms_per_step": ms, "step_ms_spread": spread,
              "positions_per_sec": M_t / (ms * 1e-3),
              "accepted_tokens_per_sec": ts["emitted_per_step"] / (ms * 1e-3),
              "accepted_drafts_per_sec": ts["accepted_per_step"] / (ms * 1e-3)}
        pt.update({k: ts[k] for k in ("tau", "tau_ci95", "tau_sets", "input_sets")})
        # the dominant GEMM (the library's events): LM head, or the draft-confidence pass
        if modec == "scheduled":
            rows = B * K
            kern = f"draft-confidence LM-head pass over {rows} rows"
        else:
            rows = B * (K + 1) + (B * K if modec == "sample" else 0)
            kern = f"LM-head GEMM over {rows} rows"
        # bf16 weights: 2 bytes each; FP8: 1 byte each plus an fp32 scale per output row
        lm_b = (1.0 * V * d + 4.0 * V if fp8 else 2.0 * V * d) + 2.0 * rows * d
        lm_f = 2.0 * rows * d * V
        pt["roofline"] = roofline(lm_b, lm_f, lm_ms, peaks_m, kern + (", FP8 weights" if fp8 else ""))
        # the whole step against its own bound
        step_b = float(wkc.weight_bytes()) / 2 + 4.0 * (V + 2 * d_ff + d) if fp8 else float(wkc.weight_bytes())
        step_f = 2.0 * M_t * 3 * d * d_ff + 2.0 * (M_t + (B * K if modec != "greedy" else 0)) * d * V
        pt["step_hbm_fraction"] = step_b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS
        pt["step_mfma_fraction"] = step_f / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS
        if modec == "scheduled":
            pt["verified_rows"] = M_t
        log(f"{label}: {ms:.4f} ms/step, tau {ts['tau']:.3f} [{ts['tau_ci95'][0]:.3f}, {ts['tau_ci95'][1]:.3f}], "
            f"{kern} {lm_ms:.3f} ms ({pt['roofline']['achieved']:.0f} {pt['roofline']['unit']})")
        del calls, outs
        return pt

    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- headline point
    wk = wl.PRESETS[args.config]
    if args.batch:
        wk = wk.with_batch(args.batch)
    mode = args.mode or {"block16": "sample", "sweep": "greedy", "sched": "scheduled",
                         "sched_stress": "scheduled", "wide": "sample"}[args.config]
    t0 = time.time()
    data = wl.generate(wk)
    sets = input_sets(wk, data, n_sets(wk))
    log(f"generated {wk.name} inputs ({len(sets)} sets) in {time.time() - t0:.1f}s")
    w_main = weights(data, wk)
    label = f"{wk.name}: B={wk.B} K={wk.K} d={wk.d} d_ff={wk.d_ff} V={wk.V} mode={mode}" + (
        f" T={wk.T}" if mode != "greedy" else "")
    head = point(wk, mode, sets, w_main, label)
    B, K, d, V, d_ff = wk.B, wk.K, wk.d, wk.V, wk.d_ff
    result = {
        "metric": METRIC, "value": head["positions_per_sec"], "unit": "positions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": f"synthetic (seeded normals, bf16 weights; no real model); {head['input_sets']} input sets rotated",
        "config": {"workload": label, "B": B, "K": K, "d": d, "d_ff": d_ff, "V": V, "mode": mode},
        "settle_s": args.settle,
        "accepted_tokens_per_sec": head["accepted_tokens_per_sec"],
        "accepted_drafts_per_sec": head["accepted_drafts_per_sec"],
        "tau": head["tau"], "tau_ci95": head["tau_ci95"], "tau_sets": head["tau_sets"],
        "input_sets": head["input_sets"], "step_ms_spread": head["step_ms_spread"],
        "step_hbm_fraction": head["step_hbm_fraction"], "roofline": head["roofline"],
    }
    result["roofline"]["traffic"] = traffic_for(args.config, mode)
    result["roofline"]["frac_kind"] = "dominant kernel (LM head); the whole step's fraction is step_hbm_fraction"
    if peaks_m:
        result["measured_peaks"] = peaks_m
    if mode == "scheduled":
        result["config"]["budget"] = wk.budget
        result["config"]["threshold"] = wk.threshold
        result["verified_rows"] = head["verified_rows"]

    cpu_jobs = [("headline", wk, sets, mode, result, data)]
    if not args.no_extra and args.config == "block16":
        extra = []
        extra.append(point(wk, "greedy", sets, w_main, "block16 greedy: B=1 K=15"))
        # FP8 (E4M3) weights with per-row fp32 scales, same block and input sets
        d8 = wl.to_fp8(data)
        w8 = bd.Weights(*(torch.from_numpy(np.ascontiguousarray(d8["q_" + n])).to(dev) for n in ("lm", "gate", "up", "down")),
                        *(to_f32(d8["s_" + n]) for n in ("lm", "gate", "up", "down")))
        del d8
        for m8 in ("sample", "greedy"):
            extra.append(point(wk, m8, sets, w8, f"block16 {m8}, FP8 E4M3 weights + fp32 row scales: B=1 K=15"
                               + (f" T={wk.T}" if m8 == "sample" else ""), fp8=True))
        del w8
        # the batch sweep (K = 7 greedy, same weight shapes): B = 1, 8, 32 HBM-bound, B = 128 MFMA-bound
        for Bs in (1, 8, 32, 128):
            wk2 = wl.SWEEP.with_batch(Bs)
            sets2 = [wl.generate(wk2, r, weights=False) for r in range(n_sets(wk2))]
            pt2 = point(wk2, "greedy", sets2, w_main, f"sweep greedy: B={Bs} K=7 (same shapes)")
            extra.append(pt2)
            if Bs == 128:
                cpu_jobs.append(("sweep B=128", wk2, sets2, "greedy", pt2, data))
        # the confidence-scheduled step: literal configuration and the budget-binding stress variant
        for wk3 in (wl.SCHED, wl.SCHED_STRESS):
            sets3 = [wl.generate(wk3, r, weights=False) for r in range(n_sets(wk3))]
            pt3 = point(wk3, "scheduled", sets3, w_main,
                        f"{wk3.name} scheduled: B={wk3.B} Kmax={wk3.K} budget={wk3.budget} "
                        f"threshold={wk3.threshold} T={wk3.T}")
            extra.append(pt3)
            if wk3.name == "sched":
                cpu_jobs.append(("sched", wk3, sets3, "scheduled", pt3, data))
        # the same block verified as a top-k tree of depth 3 (root: 4 candidates, each 2, then 1)
        for mt in ("sample", "greedy"):
            extra.append(bench_tree(bd, torch, wl, wk, sets, w_main, dev, to_bf16, to_i32, to_f32, mt, timed,
                                    tau_stats, args, peaks_m))
            log(f"block16 tree {mt}: {extra[-1]['ms_per_step']:.3f} ms/step, tau {extra[-1]['tau']:.2f}")
        # the drafter step that makes the block's drafts: 15 draft rows through the shared head
        for mp in ("sample", "greedy"):
            extra.append(bench_propose(bd, torch, wk, sets, w_main, dev, to_bf16, to_f32, mp, args.steps,
                                       args.warmup, peaks_m))
            log(f"drafter step {mp}: {extra[-1]['ms_per_call'] * 1e3:.1f} us/call")
        # commit after verification: the scheduled batch (B = 64, Kmax = 15) with tree-shaped
        # blocks on a hybrid target (8 attention layers x 2 KiB entries, 1 MiB recurrent state)
        extra.append(bench_commit(bd, torch, wl, dev, to_i32, args.steps, args.warmup, peaks_m))
        log(f"commit: {extra[-1]['ms_per_call'] * 1e3:.1f} us/call")
        # the wide model (d = 8192, d_ff = 28672, V = 128256), B = 32, K = 4, T = 0.7, sampled
        del w_main
        torch.cuda.empty_cache()
        wk4 = wl.WIDE
        d4 = wl.generate(wk4)
        sets4 = input_sets(wk4, d4, n_sets(wk4))
        w4 = weights(d4, wk4)
        pt4 = point(wk4, "sample", sets4, w4,
                    f"wide sample: B={wk4.B} K={wk4.K} d={wk4.d} d_ff={wk4.d_ff} V={wk4.V} T={wk4.T}")
        extra.append(pt4)
        cpu_jobs.append(("wide", wk4, sets4, "sample", pt4, d4))
        del w4
        result["extra"] = extra

    if not args.no_cpu:
        for name, wkc, setsc, modec, target, wdata in cpu_jobs:
            cb = cpu_baseline(wkc, setsc, modec, wdata)
            tcf = cb.pop("tau_closed_form", None)
            if target is result:
                result["cpu_baseline"] = cb
            else:
                target["cpu_baseline"] = cb
            if tcf is not None:
                target["tau_closed_form"] = tcf
            log(f"cpu baseline {name}: {cb['value']:.1f} {cb['unit']} on {cb['cores']} threads"
                + (f"; closed-form tau {tcf['tau']:.3f}" if tcf else ""))
    print(json.dumps(result), flush=True)


def bench_tree(bd, torch, wl, wk, sets, w, dev, to_bf16, to_i32, to_f32, mode, timed, tau_stats, args, peaks_m):
    """spec_verify_tree on the 16-token block shaped as a top-k tree.  Every child of a node
    is drawn from that node's draft distribution q_u with its own coin (sampled mode: the
    rule is lossless for children drawn independently from q_u); in greedy mode the first
    child of a node is q_u's argmax and its siblings are such draws."""
    B, K, V, d = wk.B, wk.K, wk.V, wk.d
    parent = wl.tree_parents(B, K, "topk")
    first = np.ones((B, K), bool)
    for b in range(B):
        seen = set()
        for j in range(K):
            first[b, j] = parent[b, j] not in seen
            seen.add(parent[b, j])
    T = 0.0 if mode == "greedy" else wk.T
    mcode = bd.SV_MODE_GREEDY if mode == "greedy" else bd.SV_MODE_SAMPLE
    ws = bd.workspace(mcode, B, K, w, dev)
    par = to_i32(parent)
    calls, outs = [], []
    for datac in sets:
        hd = to_bf16(datac["h_draft"])  # [B, K, d]: drafter row of node u is row u
        rows = hd[torch.arange(B, device=dev)[:, None], par.long()].reshape(B * K, d).contiguous()
        x_s, _ = bd.spec_draft_propose(w, rows, to_f32(datac["draft_coins"]).reshape(-1), wk.T)
        if mode == "greedy":
            x_g, _ = bd.spec_draft_propose(w, rows, None, 0.0)
            tokens = torch.where(torch.from_numpy(first.reshape(-1)).to(dev), x_g, x_s).view(B, K).contiguous()
        else:
            tokens = x_s.view(B, K).contiguous()
        h = to_bf16(datac["h"])
        u = to_f32(datac["coins"])
        out = bd.make_outputs(B, K, dev, mode=mcode, V=V, d=d)
        out.path = torch.empty(B, K + 1, dtype=torch.int32, device=dev)

        def call(h=h, hd=hd, tokens=tokens, u=u, out=out):
            bd.spec_verify_tree(w, h, hd, tokens, par, u, T, out=out, ws=ws)
        calls.append(call)
        outs.append(out)
    ms, lm, sp = timed(calls, outs, args.steps, args.warmup)
    ts = tau_stats(outs, args.steps, B)
    rows_lm = B * (K + 1) + (0 if mode == "greedy" else B * K)
    b_lm = 2.0 * V * d + 2.0 * rows_lm * d
    pt = {"workload": f"block16 tree {mode}: B={B}, {K + 1} nodes (top-k tree, depth 3)"
                      + ("" if mode == "greedy" else f", T={wk.T}, children drawn from q of their parent"),
          "ms_per_step": ms, "step_ms_spread": sp, "positions_per_sec": B * (K + 1) / (ms * 1e-3),
          "accepted_tokens_per_sec": ts["emitted_per_step"] / (ms * 1e-3)}
    pt.update({k: ts[k] for k in ("tau", "tau_ci95", "tau_sets", "input_sets")})
    pt["roofline"] = roofline(b_lm, 2.0 * rows_lm * d * V, lm, peaks_m, f"LM-head GEMM over {rows_lm} rows")
    return pt


def bench_propose(bd, torch, wk, sets, w, dev, to_bf16, to_f32, mode, steps, warmup, peaks_m):
    """spec_draft_propose on the block's K draft rows (the drafter step that makes the
    drafts): the shared LM head over K rows, then a draw from q at T (sampled) or the argmax
    (greedy).  Algorithmic bytes: W_lm once plus the K activation rows.  The input sets
    rotate through the calls; each call is timed with its own events."""
    K, V, d = wk.K, wk.V, wk.d
    rows = wk.B * K
    T = wk.T if mode == "sample" else 0.0
    ws = bd.workspace(bd.SV_MODE_PROPOSE, rows, 0, w, dev)
    xo = torch.empty(rows, dtype=torch.int32, device=dev)
    co = torch.empty(rows, dtype=torch.float32, device=dev)
    ins = [(to_bf16(dc["h_draft"]).reshape(rows, d).contiguous(),
            to_f32(dc["draft_coins"]).reshape(-1).contiguous() if T > 0 else None) for dc in sets]

    def call(i):
        hd, cn = ins[i % len(ins)]
        bd.spec_draft_propose(w, hd, cn, T, draft_out=xo, conf_out=co, ws=ws)
    t0 = time.time()
    n = 0
    while time.time() - t0 < 0.3:  # clock settle, as for the other points
        for _ in range(16):
            call(n)
            n += 1
        torch.cuda.synchronize()
    for i in range(warmup):
        call(i)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (e0, e1) in enumerate(evs):
        e0.record()
        call(i)
        e1.record()
    torch.cuda.synchronize()
    per = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
    ms = float(per.mean())
    by = 2.0 * V * d + 2.0 * rows * d
    return {"workload": f"drafter step ({mode}): {rows} draft rows of block16 through the shared LM head, "
                        f"V={V} d={d}" + (f" T={T}" if T > 0 else ""),
            "ms_per_call": ms, "call_ms_spread": {"median": float(np.median(per)), "min": float(per.min()),
                                                  "max": float(per.max())},
            "bytes_per_call": by,
            "roofline": roofline(by, 2.0 * rows * d * V, ms, peaks_m, "whole call (LM head over the draft rows + draw)")}


def bench_commit(bd, torch, wl, dev, to_i32, steps, warmup, peaks_m):
    """spec_commit on the commit workload; in place, so cache lengths are restored before
    each call (outside its events).  Algorithmic bytes: every committed request's state
    read from its snapshot and written, and every moved cache entry read and written."""
    cw = wl.COMMIT
    cc = wl.commit_case(cw, big=False)
    K1 = cw.Kmax + 1
    kv = torch.empty((cw.n_layers, 2, cc["n_blocks"], cw.block_size, cw.entry_bytes), dtype=torch.uint8, device=dev)
    rs = torch.empty((cw.B, cw.rec_bytes), dtype=torch.uint8, device=dev)
    sn = torch.empty((cw.B, K1, cw.rec_bytes), dtype=torch.uint8, device=dev)
    seq0 = to_i32(cc["seq_len"])
    seq = seq0.clone()
    acc, vl, path, bt = (to_i32(cc[k]) for k in ("accepted_len", "verify_len", "path", "block_table"))

    def call():
        bd.spec_commit(acc, seq, Kmax=cw.Kmax, kv=kv, block_table=bt, rec_state=rs, rec_snap=sn, verify_len=vl,
                       path=path)
    for _ in range(warmup):
        seq.copy_(seq0)
        call()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        seq.copy_(seq0)
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    per = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
    A = cc["accepted_len"]
    moved = sum(int(np.sum(cc["path"][b, 1: A[b] + 1] != np.arange(1, A[b] + 1))) for b in range(cw.B) if A[b] > 0)
    by = 2.0 * cw.rec_bytes * int((A >= 0).sum()) + 2.0 * moved * cw.n_layers * 2 * cw.entry_bytes
    ms = float(per.mean())
    return {"workload": f"commit: B={cw.B} Kmax={cw.Kmax} tree blocks, {cw.n_layers} attention layers x "
                        f"{cw.entry_bytes} B entries, {cw.rec_bytes >> 20} MiB recurrent state per request",
            "ms_per_call": ms, "call_ms_spread": {"median": float(np.median(per)), "min": float(per.min()),
                                                  "max": float(per.max())},
            "bytes_per_call": by,
            "roofline": roofline(by, 0.0, ms, peaks_m, "k_commit_move + k_commit_len")}


def traffic_for(config, mode):
    """HBM bytes per launch of the LM-head GEMM from the committed rocprofv3 counter runs,
    if they were taken on the current kernel source; else None."""
    path = os.path.join(HERE, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(f"{config}/{mode}")
    if not ent:
        return None
    import hashlib
    src = os.path.join(HERE, "draft_block_verification_spec_amd", "csrc", ent.get("source", ""))
    try:
        h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    return ent["bytes_per_launch"] if h == ent.get("source_sha256_16") else None


_ORACLE_W: dict = {}


def cpu_baseline(wk, sets, mode, wdata):
    """The fp64 oracle on the host cores: whole verification steps of the same workload on a
    bounded sample (one request of each input set, about ten seconds of host work), and -
    for sampled points - the closed-form expected tau of those requests,
    1 + sum_k prod_{i<=k} alpha_i with alpha_i = sum_v min(p_i, q_i)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    if _ORACLE_W.get("key") is not wdata:  # the fp64 weights of the last weight set, widened once
        _ORACLE_W.clear()
        _ORACLE_W.update(key=wdata, W=oracle.Weights.from_bits(wdata))
    W = _ORACLE_W["W"]
    B, K = wk.B, wk.K
    nb = 1
    t_steps, closed, reps = 0.0, [], 0
    t_all = time.time()
    for datac in sets:
        h64 = oracle.from_bf16_bits(datac["h"][:nb])
        hd64 = oracle.from_bf16_bits(datac["h_draft"][:nb])
        coins = datac["coins"][:nb].astype(np.float64)
        T = 0.0 if mode == "greedy" else wk.T
        draft = oracle.propose(W, hd64, T, None if T == 0 else datac["draft_coins"][:nb])["draft"]
        t1 = time.time()
        if mode == "greedy":
            oracle.verify_greedy(W, h64, draft)
        elif mode == "sample":
            r = oracle.verify_sample(W, h64, hd64, draft, coins, wk.T)
            closed.extend(oracle.tau_closed_form(a) for a in r["alpha"])
        else:
            oracle.verify_scheduled(W, h64, hd64, draft, coins, wk.T, wk.threshold, max(nb, wk.budget * nb // B))
        t_steps += time.time() - t1
        reps += 1
        if time.time() - t_all >= 20.0:
            break
    sec = t_steps / reps
    out = {"value": nb * (K + 1) / sec, "unit": "positions/s", "cores": int(threads),
           "os_cpu_count": os.cpu_count(), "kind": "oracle",
           "sample": f"{reps} verify step(s) of {nb} request x {K + 1} positions of {wk.name} ({mode}), one per "
                     f"input set; fp64, {sec:.3f} s per step (drafting not counted)"}
    if closed:
        out["tau_closed_form"] = {"tau": float(np.mean(closed)), "requests": len(closed),
                                  "rule": "1 + sum_k prod_{i<=k} alpha_i, alpha_i = sum_v min(p_i, q_i) (fp64 oracle)"}
    return out


if __name__ == "__main__":
    main()
