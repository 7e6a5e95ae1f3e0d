"""Benchmark of the draft-block verification step on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--config block16] [--no-extra] [--no-cpu]

A step is one call of the whole verification path (MLP, shared LM head over the
target and draft rows, statistics, acceptance, residual/bonus sampling, tau) on a
batch of synthetic inputs already resident in HBM.  The headline workload is the
16-token block (B=1, K=15, d=4096, d_ff=12288, V=151936, T=1 sampled); `value` is
verified positions per second (B*(K+1) target rows per step).  Rank 0 prints one
JSON line.  Extra points (greedy at B=1; the greedy batch sweep at B=8, 32, 128; the
confidence-scheduled step, literal and budget-binding; the wide model) are reported
under "extra", each with its own roofline and the spread of single-step times.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "verified positions/sec + accepted tokens/sec @B=1,128; % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps before each timed loop; the GPU clock needs ~0.1 s of work to settle")
    ap.add_argument("--config", default="block16", choices=["block16", "sweep", "sched", "sched_stress", "wide"])
    ap.add_argument("--batch", type=int, default=0, help="override B (sweep)")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--mode", default="", choices=["", "sample", "greedy", "scheduled"])
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy 1 GiB device-to-device once (a copy kernel of known size for counter scaling)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1", "n_gpus": args.gpus}))
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

    wk = wl.PRESETS[args.config]
    if args.batch:
        wk = wk.with_batch(args.batch)
    mode = args.mode or {"block16": "sample", "sweep": "greedy", "sched": "scheduled",
                         "sched_stress": "scheduled", "wide": "sample"}[args.config]
    t0 = time.time()
    data = wl.generate(wk)
    log(f"generated {wk.name} inputs in {time.time() - t0:.1f}s")
    def weights(datac, wkc):
        return bd.Weights(to_bf16(datac["w_lm"]), to_bf16(datac["w_gate"]) if wkc.d_ff else None,
                          to_bf16(datac["w_up"]) if wkc.d_ff else None, to_bf16(datac["w_down"]) if wkc.d_ff else None)

    w = w_main = weights(data, wk)

    def prepare(wkc, datac, modec, wts=None):
        """Device inputs, drafts from the library's own drafter step, outputs, workspace."""
        w = wts if wts is not None else w_main
        h = to_bf16(datac["h"])
        hd = to_bf16(datac["h_draft"])
        u = to_f32(datac["coins"])
        T = 0.0 if modec == "greedy" else wkc.T
        draft, _ = bd.spec_draft_propose(w, hd, to_f32(datac["draft_coins"]), T)
        draft = draft.contiguous()
        B, K = wkc.B, wkc.K
        mcode = {"greedy": bd.SV_MODE_GREEDY, "sample": bd.SV_MODE_SAMPLE, "scheduled": bd.SV_MODE_SCHEDULED}[modec]
        out = bd.make_outputs(B, K, dev, mode=mcode, V=wkc.V, d=wkc.d)
        ws = bd.workspace(mcode, B, K, w, dev)

        def call():
            if modec == "greedy":
                bd.spec_verify_greedy(w, h, draft, out=out, ws=ws)
            elif modec == "sample":
                bd.spec_verify_sample(w, h, hd, draft, u, T, out=out, ws=ws)
            else:
                bd.spec_verify_scheduled(w, h, hd, draft, u, T, wkc.threshold, wkc.budget, out=out, ws=ws)
        return call, out

    def timed(call, out, steps, warmup):
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        # clean timed region: whole steps only
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        # same steps again with events around the dominant LM-head GEMM (on the call's stream)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in evs:  # materialise the HIP events; the library re-records them around the GEMM
            a.record()
            b.record()
        torch.cuda.synchronize()
        e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e2.record()
        for i in range(steps):
            out.ev_lm = evs[i]
            call()
        e3.record()
        torch.cuda.synchronize()
        out.ev_lm = None
        lm_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        ms_instr = e2.elapsed_time(e3) / steps
        # and once more with an event between consecutive steps: the spread of single steps
        sev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        sev[0].record()
        for i in range(steps):
            call()
            sev[i + 1].record()
        torch.cuda.synchronize()
        per = np.array([sev[i].elapsed_time(sev[i + 1]) for i in range(steps)])
        spread = {"median": float(np.median(per)), "min": float(per.min()), "max": float(per.max())}
        return ms, lm_ms, ms_instr, spread

    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    call, out = prepare(wk, data, mode)
    ms, lm_ms, ms_instr, spread = timed(call, out, args.steps, args.warmup)
    st = int(out.dev_status.item())
    if st != 0:
        raise SystemExit(f"device status {st}")
    counters = out.counters.cpu().numpy()
    tau = float(out.tau.item())
    B, K, d, V, d_ff = wk.B, wk.K, wk.d, wk.V, wk.d_ff
    vl = out.verify_len.cpu().numpy() if out.verify_len is not None else None
    M_t = int((vl + 1).sum()) if vl is not None else B * (K + 1)
    pos_s = M_t / (ms * 1e-3)
    tok_s = float(counters[2]) / (ms * 1e-3)
    rows_lm = (B * K if mode == "scheduled" else (M_t + B * K if mode == "sample" else M_t))
    lm_bytes = 2.0 * V * d + 2.0 * rows_lm * d
    lm_flops = 2.0 * rows_lm * d * V
    ai = lm_flops / lm_bytes
    if ai < 315:
        roof = {"bound": "hbm", "achieved": lm_bytes / (lm_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": lm_flops / (lm_ms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic_for(args.config, mode, lm_bytes)
    roof["kernel"] = "LM-head GEMM (shared head over target and draft rows)"
    roof["launch_ms"] = lm_ms
    step_bytes = float(wk.weight_bytes())
    result = {
        "metric": METRIC, "value": pos_s, "unit": "positions/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded normals, bf16 weights; no real model)",
        "config": {"workload": f"{wk.name}: B={B} K={K} d={d} d_ff={d_ff} V={V} mode={mode}"
                   + (f" T={wk.T}" if mode != "greedy" else ""), "B": B, "K": K, "d": d, "d_ff": d_ff, "V": V,
                   "mode": mode},
        "accepted_tokens_per_sec": tok_s, "accepted_drafts_per_sec": float(counters[0]) / (ms * 1e-3),
        "tau": tau, "step_hbm_fraction": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "ms_per_step_with_lm_events": ms_instr, "step_ms_spread": spread, "roofline": roof,
    }
    if mode == "scheduled":
        result["config"]["budget"] = wk.budget
        result["config"]["threshold"] = wk.threshold
        result["verified_rows"] = M_t
    log(f"{wk.name}/{mode}: {ms:.3f} ms/step, {pos_s:.0f} pos/s, LM head {lm_ms:.3f} ms "
        f"({roof['achieved']:.0f} {roof['unit']})")

    if not args.no_extra and args.config == "block16":
        extra = []
        # greedy on the same block
        call_g, out_g = prepare(wk, data, "greedy")
        msg, lmg, _, sp_g = timed(call_g, out_g, args.steps, args.warmup)
        b_lm = 2.0 * V * d + 2.0 * B * (K + 1) * d
        extra.append({"workload": f"block16 greedy: B=1 K=15", "ms_per_step": msg, "step_ms_spread": sp_g,
                      "positions_per_sec": B * (K + 1) / (msg * 1e-3),
                      "accepted_tokens_per_sec": float(out_g.counters.cpu().numpy()[2]) / (msg * 1e-3),
                      "tau": float(out_g.tau.item()),
                      "roofline": {"bound": "hbm", "achieved": b_lm / (lmg * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                                   "unit": "GB/s", "frac": b_lm / (lmg * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                   "kernel": "LM-head GEMM", "launch_ms": lmg},
                      "step_hbm_fraction": step_bytes / (msg * 1e-3) / 1e9 / HBM_PEAK_GBS})
        log(f"block16/greedy: {msg:.3f} ms/step")
        del call_g, out_g
        # FP8 (E4M3) weights with per-row fp32 scales, same block: one byte per weight streamed
        d8 = wl.to_fp8(data)
        w8 = bd.Weights(*(torch.from_numpy(np.ascontiguousarray(d8["q_" + n])).to(dev) for n in ("lm", "gate", "up", "down")),
                        *(to_f32(d8["s_" + n]) for n in ("lm", "gate", "up", "down")))
        del d8
        step8 = float(wk.weight_bytes()) / 2 + 4.0 * (V + 2 * d_ff + d)
        for m8 in ("sample", "greedy"):
            call8, out8 = prepare(wk, data, m8, w8)
            ms8, lm8, _, sp8 = timed(call8, out8, args.steps, args.warmup)
            rows8 = B * (K + 1) + (B * K if m8 == "sample" else 0)
            b8 = 1.0 * V * d + 4.0 * V + 2.0 * rows8 * d
            extra.append({"workload": f"block16 {m8}, FP8 E4M3 weights + fp32 row scales: B=1 K=15"
                                      + (f" T={wk.T}" if m8 == "sample" else ""),
                          "ms_per_step": ms8, "step_ms_spread": sp8,
                          "positions_per_sec": B * (K + 1) / (ms8 * 1e-3),
                          "accepted_tokens_per_sec": float(out8.counters.cpu().numpy()[2]) / (ms8 * 1e-3),
                          "tau": float(out8.tau.item()),
                          "roofline": {"bound": "hbm", "achieved": b8 / (lm8 * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                                       "unit": "GB/s", "frac": b8 / (lm8 * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                       "kernel": f"LM-head GEMM over {rows8} rows, FP8 weights", "launch_ms": lm8},
                          "step_hbm_fraction": step8 / (ms8 * 1e-3) / 1e9 / HBM_PEAK_GBS})
            log(f"block16/{m8} fp8: {ms8:.3f} ms/step, LM head {lm8:.3f} ms")
            del call8, out8
        del w8
        # the batch sweep (K = 7 greedy, same weight shapes): B = 8, 32 HBM-bound, B = 128 MFMA-bound
        for Bs in (8, 32, 128):
            wk2 = wl.SWEEP.with_batch(Bs)
            d2 = wl.generate(wk2, weights=False)
            call2, out2 = prepare(wk2, d2, "greedy")
            ms2, lm2, _, sp2 = timed(call2, out2, max(5, args.steps // 2), max(2, args.warmup // 2))
            M2 = wk2.B * (wk2.K + 1)
            flops = 2.0 * M2 * 3 * d * d_ff + 2.0 * M2 * d * V
            lm_fl, lm_b = 2.0 * M2 * d * V, 2.0 * V * d + 2.0 * M2 * d
            pt = {"workload": f"sweep greedy: B={Bs} K=7 (same shapes)", "ms_per_step": ms2, "step_ms_spread": sp2,
                  "positions_per_sec": M2 / (ms2 * 1e-3),
                  "accepted_tokens_per_sec": float(out2.counters.cpu().numpy()[2]) / (ms2 * 1e-3),
                  "tau": float(out2.tau.item()),
                  "step_tflops": flops / (ms2 * 1e-3) / 1e12,
                  "step_mfma_fraction": flops / (ms2 * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                  "step_hbm_fraction": step_bytes / (ms2 * 1e-3) / 1e9 / HBM_PEAK_GBS}
            if lm_fl / lm_b >= 315:
                pt["roofline"] = {"bound": "mfma", "achieved": lm_fl / (lm2 * 1e-3) / 1e12,
                                  "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": lm_fl / (lm2 * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                                  "kernel": "LM-head GEMM", "launch_ms": lm2}
            else:
                pt["roofline"] = {"bound": "hbm", "achieved": lm_b / (lm2 * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": lm_b / (lm2 * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                  "kernel": "LM-head GEMM", "launch_ms": lm2}
            extra.append(pt)
            log(f"sweep B={Bs} greedy: {ms2:.3f} ms/step, {flops / (ms2 * 1e-3) / 1e12:.0f} TFLOP/s")
            del call2, out2, d2
        # the confidence-scheduled step: literal configuration and the budget-binding stress variant
        for wk3 in (wl.SCHED, wl.SCHED_STRESS):
            d3 = wl.generate(wk3, weights=False)
            call3, out3 = prepare(wk3, d3, "scheduled")
            ms3, lm3, _, sp3 = timed(call3, out3, max(5, args.steps // 2), max(2, args.warmup // 2))
            vl3 = out3.verify_len.cpu().numpy()
            M3 = int((vl3 + 1).sum())
            rows_d = wk3.B * wk3.K
            s1_fl = 2.0 * rows_d * d * V
            extra.append({"workload": f"{wk3.name} scheduled: B={wk3.B} Kmax={wk3.K} budget={wk3.budget} "
                                      f"threshold={wk3.threshold} T={wk3.T}",
                          "ms_per_step": ms3, "step_ms_spread": sp3, "verified_rows": M3,
                          "positions_per_sec": M3 / (ms3 * 1e-3),
                          "accepted_tokens_per_sec": float(out3.counters.cpu().numpy()[2]) / (ms3 * 1e-3),
                          "tau": float(out3.tau.item()),
                          "roofline": {"bound": "mfma", "achieved": s1_fl / (lm3 * 1e-3) / 1e12,
                                       "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                       "frac": s1_fl / (lm3 * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                                       "kernel": f"draft-confidence LM-head pass over {rows_d} rows",
                                       "launch_ms": lm3}})
            log(f"{wk3.name}: {ms3:.3f} ms/step, {M3} verified rows")
            del call3, out3, d3
        # the same block verified as a top-k tree of depth 3 (root: 4 candidates, each 2, then 1)
        for mt in ("sample", "greedy"):
            extra.append(bench_tree(bd, torch, wl, wk, data, w_main, dev, to_bf16, to_i32, to_f32, mt, timed,
                                    args.steps, args.warmup))
            log(f"block16 tree {mt}: {extra[-1]['ms_per_step']:.3f} ms/step, tau {extra[-1]['tau']:.2f}")
        # commit after verification: the scheduled batch (B = 64, Kmax = 15) with tree-shaped
        # blocks on a hybrid target (8 attention layers x 2 KiB entries, 1 MiB recurrent state)
        extra.append(bench_commit(bd, torch, wl, dev, to_i32, args.steps, args.warmup))
        log(f"commit: {extra[-1]['ms_per_call'] * 1e3:.1f} us/call")
        # the wide model (d = 8192, d_ff = 28672, V = 128256), B = 32, K = 4, T = 0.7, sampled
        wk4 = wl.WIDE
        d4 = wl.generate(wk4)
        w4 = weights(d4, wk4)
        call4, out4 = prepare(wk4, d4, "sample", w4)
        ms4, lm4, _, sp4 = timed(call4, out4, max(5, args.steps // 2), max(2, args.warmup // 2))
        M4t, M4 = wk4.B * (wk4.K + 1), wk4.B * (2 * wk4.K + 1)
        b4 = 2.0 * wk4.V * wk4.d + 2.0 * M4 * wk4.d
        extra.append({"workload": f"wide sample: B={wk4.B} K={wk4.K} d={wk4.d} d_ff={wk4.d_ff} V={wk4.V} T={wk4.T}",
                      "ms_per_step": ms4, "step_ms_spread": sp4,
                      "positions_per_sec": M4t / (ms4 * 1e-3),
                      "accepted_tokens_per_sec": float(out4.counters.cpu().numpy()[2]) / (ms4 * 1e-3),
                      "tau": float(out4.tau.item()),
                      "step_hbm_fraction": float(wk4.weight_bytes()) / (ms4 * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      "roofline": {"bound": "hbm", "achieved": b4 / (lm4 * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                                   "unit": "GB/s", "frac": b4 / (lm4 * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                   "kernel": f"LM-head GEMM over {M4} rows", "launch_ms": lm4}})
        log(f"wide: {ms4:.3f} ms/step")
        del call4, out4, w4, d4
        result["extra"] = extra

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(wk, data, mode, out, w, bd, torch)
    print(json.dumps(result), flush=True)


def bench_tree(bd, torch, wl, wk, data, w, dev, to_bf16, to_i32, to_f32, mode, timed, steps, warmup):
    """spec_verify_tree on the 16-token block shaped as a top-k tree.  Drafts come from
    the library's drafter step on each child's parent row: the first child of a node takes
    the argmax, later siblings are samples (coin of the child)."""
    B, K, V, d = wk.B, wk.K, wk.V, wk.d
    parent = wl.tree_parents(B, K, "topk")
    hd = to_bf16(data["h_draft"])  # [B, K, d]: drafter row of node u is row u
    rows = hd[torch.arange(B, device=dev)[:, None], to_i32(parent).long()].reshape(B * K, d).contiguous()
    x_s, _ = bd.spec_draft_propose(w, rows, to_f32(data["draft_coins"]).reshape(-1), 1.0)
    x_g, _ = bd.spec_draft_propose(w, rows, None, 0.0)
    first = np.ones((B, K), bool)
    for b in range(B):
        seen = set()
        for j in range(K):
            first[b, j] = parent[b, j] not in seen
            seen.add(parent[b, j])
    tokens = torch.where(torch.from_numpy(first.reshape(-1)).to(dev), x_g, x_s).view(B, K).contiguous()
    T = 0.0 if mode == "greedy" else wk.T
    h = to_bf16(data["h"])
    u = to_f32(data["coins"])
    par = to_i32(parent)
    mcode = bd.SV_MODE_GREEDY if mode == "greedy" else bd.SV_MODE_SAMPLE
    out = bd.make_outputs(B, K, dev, mode=mcode, V=V, d=d)
    out.path = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    ws = bd.workspace(mcode, B, K, w, dev)

    def call():
        bd.spec_verify_tree(w, h, hd, tokens, par, u, T, out=out, ws=ws)
    ms, lm, _, sp = timed(call, out, steps, warmup)
    rows_lm = B * (K + 1) + (0 if mode == "greedy" else B * K)
    b_lm = 2.0 * V * d + 2.0 * rows_lm * d
    return {"workload": f"block16 tree {mode}: B={B}, {K + 1} nodes (top-k tree, depth 3)"
                        + ("" if mode == "greedy" else f", T={wk.T}"),
            "ms_per_step": ms, "step_ms_spread": sp, "positions_per_sec": B * (K + 1) / (ms * 1e-3),
            "accepted_tokens_per_sec": float(out.counters.cpu().numpy()[2]) / (ms * 1e-3),
            "tau": float(out.tau.item()),
            "roofline": {"bound": "hbm", "achieved": b_lm / (lm * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": b_lm / (lm * 1e-3) / 1e9 / HBM_PEAK_GBS, "kernel": f"LM-head GEMM over {rows_lm} rows",
                         "launch_ms": lm}}


def bench_commit(bd, torch, wl, dev, to_i32, steps, warmup):
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
            "roofline": {"bound": "hbm", "achieved": by / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "kernel": "k_commit_move + k_commit_len",
                         "launch_ms": ms}}


def traffic_for(config, mode, lm_bytes):
    """HBM bytes per launch of the LM-head GEMM from the committed rocprofv3 counter runs,
    if they were taken on the current kernel source; else None."""
    path = os.path.join(HERE, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    key = f"{config}/{mode}"
    ent = rec.get(key)
    if not ent:
        return None
    import hashlib
    src = os.path.join(HERE, "draft_block_verification_spec_amd", "csrc", ent.get("source", ""))
    try:
        h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    return ent["bytes_per_launch"] if h == ent.get("source_sha256_16") else None


def cpu_baseline(wk, data, mode, out, w, bd, torch):
    """The fp64 oracle on the host cores: one full verification step of the same workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    W = oracle.Weights.from_bits(data)
    B, K = wk.B, wk.K
    rows = slice(0, min(B, 1 if wk.d >= 4096 else B))
    nb = rows.stop - rows.start
    h64 = oracle.from_bf16_bits(data["h"][rows])
    hd64 = oracle.from_bf16_bits(data["h_draft"][rows])
    # the drafts the GPU verified (from the library's drafter step)
    coins = data["coins"][rows].astype(np.float64)
    t0 = time.time()
    if mode == "greedy":
        draft = oracle.propose(W, hd64, 0.0, None)["draft"]
    else:
        draft = oracle.propose(W, hd64, wk.T, data["draft_coins"][rows])["draft"]
    t1 = time.time()
    reps = 0
    while True:  # repeat whole verify steps for about ten seconds of host work
        if mode == "greedy":
            oracle.verify_greedy(W, h64, draft)
        elif mode == "sample":
            oracle.verify_sample(W, h64, hd64, draft, coins, wk.T)
        else:
            oracle.verify_scheduled(W, h64, hd64, draft, coins, wk.T, wk.threshold, max(nb, wk.budget * nb // B))
        reps += 1
        if time.time() - t1 >= 10.0 or reps >= 500:
            break
    t2 = time.time()
    sec = (t2 - t1) / reps
    return {"value": nb * (K + 1) / sec, "unit": "positions/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{nb} request(s) x {K + 1} positions of {wk.name} ({mode}); fp64 verify step repeated "
                      f"{reps}x in {t2 - t1:.1f} s ({sec:.3f} s per step; drafting {t1 - t0:.1f} s not counted)"}


if __name__ == "__main__":
    main()
