"""Benchmark of the P-EAGLE parallel-drafter forward on one MI355X.

A step is one pe_draft_forward (input fusion, N decoder layers, LM head with
fused argmax) over the synthetic GPT-OSS-20B-shaped drafter workload
(H 2880, 4 layers, 64 q / 8 kv heads, head_dim 64, SwiGLU 8192, vocab
201088, K = 8, batch 2, 4096 cached positions, bf16), all inputs resident
in HBM.  Prints one JSON line:

  value      draft tokens/s = B*K / mean step time over the timed steps
  roofline   the dominant kernel (LM head with fused argmax): algorithmic
             bytes per launch / mean launch time from HIP events recorded
             around it on the forward's stream during the timed steps
  forward_roofline  the whole forward's algorithmic bytes / step time (the
                    fraction the 60% target is stated on)
  step_distribution p10 / median / p90 of single forwards timed one by one
                    after the bracketed steps
  graph      the same forward captured once in a hipGraph and replayed
  cpu_baseline      the CPU oracle on the same workload (host cores)
  extra      the other decode workloads, each timed the same way: 16384
             cached positions; the Qwen3-Coder-30B shape (B 4, ragged
             contexts); the tiny fp32 drafter (latency only)
  eagle3_chain      the sequential drafter on the same kernels
  train_forward     the training-shape forward (one drafter layer over a COD
                    layout of 8192 positions, K = 8, about 34K kept rows,
                    bf16 logits at every row): rows/s and its matrix-core
                    roofline (LM-head kernel and whole forward, TFLOP/s)
  train_step        forward, loss and backward of the same layout

Usage: python bench.py [--steps K] [--warmup W] [--workload NAME]
       [--no-cpu-baseline] [--no-graph] [--no-extra] [--copy-calibration]
       [--no-train | --train-only] [--train-steps S] [--no-step] [--no-chain]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
METRIC = "draft tokens/s per P-EAGLE forward (K=8, ctx 4K) + % of HBM roofline"
COUNTERS = os.path.join(ROOT, "profiles", "lm_head_counters.json")
# Sources of the LM-head kernel; counters taken on other sources are stale.
KERNEL_SRCS = [os.path.join(ROOT, "drafting_eagle_draft_amd", "csrc", f) for f in
               ("gemm_wg.hip", "pe_epilogue.hpp", "pe_device.hpp", "pe_internal.hpp")]


def kernel_sha256():
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def algorithmic_bytes(cfg, ctx_lens, B, K):
    """Bytes one forward must move at least once: every weight streamed once,
    the cached keys/values of each sequence read once, plus inputs/outputs."""
    e = 2 if cfg.dtype == "bf16" else 4
    H, I, V, hd = cfg.hidden, cfg.intermediate, cfg.vocab, cfg.head_dim
    nq, nkv, N = cfg.n_q_heads, cfg.n_kv_heads, cfg.n_layers
    layer_w = ((nq + 2 * nkv) * hd * H + H * nq * hd + 2 * I * H + H * I) * e
    kv = 2 * int(np.sum(ctx_lens)) * nkv * hd * e
    fc = H * 3 * H * e
    lm = V * H * e
    io = (B * 3 * H + B * H + H + 3 * H) * e + B * 8 + B * K * 4
    return {"total": fc + N * layer_w + N * kv + lm + io, "lm_head": lm + B * K * H * e,
            "layers": N * layer_w, "kv": N * kv, "fc": fc}


def _weights_f64(w, token_ids):
    """The oracle's operands in float64, converted once: every weight matrix
    and gain, and only the embedding rows the forward reads."""
    def f64(a):
        return np.asarray(a, dtype=np.float64)
    out = {k: f64(v) for k, v in w.items() if k not in ("layers", "embed")}
    out["embed_rows"] = f64(w["embed"][token_ids])
    out["layers"] = [{k: f64(v) for k, v in lw.items()} for lw in w["layers"]]
    return out


def cpu_baseline(cfg, w, inp, reps=3):
    """The oracle as it stands, on this host's cores.  Its weights and inputs
    are converted to float64 once, outside the timed span; then one untimed
    warm run and the median of ``reps`` full forwards of the same workload."""
    from threadpoolctl import threadpool_info
    from oracle import peagle_oracle as po
    t0 = time.perf_counter()
    w64 = _weights_f64(w, inp["token_ids"])
    kc = [np.asarray(c, dtype=np.float64) for c in inp["k_cache"]]
    vc = [np.asarray(c, dtype=np.float64) for c in inp["v_cache"]]
    conv_s = time.perf_counter() - t0
    args = (w64, cfg, np.asarray(inp["hidden3"], np.float64), inp["token_ids"],
            np.asarray(inp["mask_emb"], np.float64), np.asarray(inp["h_shared"], np.float64),
            inp["ctx_lens"], kc, vc, inp["K"])
    po.draft_forward(*args)
    times = []
    for _ in range(reps):
        t = time.perf_counter()
        po.draft_forward(*args)
        times.append(time.perf_counter() - t)
    t = float(np.median(times))
    del w64, kc, vc
    B, K = len(inp["token_ids"]), inp["K"]
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": B * K / t, "unit": "draft tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"the full workload: median of {reps} timed full forwards ({t:.2f} s each, "
                      f"all {B * K} rows, fp64 NumPy) after one warm run; weights, cache and inputs "
                      f"converted to fp64 once beforehand ({conv_s:.1f} s, not timed)"}


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
MFMA_F32_PEAK_TFLOPS = 157.3


def train_flops(cfg, n, rows, K):
    """Algorithmic flops of one training-shape forward over kept rows ``rows``:
    2 x weights per row for every projection of every kept row (fc once per
    position plus once for the shared hidden state), and 4 x hd x n_q per
    allowed query/key pair, each row seeing p + 1 keys."""
    H, I, V, hd = cfg.hidden, cfg.intermediate, cfg.vocab, cfg.head_dim
    nq, nkv, N = cfg.n_q_heads, cfg.n_kv_heads, cfg.n_layers
    L = len(rows)
    layer = (nq + 2 * nkv) * hd * H + H * nq * hd + 2 * I * H + H * I
    fc = 2.0 * (n + 1) * 3 * H * H
    gemm = 2.0 * L * (N * layer + V * H) + fc
    pairs = float(np.sum(np.asarray(rows) // K + 1))
    attn = N * 4.0 * hd * nq * pairs
    return {"total": gemm + attn, "gemm": gemm, "attention": attn, "lm_head": 2.0 * L * V * H,
            "pairs": pairs}


def train_leg(steps, warmup, partition=True):
    """Training-shape forward (one GPT-OSS-20B-shaped drafter layer over a
    COD layout of n = 8192, K = 8, r = 0.8; mask built once for n_max =
    20480; bf16 logits at every kept row)."""
    import torch
    from drafting_eagle_draft_amd import binding as pe
    from drafting_eagle_draft_amd import runner, synth
    cfg = synth.config("train_gptoss20b_n8192_k8")
    n, K = cfg.seq_len, cfg.K
    t0 = time.time()
    w = synth.drafter_weights(cfg)
    inp = synth.train_inputs(cfg)
    U = synth.cod_uniforms(cfg, n, K)
    rows = pe.pe_cod_rows(n, K, cfg.cod_rate, cfg.cod_floor, U.reshape(-1))
    print(f"[bench] training inputs in {time.time() - t0:.1f}s, L = {len(rows)}", file=sys.stderr,
          flush=True)
    d = runner.Drafter(cfg, w)
    del w
    mask = runner.TrainMask(cfg.n_max, K)
    buf = runner.TrainBuffers(d, mask, inp, rows)
    for _ in range(warmup):
        buf.launch(d, mask)
    torch.cuda.synchronize()
    pe.pe_profile_enable(d.handle, True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        buf.launch(d, mask)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    n_lm, lm_ms = pe.pe_profile_read(d.handle)
    pe.pe_profile_enable(d.handle, False)
    del buf
    # The same forward as S = 4 independent chunks, each recomputing its
    # depth-0 completion (sequence partitioning); outputs identical.
    S, part_ms, part_cells, part_ws = 4, None, None, None
    if partition:
        part = runner.PartitionedTrain(d, mask, inp, rows, S)
        part.launch(d, mask)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            part.launch(d, mask)
        e1.record()
        torch.cuda.synchronize()
        part_ms = e0.elapsed_time(e1) / steps
        part_cells, part_ws = part.cells_total, part.ws.numel()
        del part
    L = len(rows)
    f = train_flops(cfg, n, rows, K)
    achieved = f["total"] / (ms * 1e-3) / 1e12
    lm_tf = f["lm_head"] / (lm_ms * 1e-3) / 1e12 if lm_ms > 0 else None
    whole_ws = pe.pe_train_workspace_size(d.handle, n, K, L)
    mask.close()
    d.close()
    torch.cuda.empty_cache()
    return {
        "metric": "kept rows/s per training-shape forward (n 8192, K 8, COD r 0.8)",
        "value": L / (ms * 1e-3), "unit": "rows/s", "ms_per_step": ms, "steps": steps,
        "warmup": warmup, "dtype": cfg.dtype,
        "config": {"workload": cfg.name, "n": n, "K": K, "L": L, "n_max": cfg.n_max,
                   "layers": cfg.n_layers, "logits": "bf16 [L, V]"},
        "roofline": {"bound": "mfma", "kernel": "LM head GEMM + argmax keys",
                     "achieved": lm_tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": (lm_tf / MFMA_BF16_PEAK_TFLOPS) if lm_tf else None, "traffic": None,
                     "algorithmic_flops_per_launch": f["lm_head"], "launches": n_lm,
                     "mean_launch_ms": lm_ms},
        "forward_roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                             "algorithmic_flops": f["total"], "gemm_flops": f["gemm"],
                             "attention_flops": f["attention"], "allowed_pairs": f["pairs"]},
        "partitioned": ({"S": S, "ms_per_step": part_ms, "cells_run": part_cells,
                         "recompute_factor": part_cells / L, "value": L / (part_ms * 1e-3),
                         "workspace_bytes": part_ws, "whole_workspace_bytes": whole_ws}
                        if partition else None),
    }


def step_flops(cfg, n, rows, K):
    """Algorithmic flops of one training step (forward, loss, backward): the
    forward's; twice the projections' GEMM flops for the backward (data and
    weight gradients); and 2.5x the forward attention pairs' work for its
    backward (dP, dS^T Q, dS K, P^T dO against the forward's Q K^T, P V)."""
    f = train_flops(cfg, n, rows, K)
    bwd = 2.0 * f["gemm"] + 2.5 * f["attention"]
    return {"total": f["total"] + bwd, "forward": f["total"], "backward": bwd,
            "lm_head_dgrad": f["lm_head"], "lm_head_wgrad": f["lm_head"]}


def step_leg(steps):
    """Training step (forward, cross-entropy against synthetic next-token
    labels, backward to every weight) of one GPT-OSS-20B-shaped drafter layer
    over the COD layout of n = 8192, K = 8, r = 0.8."""
    import torch
    from drafting_eagle_draft_amd import binding as pe
    from drafting_eagle_draft_amd import runner, synth
    cfg = synth.config("train_gptoss20b_n8192_k8")
    n, K = cfg.seq_len, cfg.K
    w = synth.drafter_weights(cfg)
    inp = synth.train_inputs(cfg)
    U = synth.cod_uniforms(cfg, n, K)
    rows = pe.pe_cod_rows(n, K, cfg.cod_rate, cfg.cod_floor, U.reshape(-1))
    rng = np.random.default_rng(5)
    labels = rng.integers(0, cfg.vocab, n).astype(np.int32)
    labels[-1] = -1
    d = runner.Drafter(cfg, w, backward=True)
    del w
    mask = runner.TrainMask(cfg.n_max, K)
    st = runner.TrainStep(d, mask, inp, rows, labels)
    st.launch(d, mask)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        st.launch(d, mask)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    f = step_flops(cfg, n, rows, K)
    L = len(rows)
    ws = st.ws.numel()
    del st
    mask.close()
    d.close()
    torch.cuda.empty_cache()
    achieved = f["total"] / (ms * 1e-3) / 1e12
    return {"metric": "kept rows/s per training step (forward + loss + backward; n 8192, K 8, COD r 0.8)",
            "value": L / (ms * 1e-3), "unit": "rows/s", "ms_per_step": ms, "steps": steps, "dtype": cfg.dtype,
            "config": {"workload": cfg.name, "n": n, "K": K, "L": L, "layers": cfg.n_layers,
                       "labels": "synthetic next tokens"},
            "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "algorithmic_flops": f["total"],
                         "forward_flops": f["forward"], "backward_flops": f["backward"]},
            "workspace_bytes": ws}


def chain_leg(drafter, inp, K, steps, parallel_ms):
    """The sequential drafter the parallel one replaces, on the same kernels:
    K one-row cache extensions per sequence (each step's token and normalized
    output feed the next), timed like the parallel forward on the same
    workload."""
    import torch
    from drafting_eagle_draft_amd import runner

    ch = runner.Eagle3Chain(drafter, inp, K)
    for _ in range(3):
        ch.launch(drafter)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        ch.launch(drafter)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    B = ch.B
    del ch
    torch.cuda.empty_cache()
    return {"steps": steps, "ms_per_chain": ms, "ms_per_draft_step": ms / K,
            "value": B * K / (ms * 1e-3), "unit": "draft tokens/s",
            "parallel_speedup": ms / parallel_ms,
            "launch": "eager, one stream, K sequential pe_draft_extend calls"}


def traffic_from_counters(lm_launch_bytes):
    """HBM bytes per LM-head launch from the committed rocprofv3 PMC summary,
    or None when missing or taken on a different kernel source."""
    if not os.path.exists(COUNTERS):
        return None
    with open(COUNTERS) as f:
        c = json.load(f)
    if c.get("kernel_sha256") != kernel_sha256():
        return None
    return c.get("hbm_bytes_per_launch")


EXTRA_WORKLOADS = ("gptoss20b_k8_ctx16k", "qwen3coder30b_k8_ragged", "tiny_f32")


def decode_leg(workload, steps, warmup, graph=True, copy_calibration=False, keep=False):
    """Time `steps` pe_draft_forward calls of one decode workload (inputs
    resident in HBM, one stream, events around the whole bracket), then the
    same number of single forwards each between its own event pair, then
    (graph=True) one captured forward replayed `steps` times."""
    import torch
    from drafting_eagle_draft_amd import binding as pe
    from drafting_eagle_draft_amd import runner, synth
    dev = torch.device("cuda:0")
    cfg = synth.config(workload)
    t0 = time.time()
    w = synth.drafter_weights(cfg)
    inp = synth.decode_inputs(cfg)
    print(f"[bench] {workload}: inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    drafter = runner.Drafter(cfg, w, dev)
    buf = runner.DecodeBuffers(drafter, inp, want_logits=False)
    B, K = buf.B, buf.K

    if copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(warmup):
        buf.launch(drafter)
    torch.cuda.synchronize()

    pe.pe_profile_enable(drafter.handle, True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(steps):
        buf.launch(drafter)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    n_lm, lm_ms = pe.pe_profile_read(drafter.handle)
    pe.pe_profile_enable(drafter.handle, False)

    # Distribution of single steps (after the timed bracket, which alone
    # gives the step time): one event pair around each of another `steps`
    # forwards.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        e0.record()
        buf.launch(drafter)
        e1.record()
    torch.cuda.synchronize()
    per_step = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
    step_dist = {"p10_ms": float(np.percentile(per_step, 10)), "median_ms": float(np.median(per_step)),
                 "p90_ms": float(np.percentile(per_step, 90)), "steps": int(steps)}

    graph_out = None
    if graph:
        # One forward captured in a hipGraph and replayed: the same kernels
        # with the launches recorded once (no fill or copy nodes inside).
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            buf.launch(drafter)
        torch.cuda.current_stream().wait_stream(s)
        with torch.cuda.graph(g):
            buf.launch(drafter)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        gms = e0.elapsed_time(e1) / steps
        graph_out = {"ms_per_step": gms, "value": B * K / (gms * 1e-3), "unit": "draft tokens/s",
                     "steps": steps, "launch": "one captured forward replayed per step"}
        del g

    nbytes = algorithmic_bytes(cfg, inp["ctx_lens"], B, K)
    lm_gbs = nbytes["lm_head"] / (lm_ms * 1e-3) / 1e9 if lm_ms > 0 else None
    fwd_gbs = nbytes["total"] / (ms * 1e-3) / 1e9
    ctx = np.asarray(inp["ctx_lens"])
    leg = {
        "ms_per_step": ms,
        "value": B * K / (ms * 1e-3),
        "unit": "draft tokens/s",
        "dtype": cfg.dtype,
        "config": {"workload": cfg.name, "batch": B, "K": K,
                   "ctx": int(ctx[0]) if cfg.ctx else [int(c) for c in ctx],
                   "ctx_stride": int(inp["ctx_stride"]),
                   "layers": cfg.n_layers, "hidden": cfg.hidden, "heads": [cfg.n_q_heads, cfg.n_kv_heads],
                   "head_dim": cfg.head_dim, "intermediate": cfg.intermediate, "vocab": cfg.vocab,
                   "launch": "eager, one stream"},
        # The dominant kernel: the LM head streams most of the forward's bytes.
        "roofline": {"bound": "hbm", "kernel": "LM head GEMM + fused argmax",
                     "achieved": lm_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": (lm_gbs / HBM_PEAK_GBS) if lm_gbs else None,
                     "traffic": (traffic_from_counters(nbytes["lm_head"])
                                 if workload == "gptoss20b_k8_ctx4k" else None),
                     "algorithmic_bytes_per_launch": nbytes["lm_head"], "launches": n_lm,
                     "mean_launch_ms": lm_ms},
        # The whole forward against the same peak: the figure the 60% target is set on.
        "forward_roofline": {"bound": "hbm", "achieved": fwd_gbs, "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": fwd_gbs / HBM_PEAK_GBS,
                             "algorithmic_bytes": nbytes["total"]},
        "step_distribution": step_dist,
        "graph": graph_out,
    }
    del buf
    if keep:
        leg.update(_cfg=cfg, _w=w, _inp=inp, _drafter=drafter)
    else:
        drafter.close()
        del drafter, w
        torch.cuda.empty_cache()
    return leg


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gptoss20b_k8_ctx4k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the hipGraph replay timing")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other decode workloads (16K context, Qwen3-Coder shape, tiny fp32)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--no-train", action="store_true",
                    help="skip the training-shape forward leg")
    ap.add_argument("--train-only", action="store_true",
                    help="run only the training-shape forward leg (its own JSON line)")
    ap.add_argument("--train-steps", type=int, default=5)
    ap.add_argument("--no-step", action="store_true", help="skip the training-step leg")
    ap.add_argument("--step-only", action="store_true", help="run only the training-step leg")
    ap.add_argument("--no-partition", action="store_true",
                    help="skip the 4-chunk form of the training-shape forward")
    ap.add_argument("--no-chain", action="store_true",
                    help="skip the autoregressive EAGLE-3 chain leg")
    ap.add_argument("--chain-steps", type=int, default=20)
    ap.add_argument("--print-kernel-sha", action="store_true",
                    help="print the LM-head kernel source hash and exit")
    a = ap.parse_args()
    if a.print_kernel_sha:
        print(kernel_sha256())
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU: this path runs on a single MI355X and has no "
              f"multi-GPU mode (asked for --gpus {a.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch

    if a.train_only:
        print(json.dumps(train_leg(a.train_steps, 2, not a.no_partition)), flush=True)
        return
    if a.step_only:
        print(json.dumps(step_leg(a.train_steps)), flush=True)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    head = decode_leg(a.workload, a.steps, a.warmup, graph=not a.no_graph,
                      copy_calibration=a.copy_calibration, keep=True)
    cfg, w, inp, drafter, ms = head.pop("_cfg"), head.pop("_w"), head.pop("_inp"), head.pop("_drafter"), \
        head["ms_per_step"]
    B, K = len(inp["token_ids"]), inp["K"]
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) hidden states and cache)",
        "config": head["config"],
        "roofline": head["roofline"],
        "forward_roofline": head["forward_roofline"],
        "step_distribution": head["step_distribution"],
        "graph": head["graph"],
    }
    if not a.no_chain:
        print("[bench] autoregressive EAGLE-3 chain", file=sys.stderr, flush=True)
        out["eagle3_chain"] = chain_leg(drafter, inp, K, a.chain_steps, ms)
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, w, inp)
    else:
        out["cpu_baseline"] = None
    drafter.close()
    del drafter
    torch.cuda.empty_cache()
    if not a.no_extra:
        out["extra"] = {}
        for name in EXTRA_WORKLOADS:
            if name == a.workload:
                continue
            print(f"[bench] decode workload {name}", file=sys.stderr, flush=True)
            leg = decode_leg(name, a.steps, a.warmup, graph=not a.no_graph)
            if name == "tiny_f32":
                leg["note"] = "launch-bound parity workload: its latency is the figure, not the HBM fraction"
            out["extra"][name] = leg
    if not a.no_train:
        print("[bench] training-shape forward", file=sys.stderr, flush=True)
        out["train_forward"] = train_leg(a.train_steps, 2, not a.no_partition)
    if not a.no_step:
        print("[bench] training step", file=sys.stderr, flush=True)
        out["train_step"] = step_leg(a.train_steps)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
