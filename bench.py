#!/usr/bin/env python3
"""Benchmark of the hot/cold-residency MoE layer on one MI355X.

Workload (default): one full-shape routed MoE layer per step -- 384 experts,
top-6, hidden 4096, intermediate 2880 (one MXFP4 expert = 18,800,640 B), 16
decode tokens, 295 hot expert rows in HBM and 89 cold rows in pinned host
memory read in place (--cold-path), a residency map fitted to the routing distribution
(about 1.7% of picks cold), skewed synthetic routing shaped after the pages'
decode histogram. Steps rotate through --layers distinct layer banks and use
fresh routing and activations each step, so the 256 MB Infinity Cache cannot
hold a step's expert bytes.

One step = moe_route_split (usage counter on) -> cold expert FFN on a second
stream (enqueued first, so its few workgroups start at once) and hot expert FFN
(gate/up, down) on the main stream -> moe_finalize; every
64 steps the counter table is snapshotted (moe_usage_counts) at a drained
barrier, the adaptive policy runs with the pages' defaults, and the swaps it
proposes are applied with moe_swap_rows before the next step. All inputs are
resident (device / pinned) before the timed region.

Prints one JSON line (see the keys below). `value` is the achieved HBM
bandwidth of the whole step (algorithmic HBM bytes per step / wall time per
step); `us_per_layer` is the same step time in microseconds. `roofline` covers
the hot-bank gate/up kernel (the kernel that moves the most HBM bytes) and
`roofline_hot_bank` the hot bank's two GEMM kernels together, both timed with
HIP events on the hot bank's stream (that stream is off the step's critical
path whenever the step has a cold pick): an event before gate/up and one after
down in every timed step, and on every KERNEL_SPLIT_EVERY-th timed step one
between the two kernels as well. That middle marker holds the down launch back
by ~14 us (kernel traces: 0 us between the two kernels without it), so the
pair's time comes from the steps without it and each kernel's own time from
the steps with it. Neither uses the first timed step when there are others: it
starts from the idle device that the opening synchronize leaves and runs
slower (the step time includes it). Events on the
main stream (step and cold-path times) would each add ~5 us to the step, so
they are taken in a separate untimed pass over the first timed steps
(--profile-steps); the step time itself is the wall clock over all timed
steps. The timed steps' routing is drawn so that their cold-expert counts
follow the generator's distribution (quantiles of a larger draw per layer
bank, --no-stratify to draw every step on its own): one cold expert costs
~0.35 ms over the host link, so a short run's mean otherwise swings with how
many the draw happens to hit. `cpu_baseline` is the CPU oracle on sampled
steps of the same workload.
"""
from __future__ import annotations

import argparse
import bisect
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer µs/decode step + achieved HBM GB/s (384e top-6 MXFP4, 1 GPU)"
PEAK_HBM_GBPS = 8000.0
COLD_BANK = {"inplace": "pinned_host_in_place", "staged": "pinned_host_staged_to_hbm",
             "dma": "pinned_host_dma_copied_to_hbm"}
NOMINAL_LINK_GBPS = 63.0
KERNEL_SPLIT_EVERY = 4  # timed steps with an event between hot gate/up and down


def kernel_split_step(i: int, steps: int) -> bool:
    """Whether timed step i records an event between the hot gate/up and down
    kernels: the steps in the middle of each group of KERNEL_SPLIT_EVERY (the
    first step after the synchronize that opens the timed region runs from an
    idle device, which a short run would over-weight), or the first step when
    the run is shorter than that."""
    if steps <= KERNEL_SPLIT_EVERY // 2:
        return i == 0
    return i % KERNEL_SPLIT_EVERY == KERNEL_SPLIT_EVERY // 2


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--layers", type=int, default=8, help="distinct layer banks rotated through")
    ap.add_argument("--tokens", type=int, default=16)
    ap.add_argument("--map", default="fitted", choices=["fitted", "positional"])
    ap.add_argument("--cold-rows", type=int, default=89,
                    help="rows of each layer's cold bank (the rest of the 384 experts are hot); "
                         "89 is the workload's split, fewer show the effect of a larger HBM budget")
    ap.add_argument("--serial", action="store_true", help="cold FFN on the main stream")
    ap.add_argument("--no-policy", action="store_true", help="no counter reads or swaps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true")
    ap.add_argument("--streams", choices=["cold-side", "hot-side"], default="hot-side",
                    help="decode: which bank's FFN goes on the second stream (the other stays "
                         "on the main stream with the split and the finalize)")
    ap.add_argument("--seed", type=int, default=20260917)
    ap.add_argument("--cold-path", default=None, choices=["staged", "inplace", "dma"],
                    help="inplace: the cold FFN reads the pinned host bank directly (the pages' "
                         "method; at decode sizes each item's bytes cross the link as one "
                         "linear stream into LDS); staged: copy the step's active cold rows into "
                         "HBM with one contiguous stream each (moe_stage_rows), then run the "
                         "cold FFN from HBM. Default: inplace for steps of at most 16 tokens, "
                         "staged above (the kernels for larger steps read host memory at "
                         "~40 GB/s in place; the copy runs at the link's ~55 GB/s). dma: "
                         "the staging copy by the DMA engines (moe_stage_rows_dma) from the "
                         "active rows read back to the host after the split")
    ap.add_argument("--cold-scales", default="host", choices=["host", "device"],
                    help="host: the cold bank whole in pinned host memory (the pages' layout); "
                         "device: its E8M0 scale tensors (1/16 of the weight bytes) in HBM, so "
                         "only the E2M1 weights cross the host link (moe_bank on_host = "
                         "MOE_BANK_HOST_WEIGHTS)")
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "step40", "highconc", "offdomain",
                             "domainshift", "refit", "counter", "swap"],
                    help="decode: the default line (one layer of 16 tokens per step); prefill: "
                         "one 4096-token chunk per step (counter off), with the hot bank's MFMA "
                         "utilisation; step40: 40 layer calls of 7 tokens per step; highconc: "
                         "112 tokens per step (--map fitted or positional); offdomain: 7 tokens, "
                         "map fitted to one ranking, traffic from another, the adaptive policy "
                         "moving experts, reported in windows; domainshift: 7 tokens, traffic "
                         "from the map's ranking, then another, then the first again (equal "
                         "phases), the policy following, then a restore to the boot map; refit: "
                         "the off-domain boot, a count-only profile (--profile-tokens per layer), "
                         "a map fitted off-line to those counts and applied, then timed on fresh "
                         "traffic with no on-line policy; counter: the split kernel of 40 layers "
                         "captured in a HIP graph, with and without the usage counter, at 6, 16 "
                         "and 32 tokens; swap: full-size row swaps between the hot and the cold "
                         "bank, time per swap")
    ap.add_argument("--profile-tokens", type=int, default=50_000,
                    help="refit: decode tokens counted per layer before fitting (the pages' "
                         "floor for a count profile is 50,000)")
    ap.add_argument("--routing", default="auto", choices=["auto", "independent", "window"],
                    help="independent: every token routed on its own (skewed per-expert "
                         "probabilities); window: tokens in verify windows of 7 share a "
                         "per-window term, fitted to the pages' touched-set curve; auto: window "
                         "for the 7-token workloads and highconc (16 windows of 7), independent "
                         "for decode and prefill")
    ap.add_argument("--profile-steps", type=int, default=64,
                    help="untimed pass after the timed steps, over the first n of them again, "
                         "with events on every kernel (step, cold path and hot kernels): the "
                         "percentiles and the cold-link rate come from it (0: none)")
    ap.add_argument("--no-stratify", action="store_true",
                    help="draw each timed step's routing on its own instead of at quantiles of "
                         "cold-expert count per layer bank")
    ap.add_argument("--ctrl", default=None,
                    help="runtime control file (JSON) read at every policy barrier: freeze, "
                         "counting, budgets, dump_counts, restore_map")
    ap.add_argument("--telemetry", default=None, help="append one JSON line per policy barrier")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step (all its layer calls) as a HIP graph and replay it "
                         "(workloads whose steps run every layer bank once: step40, offdomain, "
                         "domainshift); per-kernel times are then not reported")
    return ap.parse_args()


# ------------------------------------------------------------- ceilings --

def _hip():
    h = ctypes.CDLL("libamdhip64.so")
    h.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                          ctypes.c_uint]
    return h


def device_pointer(t):
    """Device address of a pinned host tensor."""
    p = ctypes.c_void_p()
    rc = _hip().hipHostGetDevicePointer(ctypes.byref(p), ctypes.c_void_p(t.data_ptr()), 0)
    if rc != 0:
        raise RuntimeError(f"hipHostGetDevicePointer failed: {rc}")
    return p.value


def measure_ceilings(torch):
    L = ctypes.CDLL(os.path.join(ROOT, "ceiling", "libceiling.so"))
    L.ceiling_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_void_p]
    L.ceiling_stream_read.restype = ctypes.c_int
    blocks = 256 * 16
    sink = torch.empty(blocks, dtype=torch.int64, device="cuda")
    s = torch.cuda.current_stream()

    def timed(fn, reps):
        best = float("inf")
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            fn()
            b.record(s)
            b.synchronize()
            best = min(best, a.elapsed_time(b) / 1e3)
        return best

    out = {}
    dev = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    t = timed(lambda: L.ceiling_stream_read(dev.data_ptr(), dev.numel(), sink.data_ptr(), blocks,
                                            ctypes.c_void_p(s.cuda_stream)), 5)
    out["hbm_read_GBps"] = round(dev.numel() / t / 1e9, 1)
    L.ceiling_stream_read_nt.argtypes = L.ceiling_stream_read.argtypes
    L.ceiling_stream_read_nt.restype = ctypes.c_int
    t = timed(lambda: L.ceiling_stream_read_nt(dev.data_ptr(), dev.numel(), sink.data_ptr(),
                                               blocks, ctypes.c_void_p(s.cuda_stream)), 5)
    out["hbm_read_nontemporal_GBps"] = round(dev.numel() / t / 1e9, 1)
    del dev
    host = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    hp = device_pointer(host)
    t = timed(lambda: L.ceiling_stream_read(hp, host.numel(), sink.data_ptr(), blocks,
                                            ctypes.c_void_p(s.cuda_stream)), 3)
    out["host_link_zero_copy_read_GBps"] = round(host.numel() / t / 1e9, 1)
    dst = torch.empty(host.numel(), dtype=torch.uint8, device="cuda")
    t = timed(lambda: dst.copy_(host, non_blocking=True), 3)
    out["host_link_h2d_copy_GBps"] = round(host.numel() / t / 1e9, 1)
    del host, dst
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------- main --

def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the residency path runs on a single MI355X and the "
              f"library has no multi-GPU path (--gpus {args.gpus}, WORLD_SIZE {world}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import expert_weight_residency_amd as moe
    import synth
    from expert_weight_residency_amd.layer import ColdStage, LayerBuffers, enqueue_cold_ffn
    from expert_weight_residency_amd import mapfit
    from expert_weight_residency_amd.policy import (AdaptivePolicy, RuntimeControl, Telemetry,
                                                    restore_swaps, swaps_to)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    moe.lib()
    cold_path_default = args.cold_path is None
    if cold_path_default:
        args.cold_path = "staged" if args.workload == "prefill" else "inplace"
    if args.workload == "prefill":
        return run_prefill(args)
    if args.workload == "counter":
        return run_counter_cost(args)
    if args.workload == "swap":
        return run_swap_cost(args)
    lps, off_domain, shift, refit, wname = 1, False, False, False, None
    if args.workload == "step40":
        args.tokens, lps = 7, 40
        args.steps, args.warmup = min(args.steps, 32), min(args.warmup, 4)
        wname = "full_step_40_layers_t7"
    elif args.workload == "highconc":
        args.tokens = 112
        args.steps, args.warmup = min(args.steps, 64), min(args.warmup, 8)
        wname = f"full_layer_decode_t112_{args.map}_map"
    elif args.workload == "offdomain":
        # every layer bank runs on every step (as the layers of a model do), so each
        # bank's counter sees 64 x 7 x 6 picks per policy read
        args.tokens, off_domain, lps = 7, True, args.layers
        args.steps, args.warmup = 1536, min(args.warmup, 8)
        wname = f"off_domain_decode_t7_{args.layers}_layers"
    elif args.workload == "domainshift":
        # three equal phases: the map's own ranking (A), a second ranking (B), A again
        args.tokens, shift, lps = 7, True, args.layers
        args.steps, args.warmup = 1536, min(args.warmup, 8)
        wname = f"domain_shift_a_b_a_decode_t7_{args.layers}_layers"
    elif args.workload == "refit":
        # the off-domain boot, re-profiled and re-fitted off-line ("vLLM: Pin Hot
        # Experts", the count-only boot and the evening's off-line re-profile)
        args.tokens, off_domain, refit, lps = 7, True, True, args.layers
        args.steps, args.warmup = min(args.steps, 256), min(args.warmup, 8)
        args.no_policy = True
        wname = f"refit_off_domain_decode_t7_{args.layers}_layers"
    if args.cold_path == "dma" and args.graph:
        sys.exit("--cold-path dma reads the split back to the host every step: not capturable")
    if cold_path_default and args.tokens > HOST_KERNEL_MAX_TOKENS:
        # above 16 tokens the in-place cold FFN runs the operand-layout kernels,
        # which read host memory at ~40 GB/s; the staging copy runs at the link rate
        args.cold_path = "staged"
    E, k, H, I, T = 384, 6, 4096, 2880, args.tokens
    routing = args.routing
    if routing == "auto":
        routing = "window" if args.workload in ("step40", "highconc", "offdomain",
                                                 "domainshift", "refit") else "independent"
    n_cold = args.cold_rows
    if not 0 <= n_cold <= E:
        sys.exit(f"--cold-rows must be in [0, {E}]")
    n_hot = E - n_cold
    Lr, seed = args.layers, args.seed
    sz = synth.expert_sizes(H, I)
    b13, b2 = sz["w13"] + sz["s13"], sz["w2"] + sz["s2"]
    link_b, cold_hbm_b = cold_bytes_split(sz, args.cold_scales)
    log = lambda m: print(m, file=sys.stderr, flush=True)

    ceilings = {} if args.no_ceilings else measure_ceilings(torch)
    log(f"ceilings {ceilings}")

    # --- resident state: banks, maps, counters -------------------------------
    hot, cold, maps_dev, maps_host, hot_owner, cold_owner = [], [], [], [], [], []
    for l in range(Lr):
        rm, ho, co = (synth.fitted_map(E, n_cold, seed, l) if args.map == "fitted"
                      else synth.positional_map(E, n_cold))
        hb = moe.Bank(*[torch.empty(s, dtype=torch.uint8, device="cuda")
                        for s in synth.tensor_shapes(n_hot, H, I).values()], on_host=False)
        synth.fill_bank_device(hb.tensors(), torch.from_numpy(ho).cuda(), seed, l, H, I)
        cb = moe.Bank(*[torch.empty(s, dtype=torch.uint8, pin_memory=True)
                        for s in synth.tensor_shapes(n_cold, H, I).values()], on_host=True)
        synth.fill_bank_host(cb.tensors(), co, seed, l, H, I)
        hot.append(hb)
        cold.append(place_cold_scales(moe, cb, args.cold_scales))
        maps_host.append(rm.copy())
        maps_dev.append(torch.from_numpy(rm.copy()).cuda())
        hot_owner.append(ho.copy())
        cold_owner.append(co.copy())
    counts = torch.zeros((Lr, E), dtype=torch.int32, device="cuda")
    snap = torch.empty((Lr, E), dtype=torch.int32, pin_memory=True)
    staging = torch.empty(moe.moe_expert_bytes(H, I), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    log(f"{Lr} layer banks resident: {Lr * n_hot * (b13 + b2) / 2**30:.1f} GiB HBM, "
        f"{Lr * n_cold * (b13 + b2) / 2**30:.1f} GiB pinned host")

    # --- per-call inputs, generated and uploaded before timing ---------------
    # call c = step * lps + j runs on layer bank c % Lr; its routing follows that
    # bank's ranking (or, off-domain, an independent ranking of the same shape)
    # steps [0, prof): the count-only profile (refit); [prof, base): warm-up;
    # [base, S): timed
    prof = -(-args.profile_tokens // args.tokens) if refit else 0
    base = prof + args.warmup
    S = base + args.steps
    C = S * lps
    perms = [synth.layer_permutation(E, seed ^ 0x0FFD0 if off_domain else seed, l)
             for l in range(Lr)]
    perms_b = [synth.layer_permutation(E, seed ^ 0x0FFD0, l) for l in range(Lr)]
    phase_len = args.steps // 3

    def phase_of(c):  # domain-shift phase of layer call c: 0 (A), 1 (B), 2 (A)
        i = c // lps - base
        return 0 if i < phase_len else (1 if i < 2 * phase_len else 2)

    ids_np = np.empty((C, T, k), np.int32)
    w_np = np.empty((C, T, k), np.float32)
    NX = min(C, 64)
    x_np = np.empty((NX, T, H), np.uint16)
    def draw(l, c, pm):
        if routing == "window":
            return synth.window_routing(T, k, E, seed, l, c, perm=pm)
        return synth.skewed_routing(T, k, E, seed, l, c, perm=pm)

    # in-domain workloads on a fixed map: the timed calls of each layer bank
    # take their routing at evenly spaced quantiles (by distinct cold experts,
    # then distinct hot experts under the bank's boot map) of a draw four times
    # as large, in a seeded random order
    stratify = (not args.no_stratify and not (off_domain or shift or refit)
                and args.workload in ("decode", "highconc", "step40"))
    strat_info = None
    for c in range(C if not stratify else base * lps):
        pm = perms_b[c % Lr] if shift and phase_of(c) == 1 else perms[c % Lr]
        ids_np[c], w_np[c] = draw(c % Lr, c, pm)
    if stratify:
        rng_sel = np.random.default_rng([seed, 0x57A7])
        pool_cold, want = [], 0.0
        for l in range(Lr):
            calls = list(range(base * lps + ((l - base * lps) % Lr), C, Lr))
            if not calls:
                continue
            P = max(4 * len(calls), 64)
            pool = [draw(l, 1_000_000 + j, perms[l]) for j in range(P)]
            m = maps_host[l]
            key = []
            for j, (ids_j, _) in enumerate(pool):
                mm = m[ids_j]
                key.append((len(np.unique(ids_j[mm < 0])), len(np.unique(ids_j[mm >= 0])), j))
            key.sort()
            pool_cold.extend(kk[0] for kk in key)
            pick = [key[int((i + 0.5) * P / len(calls))][2] for i in range(len(calls))]
            rng_sel.shuffle(pick)
            for c, j in zip(calls, pick):
                ids_np[c], w_np[c] = pool[j]
        strat_info = {"method": "quantiles of distinct cold, then hot, experts in a 4x draw "
                                "per layer bank",
                      "expected_cold_experts_per_call": round(float(np.mean(pool_cold)), 3)}
    for c in range(NX):
        x_np[c] = synth.activations(T, H, seed, c % Lr, c)
    ids_d = torch.from_numpy(ids_np).cuda()
    w_d = torch.from_numpy(w_np).cuda()
    x_d = torch.from_numpy(x_np.view(np.int16)).cuda()
    bufs = LayerBuffers.allocate(T, k, H, I, n_hot, n_cold)
    stage = (ColdStage(min(n_cold, T * k), H, I, dma=args.cold_path == "dma")
             if args.cold_path in ("staged", "dma") else None)
    main_s = torch.cuda.Stream()
    side_s = main_s if args.serial else torch.cuda.Stream()
    # --streams cold-side: the cold path on the side stream; hot-side: the hot
    # FFN there and the cold path (the longer one in most decode steps) on the
    # main stream with the split and the finalize
    hot_s, cold_s = (side_s, main_s) if args.streams == "hot-side" else (main_s, side_s)
    policy = AdaptivePolicy(Lr, E)
    control = RuntimeControl(policy, args.ctrl)
    telemetry = Telemetry(args.telemetry)
    boot_hot = [h.copy() for h in hot_owner]
    swaps = stale = 0

    # hot-stream events of the timed steps, and every event of the profile pass
    ev = {name: [] for name in ("gu0", "gu1", "dn1")}  # gu1: the kernel_split_step steps
    pev = {name: [] for name in ("gu0", "gu1", "dn1", "c0", "c1", "s0", "s1")}
    bytes_step, hot_bytes_gu, cold_bytes, uh_list, uc_list, cold_picks = [], [], [], [], [], 0
    uh_first = []  # distinct hot experts of each step's first layer call (the timed one)

    def account(c, rm):
        ids = ids_np[c]
        m = rm[ids]
        hot_ids, cold_ids = ids[m >= 0], ids[m < 0]
        uh, uc = len(np.unique(hot_ids)), len(np.unique(cold_ids))
        ph, pc = hot_ids.size, cold_ids.size
        gu = uh * b13 + T * H * 2 + ph * I * 2
        dn = uh * b2 + ph * I * 2 + ph * H * 2
        cold_act = T * H * 2 + pc * I * 4 + pc * H * 2          # x read, h write+read, Y write
        fin = T * k * H * 2 + T * k * 4 + T * H * 2
        split = T * k * 4 + E * 4 + (T * k * 4) * 2
        return (gu, gu + dn + cold_act + fin + split + uc * cold_hbm_b, uc * link_b, uh, uc,
                pc)

    # Everything the timed loop records or waits on is created beforehand, so
    # the host work per step is the library calls themselves (the step must
    # stay bound by the device, not by the host enqueueing it).
    n_prof = 0 if args.graph else max(0, min(args.profile_steps, args.steps))
    ev_pool = [torch.cuda.Event(enable_timing=True)
               for _ in range(3 * args.steps + 7 * n_prof + 8)]

    def mark(name, stream):
        e = ev_pool.pop()
        e.record(stream)
        (pev if in_profile else ev)[name].append(e)

    in_profile = False  # set during the untimed profile pass

    fork_ev, join_hot_ev, join_cold_ev = torch.cuda.Event(), torch.cuda.Event(), torch.cuda.Event()

    def wait(dst, src, e):  # dst waits for the work enqueued on src so far
        e.record(src)
        dst.wait_event(e)

    def cold_ffn(xc, l, timed):
        full = timed and in_profile  # main-stream events only in the profile pass
        if full:
            mark("c0", cold_s)
        enqueue_cold_ffn(cold[l], bufs.cold_split, xc, k, H, I, bufs, stage, cold_s,
                         overlap=not args.serial)
        if full:
            mark("c1", cold_s)

    def step(s, timed):
        full = timed and in_profile
        if full:
            mark("s0", main_s)
        for j in range(lps):
            layer_call(s * lps + j, timed and j == 0)
        if full:
            mark("s1", main_s)

    def layer_call(c, timed, src=None):
        # hot_s runs the hot FFN, cold_s the cold path; the split and the
        # finalize are on main_s, which is one of the two (or both, --serial).
        # src: (ids, weights, x) tensors to read instead of call c's own
        # (the fixed buffers a captured graph reads)
        l = c % Lr
        ids_c, w_c, xc = src if src is not None else (ids_d[c], w_d[c], x_d[c % NX])
        moe.moe_route_split(ids_c, maps_dev[l], n_hot, n_cold, bufs.hot_split, bufs.cold_split,
                            bufs.n_invalid, counts[l] if control.counting else None, 256,
                            stream=main_s)
        if cold_s is not main_s:
            # cold bank first on its own stream: its 8 workgroups start beside the hot bank's
            wait(cold_s, main_s, fork_ev)
            cold_ffn(xc, l, timed)
        if hot_s is not main_s:
            wait(hot_s, main_s, fork_ev)
        if timed:
            mark("gu0", hot_s)
        moe.moe_expert_gate_up_mxfp4(hot[l], bufs.hot_split, xc, k, I, bufs.workspace,
                                     stream=hot_s)
        if timed and (in_profile or kernel_split_step(c // lps - base, args.steps)):
            mark("gu1", hot_s)
        moe.moe_expert_down_mxfp4(hot[l], bufs.hot_split, T, k, H, I, bufs.workspace, bufs.Y,
                                  stream=hot_s)
        if timed:
            mark("dn1", hot_s)
        if cold_s is main_s:
            cold_ffn(xc, l, timed)
        if hot_s is not main_s:
            wait(main_s, hot_s, join_hot_ev)
        if cold_s is not main_s:
            wait(main_s, cold_s, join_cold_ev)
        moe.moe_finalize(bufs.Y, w_c, bufs.out, stream=main_s)

    def apply_swaps(props):
        """Apply proposals between steps; returns (applied, refused as stale)."""
        nonlocal swaps, stale
        ok = bad = 0
        for sw in props:
            l = sw.layer
            try:
                moe.moe_swap_rows(hot[l], cold[l], sw.hot_row, sw.cold_row, sw.expect_hot_expert,
                                  sw.expect_cold_expert, maps_dev[l], hot_owner[l], cold_owner[l],
                                  staging, H, I, stream=main_s)
            except moe.MoeStale:
                bad += 1
                continue
            maps_host[l][sw.expect_hot_expert] = -1 - sw.cold_row
            maps_host[l][sw.expect_cold_expert] = sw.hot_row
            ok += 1
        swaps += ok
        stale += bad
        return ok, bad

    def barrier(step):
        unknown = control.poll()
        moe.moe_usage_counts(counts, snap, stream=main_s)
        main_s.synchronize()
        control.maybe_dump(snap.numpy())
        policy.observe(snap.numpy())
        if control.restore_pending:
            props = restore_swaps(hot_owner, cold_owner, boot_hot,
                                  limit=policy.cfg.swaps_per_barrier)
            if not props:
                control.restore_pending = False
        else:
            props = policy.decide(hot_owner, cold_owner)
        ok, bad = apply_swaps(props)
        telemetry.log(step=step, proposed=len(props), applied=ok, stale=bad,
                      frozen=policy.frozen, counting=control.counting,
                      restoring=control.restore_pending,
                      **({"unknown_ctrl_keys": unknown} if unknown else {}))

    def profile_and_refit():
        """Count-only profile over steps [0, prof) on the boot map (counter on,
        no swaps; snapshots at 8 slice boundaries), a map fitted to those
        counts (mapfit), and its swaps applied between steps."""
        nonlocal swaps
        n_slices = 8
        edges = [prof * (j + 1) // n_slices for j in range(n_slices)]

        def snapshot():
            moe.moe_usage_counts(counts, snap, stream=main_s)
            main_s.synchronize()
            return snap.numpy().copy()

        prev, slices = snapshot(), []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(prof):
            step(s, False)
            if s + 1 in edges:
                cur = snapshot()
                slices.append(mapfit.counts_between(prev, cur))
                prev = cur
                log(f"profile: {s + 1}/{prof} steps")
        torch.cuda.synchronize()
        t_prof = time.perf_counter() - t0
        total = mapfit.score(slices)
        floor = min(mapfit.MIN_TOKENS_PER_LAYER, prof * T)
        fitted = mapfit.fit_maps(total, n_cold, top_k=k, min_tokens=floor)
        boot_share = float(sum(total[l, cold_owner[l]].sum() for l in range(Lr)) / total.sum())
        changed = [mapfit.changed_cold(cold_owner[l], fitted[l].cold_owner) for l in range(Lr)]
        before = swaps
        t0 = time.perf_counter()
        props = swaps_to(hot_owner, cold_owner, [m.hot_owner for m in fitted])
        ok, bad = apply_swaps(props)
        torch.cuda.synchronize()
        t_apply = time.perf_counter() - t0
        swaps = before  # the timed run's own swap count stays that of the on-line policy
        # the swaps keep rows where they are, so compare hot sets, not row maps
        if bad or not all(set(hot_owner[l].tolist()) == set(fitted[l].hot_owner.tolist())
                          for l in range(Lr)):
            raise RuntimeError("the fitted map was not applied")
        info = {"profile_steps": prof, "profile_tokens_per_layer": prof * T,
                "floor_tokens_per_layer": floor,
                "profile_us_per_layer": round(t_prof * 1e6 / (prof * lps), 1),
                "boot_cold_share_of_profile": round(boot_share, 4),
                "fitted_cold_share_in_sample": round(mapfit.overall_cold_share(total, fitted), 4),
                "fitted_cold_share_leave_one_slice_out": [
                    round(x, 4) for x in mapfit.leave_one_out(slices, n_cold)],
                "cold_ids_changed_per_layer": round(float(np.mean(changed)), 1),
                "swaps_to_apply": ok, "apply_ms": round(t_apply * 1e3, 1),
                "device_maps_equal_host": all(
                    np.array_equal(maps_dev[l].cpu().numpy(), maps_host[l]) for l in range(Lr))}
        log(f"refit {info}")
        return info

    graph = None
    if args.graph:
        # one captured graph per step: every layer call reads fixed input
        # buffers, loaded before each replay; the banks, maps and counters it
        # reads are the live ones (swaps between steps update them in place)
        if lps % Lr:
            sys.exit("--graph needs every step to run each layer bank once "
                     "(layers per step a multiple of the rotated banks)")
        ids_st = torch.empty((lps, T, k), dtype=torch.int32, device="cuda")
        w_st = torch.empty((lps, T, k), dtype=torch.float32, device="cuda")
        x_st = torch.empty((lps, T, H), dtype=torch.int16, device="cuda")
        xsel = torch.tensor([[(s * lps + j) % NX for j in range(lps)] for s in range(S)],
                            dtype=torch.int64, device="cuda")

        def load_step(s):
            ids_st.copy_(ids_d[s * lps:(s + 1) * lps], non_blocking=True)
            w_st.copy_(w_d[s * lps:(s + 1) * lps], non_blocking=True)
            torch.index_select(x_d, 0, xsel[s], out=x_st)

        def static_step():
            for j in range(lps):
                layer_call(j, False, (ids_st[j], w_st[j], x_st[j]))

    with torch.cuda.stream(main_s):
        if refit:
            refit_info = profile_and_refit()
        for s in range(prof, base):
            step(s, False)
        torch.cuda.synchronize()
        if args.graph:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=main_s):
                static_step()
            torch.cuda.synchronize()
            log(f"captured one {lps}-layer step as a graph")

            def step(s, timed):  # noqa: F811 (the graph replaces the eager step)
                load_step(s)
                graph.replay()
        t0 = time.perf_counter()
        # the maps in force from each layer call on: the byte accounting runs
        # after the timed loop, on the map each call saw
        map_versions = [(0, [m.copy() for m in maps_host])]
        host_us, marks, win_t, win_swaps = [], [], t0, 0
        for i in range(args.steps):
            s = base + i
            h0 = time.perf_counter()
            step(s, True)
            host_us.append((time.perf_counter() - h0) * 1e6)
            if not args.no_policy and (s + 1) % policy.cfg.read_every == 0:
                before = swaps
                barrier(s + 1)
                if swaps != before:
                    map_versions.append(((s + 1) * lps, [m.copy() for m in maps_host]))
                win_swaps += swaps - before
            if (off_domain or shift) and (i + 1) % 128 == 0:
                torch.cuda.synchronize()
                now = time.perf_counter()
                marks.append((i, now - win_t, win_swaps))
                win_t, win_swaps = now, 0
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        # untimed profile pass: the first n_prof timed steps again, with events
        # on the main stream too (step boundaries, the cold path)
        in_profile = True
        for i in range(n_prof):
            step(base + i, True)
        torch.cuda.synchronize()
        in_profile = False
        prof_maps = [m.copy() for m in maps_host]

    starts = [v[0] for v in map_versions]
    cold_by_step = []
    for i in range(args.steps):
        s = base + i
        step_bytes = step_cold = 0
        for j in range(lps):
            c = s * lps + j
            maps = map_versions[bisect.bisect_right(starts, c) - 1][1]
            gu, tot, cb, uh, uc, pc = account(c, maps[c % Lr])
            step_bytes += tot
            if j == 0:
                hot_bytes_gu.append(gu)
                cold_bytes.append(cb)
                uh_first.append(uh)
            uh_list.append(uh)
            uc_list.append(uc)
            cold_picks += pc
            step_cold += pc
        bytes_step.append(step_bytes)
        cold_by_step.append(step_cold)
    windows = [{"steps": [i - 127, i + 1],
                **({"phase": "ABA"[phase_of((base + i) * lps)]} if shift else {}),
                "cold_share_of_picks": round(sum(cold_by_step[i - 127:i + 1]) / (128 * lps * T * k),
                                             4),
                "us_per_layer": round(dt * 1e6 / (128 * lps), 1),
                "swaps_applied": ws} for i, dt, ws in marks]

    K = args.steps
    ms_per_step = (t1 - t0) * 1e3 / K
    ms = lambda e, a, b: np.array([x.elapsed_time(y) for x, y in zip(e[a], e[b])])
    # the timed steps with a marker between the two hot kernels (split) and without
    split = np.array([kernel_split_step(i, args.steps) for i in range(len(ev["gu0"]))], bool)
    ev_split = {"gu0": [e for e, f in zip(ev["gu0"], split) if f], "gu1": ev["gu1"],
                "dn1": [e for e, f in zip(ev["dn1"], split) if f]}
    # the pair's steps: the others, less the first timed step when there are
    # more (it starts from the idle device the synchronize leaves, and alone
    # moved the pair of a 20-step run from 225.7 to ~230 us; the step time
    # keeps it)
    pair = ~split
    if pair.sum() > 1:
        pair[0] = False
    ev_pair = {"gu0": [e for e, f in zip(ev["gu0"], pair) if f],
               "dn1": [e for e, f in zip(ev["dn1"], pair) if f]}
    if not ev_pair["gu0"]:  # too few steps: the pair from the split steps
        ev_pair = ev_split
    gu_ms, dn_ms = ms(ev_split, "gu0", "gu1"), ms(ev_split, "gu1", "dn1")
    pair_ms = ms(ev_pair, "gu0", "dn1")
    pgu_ms, pdn_ms = ms(pev, "gu0", "gu1"), ms(pev, "gu1", "dn1")   # profile pass
    c_ms, st_ms = ms(pev, "c0", "c1"), ms(pev, "s0", "s1")

    def pct(v):  # p10 / median / p90 in microseconds
        return ({k: round(float(np.percentile(v, q) * 1e3), 1)
                 for k, q in (("p10", 10), ("p50", 50), ("p90", 90))} if len(v) else None)

    # domain shift: after the timed phases, queue a restore to the boot-time map
    # and apply it between (untimed) barriers, as the control file's restore_map does
    restore = None
    if shift and not args.no_policy:
        before, rounds = swaps, 0
        control.restore_pending = True
        with torch.cuda.stream(main_s):
            while control.restore_pending and rounds < 1000:
                barrier(-1)
                rounds += 1
        torch.cuda.synchronize()
        restore = {"swaps": swaps - before, "barriers": rounds,
                   "hot_sets_equal_boot": all(set(h.tolist()) == set(b.tolist())
                                              for h, b in zip(hot_owner, boot_hot)),
                   "device_maps_equal_host": all(
                       np.array_equal(maps_dev[l].cpu().numpy(), maps_host[l]) for l in range(Lr))}
    # per-kernel events exist only for eager steps (not inside a replayed graph)
    kern = len(gu_ms) > 0
    pair_steps = pair if pair.any() else split
    hot_bytes_gu_a = np.asarray(hot_bytes_gu, np.float64)[split] if kern else None
    has_cold = np.asarray(cold_bytes, np.float64)[split] > 0 if kern else None
    pair_cold = np.asarray(cold_bytes, np.float64)[pair_steps] > 0 if kern else None
    mean_us = lambda v: round(float(v.mean() * 1e3), 1) if len(v) else None
    achieved = float(hot_bytes_gu_a.sum() / (gu_ms.sum() / 1e3) / 1e9) if kern else None
    hot_ffn_bytes = (np.asarray(uh_first, np.float64)[pair_steps] * (b13 + b2) if kern
                     else None)
    achieved_hot = (float(hot_ffn_bytes.sum() / (pair_ms.sum() / 1e3) / 1e9)
                    if kern else None)
    value = float(np.mean(bytes_step) / (ms_per_step / 1e3) / 1e9)
    # cold bytes of the profile pass's steps (the same calls, on the maps at its time)
    prof_cold = np.array([account((base + i) * lps, prof_maps[((base + i) * lps) % Lr])[2]
                          for i in range(n_prof)], np.float64) if n_prof else np.zeros(0)
    cold_link = (float(prof_cold.sum() / max(c_ms.sum() / 1e3, 1e-12) / 1e9)
                 if len(c_ms) else None)
    cap_hot = min(n_hot, T * k)
    fam_gu, fam_dn = ffn_families(T, k, H, I, cap_hot)

    # HBM traffic of the gate/up kernel from committed rocprofv3 counter runs,
    # used only while the kernel's sources are the ones the counters were taken on
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "traffic_gate_up_full_layer_decode_t16.json")
    if os.path.exists(tpath):
        rec = json.load(open(tpath))
        if rec.get("source_sha256") == sources_sha256(rec.get("sources", [])):
            traffic = rec.get("bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wname or f"full_layer_decode_t{T}", "experts": E, "top_k": k,
                   "hidden": H, "layers_per_step": lps,
                   "traffic": ("off-domain" if off_domain else
                               "domain shift A-B-A" if shift else "in-domain"),
                   "routing": ("verify windows of 7" if routing == "window" else "independent"),
                   "intermediate": I, "tokens": T, "hot_rows": n_hot, "cold_rows": n_cold,
                   "weights": "mxfp4", "cold_bank": COLD_BANK[args.cold_path],
                   "cold_scales": args.cold_scales, "map": args.map,
                   "layer_banks_rotated": Lr, "cold_stream": not args.serial,
                   "streams": "serial" if args.serial else args.streams,
                   "graph": bool(args.graph), "policy": not args.no_policy,
                   "timed_routing": "stratified" if stratify else "independent draws"},
        "us_per_layer": round(ms_per_step * 1e3 / lps, 1),
        "tokens_per_s": round(T / (ms_per_step / 1e3), 1),
        # mean over all timed steps (wall clock) and the profile pass's
        # per-step events (each event there adds a few us to the step)
        "step_us": {"mean": round(ms_per_step * 1e3, 1),
                    "profile_pass_mean": mean_us(st_ms),
                    "profile_pass_median": (round(float(np.median(st_ms) * 1e3), 1)
                                            if len(st_ms) else None),
                    "profile_pass_steps": int(len(st_ms))},
        "hot_gate_up_us": mean_us(gu_ms),
        # the same launches split by whether the step staged cold rows beside them
        "hot_gate_up_us_by_step": ({"without_cold": mean_us(gu_ms[~has_cold]),
                                    "with_cold": mean_us(gu_ms[has_cold])} if kern else None),
        "hot_down_us": mean_us(dn_ms),
        "hot_gate_up_down_us": mean_us(pair_ms) if kern else None,
        "hot_gate_up_down_us_by_step": ({"without_cold": mean_us(pair_ms[~pair_cold]),
                                         "with_cold": mean_us(pair_ms[pair_cold])}
                                        if kern else None),
        "kernel_split_steps": int(split.sum()) if kern else 0,
        "kernel_pair_steps": int(pair_steps.sum()) if kern else 0,
        "cold_ffn_us": mean_us(c_ms),
        "hot_ffn_GBps": round(achieved_hot, 1) if kern else None,
        "kernels": {"hot_gate_up": fam_gu, "hot_down": fam_dn},
        "cold_link": {"achieved_GBps": round(cold_link, 1) if cold_link is not None else None,
                      "ceiling_GBps": ceilings.get("host_link_zero_copy_read_GBps"),
                      "nominal_GBps": NOMINAL_LINK_GBPS},
        "routing": {"hot_unique_per_step": round(float(np.mean(uh_list)), 2),
                    "cold_unique_per_step": round(float(np.mean(uc_list)), 2),
                    "cold_experts_timed": int(np.sum(uc_list)),
                    **({"cold_experts_expected": round(
                        strat_info["expected_cold_experts_per_call"] * K * lps, 1),
                        "stratified": strat_info["method"]} if strat_info else {}),
                    "cold_share_of_picks": round(cold_picks / (K * lps * T * k), 4)},
        "swaps_applied": swaps, "swaps_stale": stale,
        **({"windows": windows} if (off_domain or shift) else {}),
        **({"restore": restore} if restore else {}),
        **({"refit": refit_info} if refit else {}),
        "percentiles_us": {name: pct(v) for name, v in (("step_profile_pass", st_ms),
                                                        ("hot_gate_up", gu_ms),
                                                        ("hot_down", dn_ms),
                                                        ("hot_gate_up_down",
                                                         pair_ms if kern else []),
                                                        ("cold_path_profile_pass", c_ms))},
        # host time to enqueue one step (no waiting): it must stay below the
        # step's device time for the step to measure the device
        "host_enqueue_us": {k: round(float(np.percentile(host_us, q)), 1)
                            for k, q in (("p10", 10), ("p50", 50), ("p90", 90))},
        "ceilings": ceilings,
        "roofline": {"kernel": f"{fam_gu} (hot bank)", "bound": "hbm",
                     "achieved": round(achieved, 1) if kern else None, "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4) if kern else None,
                     "traffic": traffic if fam_gu == TRAFFIC_KERNEL else None},
        # the hot bank as a whole: gate/up + down algorithmic bytes (each
        # touched expert's 18.8 MB once) over the span from before gate/up to
        # after down, in the timed steps without a marker between the two
        "roofline_hot_bank": {"kernels": f"{fam_gu} + {fam_dn}", "bound": "hbm",
                              "achieved": round(achieved_hot, 1) if kern else None,
                              "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                              "frac": (round(achieved_hot / PEAK_HBM_GBPS, 4) if kern
                                       else None)},
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, ids_np, w_np, x_np, maps_host, Lr, H, I, E,
                                              b13 + b2, account, log, lps, first=base)
    print(json.dumps(result), flush=True)


# The kernel families the library picks for a device bank (the rule of
# launch_gate_up / launch_down in the library's ffn_mxfp4.hip, for H a
# multiple of 1024 and aligned scale tensors), named in the result.
TRAFFIC_KERNEL = "ffn_gate_up_resident"
# the largest step for which a bank in host memory runs the linear-read host
# kernels (kHostMaxTokens in the library)
HOST_KERNEL_MAX_TOKENS = 16


def ffn_families(T, k, H, I, cap):
    if T >= 256:
        return "ffn_fp4", "ffn_fp4"
    tiled = T * k >= 2 * cap
    gu = ("ffn_gate_up_resident" if T <= 16 and H % 1024 == 0 else
          "ffn_tiled" if tiled else "ffn_gate_up")
    n, wrb = -(-I // 256), I // 2
    aligned = n % 4 == 0 and max(r * wrb % 128 for r in range(8)) + wrb - 128 * (n - 1) <= 128
    dn = ("ffn_tiled" if tiled else
          "ffn_down_resident" if I % 32 == 0 and (n % 3 == 0 or aligned) else "ffn_down")
    return gu, dn


def sources_sha256(rel_paths):
    """sha256 over the named source files, in order (None if any is missing)."""
    h = hashlib.sha256()
    for rel in rel_paths:
        path = os.path.join(ROOT, rel)
        if not os.path.exists(path):
            return None
        h.update(open(path, "rb").read())
    return h.hexdigest() if rel_paths else None


def place_cold_scales(moe, cb, scales):
    """The filled cold bank (all pinned) as it is, or with its scale tensors
    moved to HBM and only the weights left on the host."""
    if scales == "host":
        return cb
    return moe.Bank(cb.w13, cb.s13.cuda(), cb.w2, cb.s2.cuda(), on_host=moe.BANK_HOST_WEIGHTS)


def cold_bytes_split(sz, scales):
    """(bytes of one cold expert that cross the host link, bytes it reads from HBM)."""
    w, sc = sz["w13"] + sz["w2"], sz["s13"] + sz["s2"]
    return (w + sc, 0) if scales == "host" else (w, sc)


def make_layer_banks(torch, moe, synth, E, n_cold, H, I, Lr, seed, map_kind="fitted",
                     cold_scales="host"):
    """Per layer: hot bank (HBM, device-filled), cold bank (pinned host), maps."""
    n_hot = E - n_cold
    hot, cold, maps_host = [], [], []
    for l in range(Lr):
        rm, ho, co = (synth.fitted_map(E, n_cold, seed, l) if map_kind == "fitted"
                      else synth.positional_map(E, n_cold))
        hb = moe.Bank(*[torch.empty(s, dtype=torch.uint8, device="cuda")
                        for s in synth.tensor_shapes(n_hot, H, I).values()], on_host=False)
        synth.fill_bank_device(hb.tensors(), torch.from_numpy(ho).cuda(), seed, l, H, I)
        cb = moe.Bank(*[torch.empty(s, dtype=torch.uint8, pin_memory=True)
                        for s in synth.tensor_shapes(n_cold, H, I).values()], on_host=True)
        synth.fill_bank_host(cb.tensors(), co, seed, l, H, I)
        hot.append(hb)
        cold.append(place_cold_scales(moe, cb, cold_scales))
        maps_host.append(rm.copy())
    return hot, cold, maps_host


def run_counter_cost(args):
    """The counter's cost ("Should a GB300 Prefetch Its Cold Experts?", section
    8, E1): moe_route_split for 40 layers captured in one HIP graph, once with
    the usage counter and once without, at 6, 16 and 32 tokens per step
    (top-6, 384 experts, each layer its own fitted map and skewed routing).
    The two graphs are replayed alternately; the difference of their median
    replay times is the counter's cost per 40-layer step. The counter table
    is checked afterwards: every replay added exactly the step's histogram."""
    import torch

    import expert_weight_residency_amd as moe
    import synth

    E, k, L, seed = 384, 6, 40, args.seed
    reps = max(50, min(args.steps, 400))
    log = lambda m: print(m, file=sys.stderr, flush=True)
    maps = [synth.fitted_map(E, args.cold_rows, seed, l) for l in range(L)]
    n_hot, n_cold = E - args.cold_rows, args.cold_rows
    maps_dev = [torch.from_numpy(m[0].copy()).cuda() for m in maps]
    s = torch.cuda.Stream()
    out = {}
    for T in (6, 16, 32):
        ids = [synth.skewed_routing(T, k, E, seed, l, 0)[0] for l in range(L)]
        ids_d = [torch.from_numpy(i).cuda() for i in ids]
        hs, cs = moe.Split.empty(n_hot, T, k), moe.Split.empty(n_cold, T, k)
        ninv = torch.zeros(1, dtype=torch.int32, device="cuda")
        counts = torch.zeros((L, E), dtype=torch.int32, device="cuda")

        def body(with_counter):
            for l in range(L):
                moe.moe_route_split(ids_d[l], maps_dev[l], n_hot, n_cold, hs, cs, ninv,
                                    counts[l] if with_counter else None, 256, stream=s)

        graphs = {}
        with torch.cuda.stream(s):
            for wc in (True, False):
                body(wc)  # eager warm-up
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    body(wc)
                graphs[wc] = g
            torch.cuda.synchronize()
            counts.zero_()
            torch.cuda.synchronize()
            times = {True: [], False: []}
            for r in range(reps + 10):
                for wc in (True, False):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(s)
                    graphs[wc].replay()
                    b.record(s)
                    if r >= 10:
                        times[wc].append((a, b))
            torch.cuda.synchronize()
        med = {wc: float(np.median([a.elapsed_time(b) for a, b in v]) * 1e3)
               for wc, v in times.items()}
        hist = np.stack([np.bincount(i.ravel(), minlength=E) for i in ids])
        exact = bool(np.array_equal(counts.cpu().numpy(), hist * (reps + 10)))
        d = med[True] - med[False]
        out[f"T{T}"] = {"picks_per_layer": T * k,
                        "us_per_40_layers_with_counter": round(med[True], 1),
                        "us_per_40_layers_without": round(med[False], 1),
                        "counter_us_per_40_layers": round(d, 1),
                        "counter_us_per_layer": round(d / L, 3),
                        "share_of_14_6_ms_step_pct": round(100 * d / 14600.0, 3),
                        "counts_exact": exact}
        log(f"T={T}: {out[f'T{T}']}")
    result = {"metric": "usage counter cost (split kernel, 40 layers in a HIP graph)",
              "value": out["T16"]["counter_us_per_40_layers"], "unit": "us per 40-layer step",
              "n_gpus": 1, "steps": reps, "warmup": 10, "higher_is_better": False,
              "dtype": "int32", "data": "synthetic",
              "config": {"workload": "counter_cost_split_40_layers", "experts": E, "top_k": k,
                         "layers": L, "hot_rows": n_hot, "cold_rows": n_cold,
                         "map": "fitted", "graph": True},
              "by_tokens": out}
    print(json.dumps(result), flush=True)


def run_swap_cost(args):
    """Full-size true swaps ("vLLM: Pin Hot Experts", "Closed, September 17
    evening": a hot row to a staging row, the cold row into the hot slot, the
    staging row into the cold slot, then the two-element map write) between a
    295-row HBM bank and an 89-row pinned host bank at H = 4096, I = 2880,
    timed one by one with events on the stream. Each swap moves one expert
    (18.8 MB) each way over the host link and one through HBM."""
    import torch

    import expert_weight_residency_amd as moe
    import synth

    E, H, I, seed = 384, 4096, 2880, args.seed
    n = max(8, min(args.steps, 64))
    rm, ho, co = synth.fitted_map(E, args.cold_rows, seed, 0)
    shapes = synth.tensor_shapes(len(ho), H, I)
    hot = moe.Bank(*[torch.empty(s, dtype=torch.uint8, device="cuda") for s in shapes.values()])
    synth.fill_bank_device(hot.tensors(), torch.from_numpy(ho).cuda(), seed, 0, H, I)
    cold = moe.Bank(*[torch.empty(s, dtype=torch.uint8, pin_memory=True)
                      for s in synth.tensor_shapes(len(co), H, I).values()], on_host=True)
    synth.fill_bank_host(cold.tensors(), co, seed, 0, H, I)
    rm_dev = torch.from_numpy(rm.copy()).cuda()
    staging = torch.empty(moe.moe_expert_bytes(H, I), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    rng = np.random.default_rng(seed)
    ev = []
    with torch.cuda.stream(s):
        for i in range(n + 2):
            a, b = int(rng.integers(len(ho))), int(rng.integers(len(co)))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            moe.moe_swap_rows(hot, cold, a, b, int(ho[a]), int(co[b]), rm_dev, ho, co, staging,
                              H, I, stream=s)
            e1.record(s)
            if i >= 2:
                ev.append((e0, e1))
        torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    eb = moe.moe_expert_bytes(H, I)
    result = {"metric": "row swap time (full-size expert, hot HBM <-> cold pinned host)",
              "value": round(float(np.median(us)), 1), "unit": "us per swap", "n_gpus": 1,
              "steps": n, "warmup": 2, "higher_is_better": False, "dtype": "u8",
              "data": "synthetic",
              "config": {"workload": "swap_full_size", "experts": E, "hidden": H,
                         "intermediate": I, "hot_rows": len(ho), "cold_rows": len(co),
                         "expert_bytes": eb},
              "us_per_swap": {"p10": round(float(np.percentile(us, 10)), 1),
                              "p50": round(float(np.median(us)), 1),
                              "p90": round(float(np.percentile(us, 90)), 1)},
              "host_link_GBps_both_directions": round(2 * eb / (np.median(us) * 1e-6) / 1e9, 1),
              "maps_equal": bool(np.array_equal(
                  rm_dev.cpu().numpy()[np.concatenate([ho, co])],
                  np.concatenate([np.arange(len(ho)), -1 - np.arange(len(co))])))}
    print(json.dumps(result), flush=True)


def run_prefill(args):
    """One 4096-token prefill chunk of the full layer per step: split (counter
    off: more than 256 tokens), hot FFN on the main stream, cold FFN on a side
    stream, finalize. The hot bank runs the FP4-instruction kernels; their MFMA
    utilisation is reported against half the dense fp8 peak (two terms per
    activation), and their HBM rate
    against 8 TB/s."""
    import torch

    import expert_weight_residency_amd as moe
    import synth
    from expert_weight_residency_amd.layer import ColdStage, LayerBuffers, enqueue_cold_ffn

    E, k, H, I, T = 384, 6, 4096, 2880, 4096
    n_cold = args.cold_rows
    if not 0 <= n_cold <= E:
        sys.exit(f"--cold-rows must be in [0, {E}]")
    n_hot = E - n_cold
    Lr, seed = min(args.layers, 2), args.seed
    sz = synth.expert_sizes(H, I)
    b13, b2 = sz["w13"] + sz["s13"], sz["w2"] + sz["s2"]
    log = lambda m: print(m, file=sys.stderr, flush=True)
    steps, warmup = min(args.steps, 16), min(args.warmup, 2)
    hot, cold, maps_host = make_layer_banks(torch, moe, synth, E, n_cold, H, I, Lr, seed, args.map,
                                            args.cold_scales)
    link_b, _ = cold_bytes_split(sz, args.cold_scales)
    maps_dev = [torch.from_numpy(m.copy()).cuda() for m in maps_host]
    S = warmup + steps
    ids_np = np.empty((S, T, k), np.int32)
    w_np = np.empty((S, T, k), np.float32)
    x_d = torch.empty((S, T, H), dtype=torch.int16, device="cuda")
    for s in range(S):
        ids_np[s], w_np[s] = synth.skewed_routing(T, k, E, seed, s % Lr, s)
        x_d[s] = torch.from_numpy(synth.activations(T, H, seed, s % Lr, s).view(np.int16)).cuda()
    ids_d = torch.from_numpy(ids_np).cuda()
    w_d = torch.from_numpy(w_np).cuda()
    bufs = LayerBuffers.allocate(T, k, H, I, n_hot, n_cold)
    stage = (ColdStage(min(n_cold, T * k), H, I, dma=args.cold_path == "dma")
             if args.cold_path in ("staged", "dma") else None)
    main_s = torch.cuda.Stream()
    cold_s = main_s if args.serial else torch.cuda.Stream()
    torch.cuda.synchronize()
    log(f"prefill: {Lr} layer banks resident, {S} steps of inputs uploaded")

    ev = {n: [] for n in ("gu0", "gu1", "dn1", "c0", "c1")}

    def rec(name, stream):
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        ev[name].append(e)

    def step(s, timed):
        l = s % Lr
        moe.moe_route_split(ids_d[s], maps_dev[l], n_hot, n_cold, bufs.hot_split,
                            bufs.cold_split, bufs.n_invalid, None, 256, stream=main_s)
        if cold_s is not main_s:
            cold_s.wait_stream(main_s)
        if timed:
            rec("gu0", main_s)
        moe.moe_expert_gate_up_mxfp4(hot[l], bufs.hot_split, x_d[s], k, I, bufs.workspace,
                                     stream=main_s)
        if timed:
            rec("gu1", main_s)
        moe.moe_expert_down_mxfp4(hot[l], bufs.hot_split, T, k, H, I, bufs.workspace, bufs.Y,
                                  stream=main_s)
        if timed:
            rec("dn1", main_s)
            rec("c0", cold_s)
        enqueue_cold_ffn(cold[l], bufs.cold_split, x_d[s], k, H, I, bufs, stage, cold_s,
                         overlap=cold_s is not main_s)
        if timed:
            rec("c1", cold_s)
        if cold_s is not main_s:
            main_s.wait_stream(cold_s)
        moe.moe_finalize(bufs.Y, w_d[s], bufs.out, stream=main_s)

    with torch.cuda.stream(main_s):
        for s in range(warmup):
            step(s, False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(warmup + i, True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()

    ms = (t1 - t0) * 1e3 / steps
    gu = np.array([a.elapsed_time(b) for a, b in zip(ev["gu0"], ev["gu1"])]) / 1e3
    dn = np.array([a.elapsed_time(b) for a, b in zip(ev["gu1"], ev["dn1"])]) / 1e3
    cf = np.array([a.elapsed_time(b) for a, b in zip(ev["c0"], ev["c1"])]) / 1e3
    uh, uc, ph, pc = [], [], [], []
    for i in range(steps):
        s = warmup + i
        m = maps_host[s % Lr][ids_np[s]]
        uh.append(len(np.unique(ids_np[s][m >= 0])))
        uc.append(len(np.unique(ids_np[s][m < 0])))
        ph.append(int((m >= 0).sum()))
        pc.append(int((m < 0).sum()))
    uh, uc, ph, pc = map(np.array, (uh, uc, ph, pc))
    fl_gu = 2.0 * ph * (2 * I) * H          # gate/up flops per step (hot)
    fl_dn = 2.0 * ph * H * I
    # the contraction runs on the block-scaled FP4 instruction with each bf16
    # activation carried as two E4M3 terms: two fp8-rate MFMAs per product,
    # so the algorithmic flops are priced at half the 5.0 PFLOP/s fp8 peak
    peak_fp4x2 = 5000.0 / 2
    tf_gu = float(fl_gu.sum() / gu.sum() / 1e12)
    tf_dn = float(fl_dn.sum() / dn.sum() / 1e12)
    tf_hot = float((fl_gu + fl_dn).sum() / (gu + dn).sum() / 1e12)
    hbm_hot = float((uh * (b13 + b2)).sum() / (gu + dn).sum() / 1e9)
    bytes_step = uh * (b13 + b2) + T * H * 2 * 2 + (ph + pc) * (I * 4 + H * 4) + T * H * 2
    result = {
        "metric": METRIC,
        "value": round(float(np.mean(bytes_step) / (ms / 1e3) / 1e9), 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"full_layer_prefill_t{T}", "experts": E, "top_k": k,
                   "hidden": H, "intermediate": I, "tokens": T, "hot_rows": n_hot,
                   "cold_rows": n_cold, "weights": "mxfp4", "cold_bank": COLD_BANK[args.cold_path],
                   "cold_scales": args.cold_scales,
                   "map": args.map, "layer_banks_rotated": Lr, "counter": False,
                   "cold_stream": not args.serial},
        "us_per_layer": round(ms * 1e3, 1),
        "tokens_per_s": round(T / (ms / 1e3), 1),
        "hot_gate_up_us": round(float(gu.mean() * 1e6), 1),
        "hot_down_us": round(float(dn.mean() * 1e6), 1),
        "cold_ffn_us": round(float(cf.mean() * 1e6), 1),
        "hot_us": round(float((gu + dn).mean() * 1e6), 1),
        "hot_tokens_per_s": round(float(T / (gu + dn).mean()), 1),
        # the dominant kernels of a prefill step, against the matrix peak
        "roofline": {"kernel": "ffn_fp4 (hot bank, gate/up + down, activation split included)",
                     "bound": "mfma", "achieved": round(tf_hot, 1), "peak": peak_fp4x2,
                     "unit": "TFLOP/s", "frac": round(tf_hot / peak_fp4x2, 4),
                     "traffic": None,
                     "gate_up_TFLOPs": round(tf_gu, 1),
                     "down_TFLOPs": round(tf_dn, 1)},
        "hot_hbm": {"achieved": round(hbm_hot, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": round(hbm_hot / PEAK_HBM_GBPS, 4)},
        "cold_link_GBps": round(float((uc * link_b).sum() / cf.sum() / 1e9), 1),
        "routing": {"hot_unique_per_step": round(float(uh.mean()), 2),
                    "cold_unique_per_step": round(float(uc.mean()), 2),
                    "cold_share_of_picks": round(float(pc.sum() / (ph + pc).sum()), 4)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_prefill(args, ids_np[warmup], w_np[warmup],
                                                      warmup % Lr, H, I, E, ms, log)
    print(json.dumps(result), flush=True)


def cpu_baseline_prefill(args, ids, w, layer, H, I, E, gpu_ms, log):
    """The oracle on the first 48 tokens of one timed prefill step (all their
    picks, hot and cold, plus finalize), scaled linearly to the 4096 tokens."""
    import oracle
    import synth
    n = 48
    ids, w = ids[:n], w[:n]
    x = synth.activations(4096, H, args.seed, layer, args.warmup)[:n]
    U = np.unique(ids)
    bank = oracle.Bank(**synth.make_bank_host(U, args.seed, layer, H, I))
    rm = np.full(E, -(10 ** 6), np.int32)
    rm[U] = np.arange(len(U), dtype=np.int32)
    t0 = time.perf_counter()
    oracle.moe_layer(bank, None, rm, ids, w, x, H, I)
    dt = time.perf_counter() - t0
    per_step = dt * 4096 / n
    return {"value": round(4096 / per_step, 2), "unit": "tokens/s", "cores": oracle.max_threads(),
            "kind": "oracle", "ms_per_step": round(per_step * 1e3, 1), **host_cpu_info(),
            "gpu_tokens_per_s": round(4096 / (gpu_ms / 1e3), 1),
            "sample": f"first {n} of the 4096 tokens of one timed step ({ids.size} picks, hot "
                      "and cold, plus finalize), time scaled by 4096/48"}


def host_cpu_info():
    """CPU model, physical cores and logical CPUs of this host, and the CPUs
    this process may run on (from /proc/cpuinfo and the affinity mask)."""
    model, cores, logical = None, set(), 0
    try:
        phys = core = None
        for line in open("/proc/cpuinfo"):
            key, _, val = line.partition(":")
            key, val = key.strip(), val.strip()
            if key == "processor":
                logical += 1
            elif key == "model name" and model is None:
                model = val
            elif key == "physical id":
                phys = val
            elif key == "core id":
                core = val
                cores.add((phys, core))
    except OSError:
        pass
    return {"cpu_model": model, "physical_cores": len(cores) or None, "logical_cpus": logical,
            "usable_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline(args, ids_np, w_np, x_np, maps_host, Lr, H, I, E, bexp, account, log, lps=1,
                 first=None):
    """The oracle on sampled steps of the same workload (whole layer: all picks,
    hot and cold, plus finalize), until about 10 s of CPU time, on all the
    threads OpenMP gives it; then on one thread, over the first picks of one
    step (about 5 s), scaled to the whole layer."""
    import oracle
    import synth
    t_tot, b_tot, n = 0.0, 0.0, 0
    first = args.warmup if first is None else first
    for s in range(first, first + min(args.steps, 4)):
        c = s * lps  # the step's first layer call
        l = c % Lr
        ids = ids_np[c]
        U = np.unique(ids)
        bank = oracle.Bank(**synth.make_bank_host(U, args.seed, l, H, I))
        rm = np.full(E, -(10 ** 6), np.int32)
        rm[U] = np.arange(len(U), dtype=np.int32)
        t0 = time.perf_counter()
        oracle.moe_layer(bank, None, rm, ids, w_np[c], x_np[c % len(x_np)], H, I)
        t_tot += time.perf_counter() - t0
        b_tot += account(c, maps_host[l])[1]
        n += 1
        if t_tot > 10.0:
            break
    per = t_tot / n
    threads = oracle.max_threads()
    # one thread: the first tokens of the first sampled step, about 1/8 of its
    # picks (at least one token), time scaled by picks
    c = first * lps
    T_all, k = ids_np.shape[1], ids_np.shape[2]
    t1 = max(1, T_all // 8)
    ids1 = ids_np[c][:t1]
    U = np.unique(ids1)
    bank = oracle.Bank(**synth.make_bank_host(U, args.seed, c % Lr, H, I))
    rm = np.full(E, -(10 ** 6), np.int32)
    rm[U] = np.arange(len(U), dtype=np.int32)
    t0 = time.perf_counter()
    oracle.moe_layer(bank, None, rm, ids1, w_np[c][:t1], x_np[c % len(x_np)][:t1], H, I,
                     nthreads=1)
    per1 = (time.perf_counter() - t0) * T_all / t1
    return {"value": round(b_tot / n / per / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "us_per_layer": round(per * 1e6, 1),
            "us_per_layer_1core": round(per1 * 1e6, 1),
            **host_cpu_info(),
            "sample": f"{n} of the timed steps (one full layer each: all {T_all} tokens x "
                      f"{k} picks, hot and cold, plus finalize; same weights, routing and "
                      f"activations) on {threads} OpenMP threads; the 1-core figure: the first "
                      f"{t1} tokens ({t1 * k} picks) of one step on one thread, scaled by "
                      f"{T_all}/{t1}"}


if __name__ == "__main__":
    main()
