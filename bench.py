#!/usr/bin/env python3
"""KDA benchmark on one MI355X.

Headline workload (one "step" = one pass of the hot path over one batch):
batched decode, B = 64 sequences x H = 32 heads, d_k = d_v = 128, bf16
q/k/v/beta, fp32 log_alpha and fp32 state; one step advances every sequence
by one token (kda_decode_step over all 2048 head states).  The default run
times 1024 consecutive steps, the length of the workload.  ``value`` is decode
tokens/s (64 tokens per step) with all inputs already resident in HBM.

Also reported (same JSON line), each timed with HIP events:
  * the roofline of the decode kernel (algorithmic bytes per launch over the
    measured average launch duration, against 8 TB/s), and the same decode at
    B = 256 (512 MiB of state, twice the last-level cache);
  * the chunked-prefill workload (B = 1, H = 32, T = 32768, bf16 inputs,
    gated channel mix): tokens/s and roofline;
  * the million-token prefill (B = 1, H = 32, T = 1,048,576, the same
    distributions), the packed prefill of 16 sequences with log-uniform
    lengths in [1024, 65536], half resumed from states, and the small fp32
    prefill (B = 1, H = 1, T = 256);
  * the backward pass (gradients of a prefill) at a training shape,
    B = 8 x T = 4096, H = 32;
  * the fp64 CPU oracle on the host cores: a bounded sample of the decode
    workload on every core, and a 4096-token slice of the chunked-prefill
    workload on one thread.

    python bench.py [--gpus 1] [--steps 1024] [--warmup 32] [--no-prefill]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/sec & decode tokens/sec; % MFMA peak / % HBM BW peak"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
D = 128

# Algorithmic bytes per head of one decode step: the fp32 state read once and
# written once (2 x 64 KiB), q and k (bf16, 256 B each), v (bf16, 256 B),
# beta (bf16, 2 B), log_alpha (fp32, 512 B), o (fp32, 512 B).
DECODE_BYTES_PER_HEAD = 2 * D * D * 4 + 2 * D * 2 + D * 2 + 2 + D * 4 + D * 4
# Prefill, per head-token: q, k, v (bf16), beta (bf16), log_alpha (fp32), o (fp32);
# plus the final state once per head.
PREFILL_BYTES_PER_HEAD_TOKEN = 3 * D * 2 + 2 + D * 4 + D * 4
# Chunked-algorithm flops per head-token at chunk 64 (d_k = d_v = 128).
PREFILL_FLOPS_PER_HEAD_TOKEN = 9_024_853 / 64
# Backward (bf16 inputs, the chunked form), per head-token: reads q, k, v
# (bf16), beta (bf16), log_alpha and d_o (fp32); writes dq, dk, dv, d log_alpha
# (fp32) and d beta (fp32).
BACKWARD_BYTES_PER_HEAD_TOKEN = 3 * D * 2 + 2 + 2 * D * 4 + 4 * D * 4 + 4
# Its matrix products per 64-token chunk and head (C = 64, d = 128, a
# multiply-add counted as 2): eight C x d x d products (the recomputed
# X = Kt S0 and leaving state, Ke dS1, Qt^T dO, Kt^T B dW', dQt, dKt, dKe) and
# twelve C x C x d ones (the recomputed A, P and U; P^T dO, T^T dU, dP, dT,
# dM = -T^T dT T^T, and the dA / dP terms of dq and dk).
BACKWARD_FLOPS_PER_HEAD_TOKEN = (8 * 2 * 64 * D * D + 12 * 2 * 64 * 64 * D) / 64


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024, help="timed decode steps")
    ap.add_argument("--warmup", type=int, default=32, help="untimed decode steps first")
    ap.add_argument("--batch", type=int, default=64)
    ap.add_argument("--heads", type=int, default=32)
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill measurement")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass measurement")
    ap.add_argument("--backward-reps", type=int, default=5)
    ap.add_argument("--no-raw", action="store_true",
                    help="skip the prefill from raw projections (same kernels: keeps kernel traces to one kind)")
    ap.add_argument("--no-tokens", action="store_true",
                    help="skip the multi-token (speculative verify / commit) decode measurement")
    ap.add_argument("--no-slots", action="store_true",
                    help="skip the decode measurement with the states in a slot-addressed pool")
    ap.add_argument("--eager", action="store_true",
                    help="time direct decode calls instead of a replayed HIP graph of them")
    ap.add_argument("--prefill-T", type=int, default=32768)
    ap.add_argument("--prefill-reps", type=int, default=10)
    ap.add_argument("--prefill-warmup", type=int, default=30,
                    help="untimed prefill calls first: right after the decode section the first "
                         "~30 calls run up to 25%% slower while the GPU settles")
    ap.add_argument("--cpu-steps", type=int, default=512,
                    help="decode steps of the workload the CPU oracle runs (all heads, every core)")
    ap.add_argument("--no-million", action="store_true", help="skip the million-token prefill")
    ap.add_argument("--no-varlen", action="store_true", help="skip the packed prefill")
    ap.add_argument("--no-small", action="store_true", help="skip the small fp32 prefill")
    ap.add_argument("--no-large-decode", action="store_true", help="skip the B = 256 decode")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB "
                         "(a reference kernel for the HBM byte counters)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_traffic(summary: str, kernel: str):
    """HBM bytes per launch of `kernel` from a committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, scaled by a reference copy), or None
    when there is none or the kernel's sources changed since it was taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", summary)
    try:
        with open(path) as f:
            rec = json.load(f)["kernels"][kernel]
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
    except (OSError, KeyError, ValueError):
        return None
    return rec["traffic_bytes_per_launch"] if h.hexdigest() == rec["sources_sha256"] else None


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads and sequences would shard across GPUs with no exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import gated_delta_rule_113_amd as kda
    import kda_inputs as ki

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    kda.load_library()
    B, H, K, W = args.batch, args.heads, args.steps, args.warmup

    # ---------------- decode: inputs resident in HBM -----------------------
    n_gen = max(K, W, 1)
    log(f"generating {n_gen} decode steps for B={B} H={H}")
    t0 = time.time()
    inp = ki.decode_steps(1, steps=n_gen, N=B, H=H)
    log(f"generated in {time.time() - t0:.1f}s; uploading")

    def up(x, bf16):
        if bf16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    q, k, v, beta = (up(x, True) for x in (inp.q, inp.k, inp.v, inp.beta))
    la = up(inp.log_alpha, False)
    state0 = up(inp.initial_state, False)
    state = state0.clone()
    o = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    if args.copy_mib > 0:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"reference copy: {args.copy_mib} MiB read + {args.copy_mib} MiB written")
        del src, dst

    def step(s, st):
        kda.kda_decode_step(q[s], k[s], v[s], beta[s], la[s], st, out=o)

    # The timed steps are captured once into a HIP graph and replayed, so the
    # per-call host cost of the Python binding does not leave the GPU idle
    # between steps (the decode entry point allocates nothing and issues only
    # its kernel, so it can be captured).  --eager times direct calls instead.
    graph = None
    if not args.eager:
        try:
            side = torch.cuda.Stream(dev)
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                step(0, state)  # warm the binding on the capture stream
            stream.wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for s in range(K):
                    step(s % n_gen, state)
            torch.cuda.synchronize()
        except Exception as e:  # fall back to direct calls
            log(f"graph capture failed ({e}); timing direct calls")
            graph = None

    def run_steps(count, first=0):
        if graph is not None and count == K and first == 0:
            graph.replay()
        else:
            for s in range(first, first + count):
                step(s % n_gen, state)

    log(f"warmup {W} steps")
    run_steps(W)
    if graph is not None:
        graph.replay()  # one untimed replay of the captured steps
    torch.cuda.synchronize()
    state.copy_(state0)
    torch.cuda.synchronize()

    log(f"timing {K} steps ({'graph replay' if graph is not None else 'direct calls'})")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    run_steps(K)
    ev1.record(stream)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    ms_per_step = total_ms / K
    tokens_per_s = B * K / (total_ms / 1e3)
    bytes_per_launch = DECODE_BYTES_PER_HEAD * B * H
    achieved = bytes_per_launch / (ms_per_step / 1e3) / 1e9
    if not bool(torch.isfinite(state).all()):
        raise RuntimeError("decode produced non-finite states")
    log(f"decode: {ms_per_step * 1e3:.2f} us/step, {tokens_per_s / 1e6:.3f} M tokens/s, "
        f"{achieved:.0f} GB/s")

    # Streaming ceiling for context: an in-place read-modify-write of the same
    # state tensor (the same 128 MiB of live, random-valued state read and
    # written once; scaling by 1 leaves it unchanged).  HBM throughput on this
    # part depends on the data: zero-filled buffers stream markedly faster.
    ceil_reps = 64
    state.mul_(1.0)
    torch.cuda.synchronize()
    ec0 = torch.cuda.Event(enable_timing=True)
    ec1 = torch.cuda.Event(enable_timing=True)
    ec0.record(stream)
    for _ in range(ceil_reps):
        state.mul_(1.0)
    ec1.record(stream)
    torch.cuda.synchronize()
    ceil_ms = ec0.elapsed_time(ec1) / ceil_reps
    ceil_gbs = 2 * B * H * D * D * 4 / (ceil_ms / 1e3) / 1e9
    log(f"state read-modify-write ceiling: {ceil_ms * 1e3:.2f} us ({ceil_gbs:.0f} GB/s); "
        f"decode reaches {achieved / ceil_gbs * 100:.0f}% of it")

    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded: bf16 L2-normalised q/k, N(0,1) v, sigmoid beta, "
                "-softplus log_alpha, N(0,0.02^2) fp32 states)",
        "config": {
            "workload": f"batched KDA decode: B={B} sequences x H={H} heads, d_k=d_v=128, "
                        "bf16 q/k/v/beta, fp32 log_alpha/state/o, consecutive single-token steps",
            "global_batch": B, "heads": H, "d_k": D, "d_v": D, "seq_len": 1,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic("decode_B64_H32_hbm_traffic.json", "decode_step_kernel<bf16_t>"),
            "kernel": "decode_step_kernel<bf16_t>",
            "algorithmic_bytes_per_launch": bytes_per_launch,
            "avg_launch_ms_timed_region": ms_per_step,
            "timed_region": "graph replay of the timed steps" if graph is not None else "direct calls",
            "state_bytes": B * H * D * D * 4,
            "note": "the 128 MiB of state fit in the 256 MB last-level (Infinity) cache, so across "
                    "consecutive steps part of the state stream is served from it",
        },
        "state_rmw_ceiling": {
            "what": "torch in-place scale by 1 of the live state tensor: the state bytes read and "
                    "written once, no other work",
            "us": ceil_ms * 1e3,
            "GBps": ceil_gbs,
            "decode_frac_of_ceiling": achieved / ceil_gbs,
        },
    }

    # ---------------- decode with the states in a pool (secondary) ---------
    # The same B x H decode, but the states live in a pool of 4B entries and
    # each sequence names its entry by an int32 slot (seeded distinct slots).
    if not args.no_slots:
        P = 4 * B
        pool = torch.zeros((P, H, D, D), dtype=torch.float32, device=dev)
        slots_np = np.random.default_rng(113).permutation(P)[:B].astype(np.int32)
        slots = torch.from_numpy(slots_np).to(dev)
        pool.index_copy_(0, slots.long(), state0)
        Ks = min(K, 256)

        def sstep(s):
            kda.kda_decode_step_slots(q[s], k[s], v[s], beta[s], la[s], pool, slots, out=o)

        sgraph = None
        if not args.eager:
            try:
                side = torch.cuda.Stream(dev)
                side.wait_stream(stream)
                with torch.cuda.stream(side):
                    sstep(0)
                stream.wait_stream(side)
                torch.cuda.synchronize()
                sgraph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(sgraph):
                    for s in range(Ks):
                        sstep(s % n_gen)
                torch.cuda.synchronize()
            except Exception as e:
                log(f"graph capture of the slot steps failed ({e}); timing direct calls")
                sgraph = None

        def run_slots():
            if sgraph is not None:
                sgraph.replay()
            else:
                for s in range(Ks):
                    sstep(s % n_gen)

        run_slots()  # untimed
        torch.cuda.synchronize()
        pool.index_copy_(0, slots.long(), state0)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        run_slots()
        b.record(stream)
        torch.cuda.synchronize()
        sms = a.elapsed_time(b) / Ks
        sgbs = bytes_per_launch / (sms / 1e3) / 1e9
        if not bool(torch.isfinite(pool).all()):
            raise RuntimeError("slot decode produced non-finite states")
        log(f"decode from a pool of {P} entries: {sms * 1e3:.2f} us/step, {sgbs:.0f} GB/s")
        result["decode_slots"] = {
            "workload": f"the same decode, states in a pool of {P} x H={H} entries addressed by "
                        f"{B} distinct int32 slots",
            "steps": Ks,
            "ms_per_step": sms,
            "tokens_per_s": B / (sms / 1e3),
            "roofline": {"bound": "hbm", "achieved": sgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": sgbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": bytes_per_launch},
        }
        del pool, sgraph

    # ---------------- K draft tokens per call (secondary) --------------------
    # Speculative decoding: verify K = 4 draft tokens of every sequence in one
    # call (state only read), then commit an accepted prefix (a second call
    # that recomputes the tokens and rewrites the state).
    if not args.no_tokens:
        Kd = 4
        tq, tk, tv, tb, tla = (x[:Kd].transpose(0, 1).contiguous() for x in (q, k, v, beta, la))
        tstate = state0.clone()
        to = torch.empty((B, Kd, H, D), dtype=torch.float32, device=dev)
        commit = torch.full((B,), 2, dtype=torch.int32, device=dev)

        def timed(fn, reps=50):
            fn()
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / reps

        vms = timed(lambda: kda.kda_decode_tokens(tq, tk, tv, tb, tla, tstate, out=to))
        cms = timed(lambda: kda.kda_decode_tokens(tq, tk, tv, tb, tla, tstate, commit, out=to))
        in_bytes = Kd * B * H * (3 * D * 2 + 2 + D * 4 + D * 4)   # q, k, v, beta, log_alpha in; o out
        st_bytes = B * H * D * D * 4
        vgbs = (st_bytes + in_bytes) / (vms / 1e3) / 1e9
        cgbs = (2 * st_bytes + in_bytes) / (cms / 1e3) / 1e9
        log(f"verify {Kd} tokens: {vms * 1e3:.2f} us ({vgbs:.0f} GB/s); commit: {cms * 1e3:.2f} us "
            f"({cgbs:.0f} GB/s)")
        result["decode_tokens"] = {
            "workload": f"B={B} x H={H}, K={Kd} draft tokens per sequence from its state "
                        "(speculative verify, then commit of an accepted prefix)",
            "verify_ms": vms,
            "verify_tokens_per_s": B * Kd / (vms / 1e3),
            "commit_ms": cms,
            "roofline_verify": {"bound": "hbm", "achieved": vgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": vgbs / HBM_PEAK_GBS,
                                "algorithmic_bytes_per_launch": st_bytes + in_bytes},
            "roofline_commit": {"bound": "hbm", "achieved": cgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": cgbs / HBM_PEAK_GBS,
                                "algorithmic_bytes_per_launch": 2 * st_bytes + in_bytes},
        }
        del tq, tk, tv, tb, tla, tstate, to

    # ---------------- prefill (secondary) ---------------------------------
    if not args.no_prefill:
        T = args.prefill_T
        log(f"generating prefill inputs B=1 H={H} T={T}")
        pin = ki.workload_chunked(T=T, H=H)
        pq, pk, pv, pb = (up(x, True) for x in (pin.q, pin.k, pin.v, pin.beta))
        pla = up(pin.log_alpha, False)
        po = torch.empty((1, T, H, D), dtype=torch.float32, device=dev)
        ps = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
        pws = torch.empty(max(1, kda.prefill_workspace_size(1, T, H, torch.bfloat16)), dtype=torch.uint8,
                          device=dev)
        for _ in range(max(1, args.prefill_warmup)):
            kda.kda_prefill(pq, pk, pv, pb, pla, None, out=po, final_state=ps, workspace=pws)
        torch.cuda.synchronize()
        times = []
        for _ in range(args.prefill_reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            kda.kda_prefill(pq, pk, pv, pb, pla, None, out=po, final_state=ps, workspace=pws)
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        pms = float(np.median(times))
        pbytes = PREFILL_BYTES_PER_HEAD_TOKEN * T * H + H * D * D * 4
        pflops = PREFILL_FLOPS_PER_HEAD_TOKEN * T * H
        pgbs = pbytes / (pms / 1e3) / 1e9
        ptf = pflops / (pms / 1e3) / 1e12
        log(f"prefill: {pms:.3f} ms, {T / pms * 1e3 / 1e6:.2f} M tokens/s, {pgbs:.0f} GB/s")
        result["prefill"] = {
            "workload": f"chunked KDA prefill: B=1, H={H}, T={T}, d_k=d_v=128, bf16 q/k/v/beta, "
                        "fp32 log_alpha/state/o, gated channel mix, zero initial state",
            "ms": pms,
            "timing": f"median of {args.prefill_reps} calls, each between two HIP events, after "
                      f"{max(1, args.prefill_warmup)} untimed calls",
            "tokens_per_s": T / (pms / 1e3),
            "head_tokens_per_s": T * H / (pms / 1e3),
            "roofline": {"bound": "hbm", "achieved": pgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": pgbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic("prefill_H32_T32768_hbm_traffic.json", "prefill_call"),
                         "algorithmic_bytes_per_launch": pbytes,
                         "note": "achieved = algorithmic bytes / time of one call (3 kernels); traffic = "
                                 "measured HBM bytes of one call"},
            "mfma": {"algorithmic_tflops": ptf, "peak_tflops_bf16": BF16_MFMA_PEAK_TFLOPS,
                     "frac": ptf / BF16_MFMA_PEAK_TFLOPS,
                     "algorithmic_flops_per_launch": pflops},
        }
        if args.no_raw:
            del pq, pk, pv, pb, pla, po, ps, pws
        else:
            time_raw_prefill(kda, torch, np, stream, args.prefill_reps, args.prefill_warmup, pq, pk, pv, pb, pla,
                             po, ps, pms, T, result, pws)
            del pq, pk, pv, pb, pla, po, ps, pws

    if not args.no_large_decode:
        time_decode_large(kda, ki, torch, np, dev, up, stream, H, result)
    if not args.no_million:
        time_prefill_million(kda, ki, torch, np, dev, up, stream, H, result)
    if not args.no_varlen:
        time_prefill_varlen(kda, ki, torch, np, dev, up, stream, H, result)
    if not args.no_small:
        time_prefill_small(kda, ki, torch, np, dev, up, stream, result)

    # ---------------- backward pass (secondary) ---------------------------
    if not args.no_backward:
        time_backward(kda, ki, torch, np, dev, up, stream, args.backward_reps, result)

    # ---------------- CPU oracle baseline ---------------------------------
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(ki, np, B, H, args.cpu_steps, inp if n_gen >= args.cpu_steps else None)

    print(json.dumps(result), flush=True)
    return 0


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(ki, np, B, H, steps, inp=None):
    """The fp64 oracle on the host: `steps` steps of the decode workload (all
    B x H heads, every core the process may use), and one thread on the first
    4096 tokens of 16 heads of the chunked-prefill workload."""
    import oracle

    if inp is None:
        inp = ki.decode_steps(1, steps=steps, N=B, H=H)
    qf, kf, vf, bf, laf = (x[:steps] for x in inp.widened())
    threads = len(os.sched_getaffinity(0))
    log(f"cpu oracle: {steps} decode steps x {B * H} heads on {threads} threads")
    t0 = time.time()
    oracle.decode_chain(qf, kf, vf, bf, laf, inp.initial_state, n_threads=threads)
    dt = time.time() - t0
    Ts, Hs = 4096, 16
    pin = ki.workload_chunked(T=Ts, H=32, heads=range(Hs))
    t1 = time.time()
    oracle.prefill(*pin.widened(), None, n_threads=1)
    dt1 = time.time() - t1
    log(f"cpu oracle: decode {B * steps / dt:.1f} tokens/s in {dt:.1f}s; one thread, prefill "
        f"{Ts * Hs / dt1:.0f} head-tokens/s in {dt1:.1f}s")
    return {
        "value": B * steps / dt,
        "unit": "tokens/s",
        "cores": oracle.max_threads(threads),
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": f"the first {steps} of the decode workload's 1024 steps, all {B}x{H} heads, fp64 "
                  f"token-by-token recurrence, {dt:.1f} s wall on {oracle.max_threads(threads)} threads",
        "one_thread_prefill": {
            "sample": f"the first {Ts} tokens of heads 0..{Hs - 1} of the chunked-prefill workload "
                      "(T = 32768, gated mix), fp64 token-by-token, one thread",
            "seconds": dt1,
            "head_tokens_per_s": Ts * Hs / dt1,
            "tokens_per_s_at_32_heads": Ts * Hs / dt1 / 32,
        },
    }


def _median_ms(torch, np, stream, fn, reps, warmup=1):
    for _ in range(max(1, warmup)):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return float(np.median(ts))


def _prefill_roofline(head_tokens, n_states, ms, traffic=None):
    pbytes = PREFILL_BYTES_PER_HEAD_TOKEN * head_tokens + 2 * n_states * D * D * 4
    pflops = PREFILL_FLOPS_PER_HEAD_TOKEN * head_tokens
    gbs = pbytes / (ms / 1e3) / 1e9
    tf = pflops / (ms / 1e3) / 1e12
    return {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS, "traffic": traffic, "algorithmic_bytes_per_launch": pbytes,
            "mfma_algorithmic_tflops": tf, "mfma_frac": tf / BF16_MFMA_PEAK_TFLOPS}


def time_decode_large(kda, ki, torch, np, dev, up, stream, H, result, B=256, steps=1024, distinct=64):
    """The decode at B = 256 (512 MiB of fp32 state, twice the 256 MB
    last-level cache, so the state stream comes from DRAM): `steps` steps
    cycling over `distinct` seeded steps of inputs (a few KiB per head and
    step; the state stream does not depend on their values)."""
    log(f"generating {distinct} decode steps for B={B} H={H}")
    inp = ki.decode_steps(11, steps=distinct, N=B, H=H)
    q, k, v, b = (up(x, True) for x in (inp.q, inp.k, inp.v, inp.beta))
    la = up(inp.log_alpha, False)
    state = up(inp.initial_state, False)
    o = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    del inp

    def run():
        for s in range(steps):
            j = s % distinct
            kda.kda_decode_step(q[j], k[j], v[j], b[j], la[j], state, out=o)

    graph = None
    try:
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            kda.kda_decode_step(q[0], k[0], v[0], b[0], la[0], state, out=o)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        torch.cuda.synchronize()
    except Exception as e:
        log(f"graph capture failed ({e}); timing direct calls")
        graph = None
    fn = graph.replay if graph is not None else run
    ms = _median_ms(torch, np, stream, fn, reps=3) / steps
    if not bool(torch.isfinite(state).all()):
        raise RuntimeError("decode produced non-finite states")
    nbytes = DECODE_BYTES_PER_HEAD * B * H
    gbs = nbytes / (ms / 1e3) / 1e9
    # the streaming ceiling of the same state tensor (read and written once)
    cms = _median_ms(torch, np, stream, lambda: state.mul_(1.0), reps=16, warmup=4)
    cgbs = 2 * B * H * D * D * 4 / (cms / 1e3) / 1e9
    log(f"decode B={B}: {ms * 1e3:.2f} us/step, {B / ms * 1e3 / 1e6:.3f} M tokens/s, {gbs:.0f} GB/s "
        f"(state read-modify-write ceiling {cgbs:.0f} GB/s)")
    result["decode_large"] = {
        "workload": f"the decode workload at B={B} sequences x H={H} heads (fp32 state {B * H * D * D * 4 >> 20} "
                    f"MiB), {steps} consecutive steps cycling over {distinct} seeded input steps",
        "ms_per_step": ms,
        "tokens_per_s": B / (ms / 1e3),
        "timing": f"median of 3 {'graph replays' if graph is not None else 'runs'} of {steps} steps",
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": nbytes},
        "state_rmw_ceiling": {"what": "torch in-place scale by 1 of the same state tensor", "us": cms * 1e3,
                              "GBps": cgbs, "decode_frac_of_ceiling": gbs / cgbs},
    }
    del q, k, v, b, la, state, o, graph


def time_prefill_million(kda, ki, torch, np, dev, up, stream, H, result, T=1 << 20, reps=5):
    """The million-token prefill: B = 1, H = 32, T = 1,048,576, bf16 inputs,
    the gated channel mix, zero initial state (the parity-tested inputs)."""
    log(f"generating million-token prefill inputs B=1 H={H} T={T}")
    t0 = time.time()
    inp = ki.workload_million(T=T, H=H)
    q, k, v, b = (up(x, True) for x in (inp.q, inp.k, inp.v, inp.beta))
    la = up(inp.log_alpha, False)
    del inp
    log(f"generated and uploaded in {time.time() - t0:.0f}s")
    o = torch.empty((1, T, H, D), dtype=torch.float32, device=dev)
    st = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, kda.prefill_workspace_size(1, T, H, torch.bfloat16)), dtype=torch.uint8, device=dev)
    ms = _median_ms(torch, np, stream,
                    lambda: kda.kda_prefill(q, k, v, b, la, None, out=o, final_state=st, workspace=ws),
                    reps=reps, warmup=2)
    if not bool(torch.isfinite(st).all()):
        raise RuntimeError("million-token prefill produced non-finite states")
    roof = _prefill_roofline(T * H, H, ms)
    log(f"prefill T={T}: {ms:.2f} ms, {T / ms * 1e3 / 1e6:.2f} M tokens/s, {roof['achieved']:.0f} GB/s")
    result["prefill_million"] = {
        "workload": f"million-token KDA prefill: B=1, H={H}, T={T}, d_k=d_v=128, bf16 q/k/v/beta, fp32 "
                    "log_alpha/state/o, gated channel mix (10% long-memory, 10% fast-forgetting "
                    "channels per head), zero initial state",
        "ms": ms,
        "timing": f"median of {reps} calls, each between two HIP events, after 2 untimed calls",
        "workspace_bytes": ws.numel(),
        "tokens_per_s": T / (ms / 1e3),
        "head_tokens_per_s": T * H / (ms / 1e3),
        "roofline": roof,
    }
    del q, k, v, b, la, o, st, ws


def time_prefill_varlen(kda, ki, torch, np, dev, up, stream, H, result, reps=10):
    """The packed prefill: 16 sequences, lengths log-uniform in [1024, 65536]
    (seeded), even-indexed ones resumed from N(0, 0.02^2) states."""
    inp = ki.workload_varlen(H=H)
    cu = inp.cu_seqlens
    N, Tt = cu.size - 1, int(cu[-1])
    log(f"packed prefill: {N} sequences, {Tt} tokens")
    q, k, v, b = (up(x, True) for x in (inp.q, inp.k, inp.v, inp.beta))
    la = up(inp.log_alpha, False)
    s0 = up(inp.initial_state, False)
    cud = torch.from_numpy(cu).to(dev)
    del inp
    o = torch.empty((1, Tt, H, D), dtype=torch.float32, device=dev)
    st = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, kda.varlen_prefill_workspace_size(N, Tt, H, torch.bfloat16)), dtype=torch.uint8,
                     device=dev)
    ms = _median_ms(torch, np, stream,
                    lambda: kda.kda_varlen_prefill(q, k, v, b, la, cud, s0, out=o, final_state=st,
                                                   workspace=ws),
                    reps=reps, warmup=5)
    roof = _prefill_roofline(Tt * H, N * H, ms)
    log(f"packed prefill: {ms:.2f} ms, {Tt / ms * 1e3 / 1e6:.2f} M tokens/s, {roof['achieved']:.0f} GB/s")
    result["prefill_varlen"] = {
        "workload": f"packed KDA prefill: {N} sequences of log-uniform lengths in [1024, 65536] "
                    f"(seeded; {Tt} tokens in all, longest {int(np.max(np.diff(cu)))}), H={H}, bf16 inputs, "
                    "gated channel mix, even-indexed sequences resumed from N(0, 0.02^2) fp32 states",
        "ms": ms,
        "timing": f"median of {reps} calls, each between two HIP events, after 5 untimed calls",
        "tokens_per_s": Tt / (ms / 1e3),
        "head_tokens_per_s": Tt * H / (ms / 1e3),
        "roofline": roof,
    }
    del q, k, v, b, la, s0, cud, o, st, ws


def time_prefill_small(kda, ki, torch, np, dev, up, stream, result, calls=200):
    """The small fp32 prefill: B = 1, H = 1, T = 256 (one unit: the token
    kernel, bound by its 256 dependent steps and the launch)."""
    inp = ki.workload_single(T=256)
    q, k, v, b, la = (up(x, False) for x in (inp.q, inp.k, inp.v, inp.beta, inp.log_alpha))
    o = torch.empty((1, 256, 1, D), dtype=torch.float32, device=dev)
    st = torch.empty((1, 1, D, D), dtype=torch.float32, device=dev)

    def run():
        for _ in range(calls):
            kda.kda_prefill(q, k, v, b, la, None, out=o, final_state=st)

    ms = _median_ms(torch, np, stream, run, reps=3) / calls
    log(f"small fp32 prefill: {ms * 1e3:.1f} us per call, {256 / ms * 1e3 / 1e6:.2f} M tokens/s")
    result["prefill_small"] = {
        "workload": "single-sequence fp32 KDA prefill: B=1, H=1, T=256, d_k=d_v=128, zero initial state",
        "ms": ms,
        "timing": f"median of 3 runs of {calls} consecutive calls (direct calls from Python), per call",
        "tokens_per_s": 256 / (ms / 1e3),
        "note": "one (sequence, head) unit on one CU: latency of 256 dependent token steps plus the "
                "launch, not a bandwidth or matrix-core figure",
    }


def time_raw_prefill(kda, torch, np, stream, reps, warmup, pq, pk, pv, pb, pla, po, ps, pms, T, result, pws):
    """The chunked prefill on raw projections: the same resident buffers read as
    raw q, k, v, beta logits and gate logits (the kernels take no value-dependent
    branch, so any values time alike); the unit-norm, sigmoid and softplus
    preparation runs inside the staging."""
    for _ in range(max(1, warmup // 3)):
        kda.kda_prefill_raw(pq, pk, pv, pb, pla, None, out=po, final_state=ps, workspace=pws)
    torch.cuda.synchronize()
    rtimes = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        kda.kda_prefill_raw(pq, pk, pv, pb, pla, None, out=po, final_state=ps, workspace=pws)
        b.record(stream)
        torch.cuda.synchronize()
        rtimes.append(a.elapsed_time(b))
    rms = float(np.median(rtimes))
    log(f"prefill from raw projections: {rms:.3f} ms ({(rms / pms - 1) * 100:+.1f}% over prepared)")
    result["prefill"]["raw"] = {
        "workload": "the same shape from raw projections (q, k normalised per head, sigmoid "
                    "write strength, minus-softplus log gate, all inside the kernels)",
        "ms": rms,
        "tokens_per_s": T / (rms / 1e3),
        "overhead_vs_prepared": rms / pms - 1,
    }


def time_backward(kda, ki, torch, np, dev, up, stream, reps, result):
    """Gradients of a prefill at a training shape (B = 8 sequences of 4096
    tokens, H = 32, bf16 inputs, gated channel mix), timed with HIP events
    (median of the repeats) beside the chunked forward on the same inputs."""
    B, T, H = ki.BACKWARD_SHAPE
    log(f"generating backward inputs B={B} T={T} H={H}")
    inp = ki.workload_backward()
    d_o, d_s = ki.loss_gradients(ki.BACKWARD_WORKLOAD, (B, T, H, D), B, H)
    q, k, v, b = (up(x, True) for x in (inp.q, inp.k, inp.v, inp.beta))
    la, do, ds = up(inp.log_alpha, False), up(d_o, False), up(d_s, False)
    del inp, d_o, d_s

    # the first calls after the prefill section run up to 15% slower while the
    # GPU settles: five untimed calls first
    warm = 5

    def med(fn):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            e.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(e))
        return float(np.median(ts))

    ws = torch.empty(kda.backward_workspace_size(B, T, H, torch.bfloat16), dtype=torch.uint8, device=dev)
    bms = med(lambda: kda.kda_backward(q, k, v, b, la, do, None, ds, workspace=ws))
    fms = med(lambda: kda.kda_prefill(q, k, v, b, la, None))
    nbytes = BACKWARD_BYTES_PER_HEAD_TOKEN * B * T * H
    flops = BACKWARD_FLOPS_PER_HEAD_TOKEN * B * T * H
    gbs = nbytes / (bms / 1e3) / 1e9
    tf = flops / (bms / 1e3) / 1e12
    log(f"backward: {bms:.2f} ms ({B * T * H / bms / 1e3:.1f} M head-tokens/s, {gbs:.0f} GB/s, "
        f"{tf:.1f} TFLOP/s); forward on the same inputs {fms:.2f} ms")
    result["backward"] = {
        "workload": f"gradients of a prefill: B={B} x T={T} tokens, H={H}, bf16 q/k/v/beta, fp32 "
                    "log_alpha/d_o/d_final_state, gated channel mix, zero initial state",
        "ms": bms,
        "timing": f"median of {reps} calls, each between two HIP events, after {warm} untimed calls; "
                  "caller-provided workspace",
        "workspace_bytes": ws.numel(),
        "tokens_per_s": B * T / (bms / 1e3),
        "head_tokens_per_s": B * T * H / (bms / 1e3),
        "forward_ms_same_inputs": fms,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": nbytes,
                     "traffic": measured_traffic("backward_B8_T4096_H32_hbm_traffic.json", "backward_call"),
                     "mfma_algorithmic_tflops": tf, "mfma_frac": tf / BF16_MFMA_PEAK_TFLOPS,
                     "algorithmic_flops_per_launch": flops,
                     "note": "the chunked backward (four kernels); algorithmic bytes = inputs read "
                             "and gradients written once; traffic = the measured HBM bytes of one call "
                             "(its workspace round trips included)"},
    }
    del q, k, v, b, la, do, ds


if __name__ == "__main__":
    sys.exit(main())
