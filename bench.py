"""Benchmark of the gated delta rule forward (KDA) on one MI355X.

A step is one kda_chunk_fwd call over the packed variable-length workload
(H = 32, dk = dv = 128, T = 65536 tokens in 8 sequences, bf16 q/k/v/o, fp32
per-channel log-decay and beta, chunk 64): cumulative decay, stability scaling, UT
transform, sequential state pass and chunk output, all in one fused kernel launch.
Inputs are seeded synthetic tensors resident in HBM before the timed region. The
backward on the same device inputs is timed first and the forward right after it, so that
the forward's timed calls do not start from the idle power state in which the host-side
input generation leaves the GPU (the Gated Delta Rule-2 pair likewise).

Printed (one JSON line on stdout):
  value          tokens/s of that step (65536 tokens per step), from the mean over the
                 timed steps; ms_per_step_median is the median of the per-call times
  roofline       the chunk kernel against the HBM roofline: algorithmic bytes per
                 launch / average launch time (HIP events on the launch stream),
                 and the HBM bytes measured by rocprofv3 counters when given
  mfma           the same kernel's algorithmic flops against the bf16 MFMA peak
  decode         kda_recurrent_step on 256 sequences x 32 heads, 512 consecutive
                 steps on a resident fp32 state: tokens/s and HBM GB/s
  gdr2           the Gated Delta Rule-2 forward and decode step on the same workloads
  gates          the fused prologue (L2Norm, decay gate, sigmoid) and epilogue (gated
                 RMSNorm) on the chunk workload's rows, against the HBM roofline
  bwd            kda_chunk_bwd (all gradients) on the chunk workload
  small_configs  kda_chunk_fwd on the tiny fp32 (B1 H2 T256 dk=dv=64), B2 H16 T4096 and
                 GDN B1 H16 T8192 workloads and the B2 H16 T4096 shape in fp32, each with its
                 matrix-core rate (median time) against the peak of its arithmetic type
  cpu_baseline   the fp64 CPU oracle on a bounded sample of the same workload
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA fwd tokens/s at H=32,dk=dv=128,T=64K; % MFMA peak; decode HBM GB/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
MFMA_F32_PEAK_TFLOPS = 157.3    # MI355X dense fp32 (matrix cores)
CHUNK = 64

# HBM traffic of one chunk-forward call (for the packed KDA and Gated Delta Rule-2 workloads:
# the segment planner, the items, the segment chain and the output corrections), from two
# rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE, KiB per dispatch)
# each scaled by the counter/byte ratio measured on a plain 1 GiB copy kernel in the same
# runs. It is reported only while the kernel source is the one the counters were taken on
# (its SHA-256 below); otherwise traffic is null.
MEASURED_TRAFFIC = {      # profiles/kda_chunk_fwd_varlen_h32_t65536.md
    "bytes": 3792918794,
    "kernel_sha256": "c3ba2b158da694e96aabb8bb8d51a22ac73eeb9da47893f28d0fc58c7c2bd8cd",
}
MEASURED_TRAFFIC_GDR2 = {  # profiles/kda_gdr2_chunk_fwd_varlen_h32_t65536.md
    "bytes": 5926890387,
    "kernel_sha256": "c3ba2b158da694e96aabb8bb8d51a22ac73eeb9da47893f28d0fc58c7c2bd8cd",
}
# one kda_chunk_bwd call (state history, reverse carry, gradients): its own source and that of
# the forward kernel whose history mode it runs
MEASURED_TRAFFIC_BWD = {  # profiles/kda_chunk_bwd_varlen_h32_t65536.md
    "bytes": 19504313182,
    "kernel_sha256": "2286d7707f2052a2ae67b1e87ac3eda8181d747c71ccfc3ae43561b2ffc0ceee",
    "hist_sha256": "c3ba2b158da694e96aabb8bb8d51a22ac73eeb9da47893f28d0fc58c7c2bd8cd",
}
MEASURED_TRAFFIC_PROLOGUE = {  # profiles/kda_prologue_h32_t65536.md
    "bytes": 4320464550,
    "kernel_sha256": "7b71bd805a0b3f8716f80570bf27cba8d0b6c9ff81b3b572063d4f27f5b0b336",
}
MEASURED_TRAFFIC_EPILOGUE = {  # profiles/kda_epilogue_h32_t65536.md
    "bytes": 1610632255,
    "kernel_sha256": "7b71bd805a0b3f8716f80570bf27cba8d0b6c9ff81b3b572063d4f27f5b0b336",
}
CSRC = os.path.join(ROOT, "gated_delta_rule_13_amd", "csrc")
CHUNK_KERNEL_SRC = os.path.join(CSRC, "kda_chunk_mfma.hip")
BWD_KERNEL_SRC = os.path.join(CSRC, "kda_chunk_bwd.hip")
GATES_KERNEL_SRC = os.path.join(CSRC, "kda_gates.hip")


def measured_traffic(record=None, src=CHUNK_KERNEL_SRC):
    """HBM bytes per launch from the committed rocprofv3 counters, or None once the
    kernel source ``src`` differs from the one they were taken on."""
    import hashlib
    record = MEASURED_TRAFFIC if record is None else record
    if not record:
        return None
    def digest(path):
        with open(path, "rb") as f:
            return hashlib.sha256(f.read()).hexdigest()
    if digest(src) != record["kernel_sha256"]:
        return None
    if "hist_sha256" in record and digest(CHUNK_KERNEL_SRC) != record["hist_sha256"]:
        return None
    return record["bytes"]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def chunk_alg_flops_per_head_token(dk: int, dv: int, C: int = CHUNK) -> float:
    """Three C x dk x dv contractions (W S or K^ S, Q^ S, K_dec^T V'), A_kk, A_qk and the
    beta-scaled key product at C dk each, T V and A_qk V' at C dv each, and the
    triangular inverse, counted without the zero halves of triangular tiles."""
    return 6 * dk * dv + 3 * C * dk + 2 * C * dv + C * C / 3


def chunk_alg_bytes(x) -> float:
    """Inputs read once and outputs written once: q, k, v (bf16), g (fp32 per channel),
    beta (fp32) or the Gated Delta Rule-2 gates (erase fp32 [dk], write fp32 [dv]),
    o (bf16), plus the initial / final state of every chain (fp32)."""
    B, H, T, dk = x.q.shape
    dv = x.v.shape[-1]
    gates = 4 * (dk + dv) if x.erase is not None else 4
    per_tok = 2 * (2 * dk + dv) + 4 * (dk if x.g.ndim == 4 else 1) + gates + 2 * dv
    n_chains = x.n_seqs * H
    state = 4 * dk * dv * n_chains * (2 if x.s0 is not None else 1)
    return float(per_tok * B * H * T + state)


def decode_alg_bytes_per_step(N: int, H: int, dk: int, dv: int, gdr2: bool = False) -> float:
    """State read and written once (fp32), q, k, v (bf16), g (fp32), beta or the Gated
    Delta Rule-2 gates (erase [dk], write [dv], fp32), o (bf16)."""
    gates = 4 * (dk + dv) if gdr2 else 4
    per_chain = 2 * dk * dv * 4 + 2 * (2 * dk + dv) + 4 * dk + gates + 2 * dv
    return float(per_chain * N * H)


def prologue_alg_bytes(B: int, H: int, T: int, dk: int, qk_bytes: int = 2) -> float:
    """q, k read and written (bf16), u read and g written (fp32 per channel), the beta
    pre-activation read and beta written (fp32), plus A_log and dt_bias once."""
    per_row = 4 * dk * qk_bytes + 2 * 4 * dk + 2 * 4
    return float(per_row * B * H * T + 4 * H * (1 + dk))


def epilogue_alg_bytes(B: int, H: int, T: int, dv: int, o_bytes: int = 2) -> float:
    """o and z read, the gated output written (bf16), plus the RMSNorm weight once."""
    return float(3 * o_bytes * dv * B * H * T + 4 * dv)


def time_calls(torch, call, steps: int, warmup: int, per_call: bool = False):
    """Milliseconds per call over ``steps`` back-to-back calls after ``warmup`` untimed ones,
    HIP events on the launch stream, the timed region bracketed by device synchronisations.
    Returns the mean (the bracket's time / steps); with ``per_call`` also the median of the
    per-call times (one event pair around each call, recorded in the same stream)."""
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(torch.device("cuda:0"))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        call()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    mean = ev[0].elapsed_time(ev[steps]) / steps
    if not per_call:
        return mean
    return mean, statistics.median(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))


def bench_gates(torch, kda, cfg, steps: int, warmup: int):
    """The fused prologue and epilogue around the operator on the workload's B, H, T."""
    from kda_workloads import make_gate_inputs
    dev = torch.device("cuda:0")
    up = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)  # noqa
    t0 = time.time()
    x = make_gate_inputs(cfg)
    bf = torch.bfloat16
    q_in, k_in, z = up(x.q_in, bf), up(x.k_in, bf), up(x.z, bf)
    u, A_log, dt_bias, beta_in, w = (up(a) for a in (x.u, x.A_log, x.dt_bias, x.beta_in,
                                                      x.weight))
    del x
    log(f"gate inputs generated and resident in {time.time() - t0:.1f}s")
    q, k = torch.empty_like(q_in), torch.empty_like(k_in)
    g, beta = torch.empty_like(u), torch.empty_like(beta_in)
    o = torch.empty_like(z)
    st = kda.load_library()
    stream = torch.cuda.current_stream(dev).cuda_stream
    B, H, T, dk = q_in.shape
    dv = z.shape[-1]

    def prologue():
        rc = st.kda_prologue(q_in.data_ptr(), k_in.data_ptr(), u.data_ptr(), A_log.data_ptr(),
                             dt_bias.data_ptr(), beta_in.data_ptr(), q.data_ptr(), k.data_ptr(),
                             g.data_ptr(), beta.data_ptr(), B, H, T, dk, kda.KDA_BF16, stream)
        if rc != kda.KDA_OK:
            raise RuntimeError(f"kda_prologue returned {rc}")

    def epilogue():
        rc = st.kda_epilogue(q.data_ptr(), z.data_ptr(), w.data_ptr(), 1e-6, o.data_ptr(),
                             B, H, T, dv, kda.KDA_BF16, stream)
        if rc != kda.KDA_OK:
            raise RuntimeError(f"kda_epilogue returned {rc}")
    out = {}
    for name, call, nbytes, rec in (
            ("prologue", prologue, prologue_alg_bytes(B, H, T, dk), MEASURED_TRAFFIC_PROLOGUE),
            ("epilogue", epilogue, epilogue_alg_bytes(B, H, T, dv), MEASURED_TRAFFIC_EPILOGUE)):
        ms = time_calls(torch, call, steps, warmup)
        gbs = nbytes / (ms / 1e3) / 1e9
        out[name] = {"us_per_launch": ms * 1e3, "roofline": {
            "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic(rec, GATES_KERNEL_SRC),
            "alg_bytes_per_launch": nbytes}}
        log(f"{name}: {ms * 1e3:.1f} us/launch, {gbs:.0f} GB/s")
    return out


def bwd_alg_bytes(x) -> float:
    """Inputs read once and outputs written once: q, k, v, dO (bf16), g (fp32 per channel),
    beta (fp32); dq, dk, dv (bf16), dg, dbeta (fp32); plus the initial state, the final
    state's gradient and the initial state's gradient of every chain (fp32)."""
    B, H, T, dk = x.q.shape
    dv = x.v.shape[-1]
    g = 4 * (dk if x.g.ndim == 4 else 1)
    per_tok = 2 * 2 * (2 * dk + dv) + 2 * dv + 2 * (g + 4)
    n_chains = x.n_seqs * H
    state = 4 * dk * dv * n_chains * (3 if x.s0 is not None else 2)
    return float(per_tok * B * H * T + state)


def device_inputs(torch, x, cotangents: bool = False) -> dict:
    """The workload's inputs (and, with ``cotangents``, the backward's dO and dS_T) uploaded
    once to the device, shared by the backward and forward measurements."""
    dev = torch.device("cuda:0")
    up = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)  # noqa
    dt = torch.bfloat16 if x.cfg.dtype == "bf16" else torch.float32
    d = {"q": up(x.q, dt), "k": up(x.k, dt), "v": up(x.v, dt), "g": up(x.g),
         "beta": up(x.beta), "s0": up(x.s0) if x.s0 is not None else None,
         "cu": up(x.cu_seqlens, torch.int32) if x.cu_seqlens is not None else None,
         "erase": up(x.erase) if x.erase is not None else None,
         "write": up(x.write) if x.write is not None else None}
    if cotangents:
        from kda_workloads import make_cotangents
        ct = make_cotangents(x.cfg, x.n_seqs)
        d["do"], d["dsT"] = up(ct.do, dt), up(ct.dsT)
    return d


def bench_bwd(torch, kda, x, d, steps: int, warmup: int):
    """kda_chunk_bwd on the workload (all gradients, with the final-state cotangent), on the
    device inputs ``d`` (``device_inputs(..., cotangents=True)``)."""
    dev = torch.device("cuda:0")
    q, k, v, do, g, beta, dsT, s0, cu = (d[n] for n in ("q", "k", "v", "do", "g", "beta", "dsT",
                                                        "s0", "cu"))
    B, H, T, dk = x.q.shape
    dv = x.v.shape[-1]
    outs = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(g),
            torch.empty_like(beta)]
    ds0 = torch.empty((x.n_seqs, H, dk, dv), dtype=torch.float32, device=dev)
    ns = x.n_seqs if cu is not None else 0
    gm = kda.KDA_GATE_PER_CHANNEL if x.g.ndim == 4 else kda.KDA_GATE_PER_HEAD
    wsb = kda.kda_chunk_bwd_workspace_size(B, H, T, dk, dv, ns, kda.KDA_BF16)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    if x.erase is not None:   # Gated Delta Rule-2: erase / write gates and their gradients
        erase, write = d["erase"], d["write"]
        outs = outs[:4] + [torch.empty_like(erase), torch.empty_like(write)]

    def call():
        if x.erase is not None:
            rc = kda.kda_gdr2_chunk_bwd(ptr(q), ptr(k), ptr(v), ptr(g), ptr(erase), ptr(write),
                                        ptr(s0), ptr(do), ptr(dsT),
                                        *[o.data_ptr() for o in outs], ds0.data_ptr(),
                                        ptr(cu), ns, B, H, T, dk, dv, kda.KDA_BF16, gm,
                                        ws.data_ptr(), wsb, stream)
        else:
            rc = kda.kda_chunk_bwd(ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), ptr(s0), ptr(do),
                                   ptr(dsT), *[o.data_ptr() for o in outs], ds0.data_ptr(),
                                   ptr(cu), ns, B, H, T, dk, dv, kda.KDA_BF16, gm,
                                   ws.data_ptr(), wsb, stream)
        if rc != kda.KDA_OK:
            raise RuntimeError(f"kda_chunk_bwd returned {rc}")
    ms = time_calls(torch, call, steps, warmup)
    return ms, wsb


def bench_chunk(torch, kda, x, steps: int, warmup: int, d=None):
    """One chunk-forward call per step through the C ABI, with the workspace the library
    recommends allocated once beforehand (as a caller would), on the device inputs ``d``
    (uploaded here when not given). Returns the mean and median milliseconds per call and
    the workspace bytes."""
    dev = torch.device("cuda:0")
    if d is None:
        d = device_inputs(torch, x)
    dt = torch.bfloat16 if x.cfg.dtype == "bf16" else torch.float32
    code = kda.KDA_BF16 if dt == torch.bfloat16 else kda.KDA_F32
    q, k, v, g, beta, cu, s0 = (d[n] for n in ("q", "k", "v", "g", "beta", "cu", "s0"))
    o = torch.empty(tuple(x.v.shape), dtype=dt, device=dev)
    sT = torch.empty((x.n_seqs, x.q.shape[1], x.q.shape[3], x.v.shape[3]), dtype=torch.float32,
                     device=dev)
    B, H, T, dk = x.q.shape
    dv = x.v.shape[-1]
    ns = x.n_seqs if cu is not None else 0
    wsb = kda.kda_chunk_fwd_workspace_size(B, H, T, dk, dv, ns, code)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    gm = kda.KDA_GATE_PER_CHANNEL if x.g.ndim == 4 else kda.KDA_GATE_PER_HEAD
    stream = torch.cuda.current_stream(dev).cuda_stream
    ptr = lambda a: a.data_ptr() if a is not None else None  # noqa: E731
    common = (ptr(s0), ptr(sT), ptr(o), ptr(cu), ns, B, H, T, dk, dv, code, gm, ptr(ws), wsb,
              stream)
    if x.erase is not None:
        erase, write = d["erase"], d["write"]

        def call():
            rc = kda.kda_gdr2_chunk_fwd(ptr(q), ptr(k), ptr(v), ptr(g), ptr(erase),
                                        ptr(write), *common)
            if rc != kda.KDA_OK:
                raise RuntimeError(f"kda_gdr2_chunk_fwd returned {rc}")
    else:
        def call():
            rc = kda.kda_chunk_fwd(ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), *common)
            if rc != kda.KDA_OK:
                raise RuntimeError(f"kda_chunk_fwd returned {rc}")
    mean, median = time_calls(torch, call, steps, warmup, per_call=True)
    return mean, median, wsb


def bench_decode(torch, kda, cfg, reps: int = 5):
    from kda_workloads import decode_initial_state, decode_step_inputs
    dev = torch.device("cuda:0")
    N, H, dk, dv, S = cfg.B, cfg.H, cfg.dk, cfg.dv, cfg.T
    t0 = time.time()
    qs = torch.empty((S, N, H, dk), dtype=torch.bfloat16, device=dev)
    ks = torch.empty_like(qs)
    vs = torch.empty((S, N, H, dv), dtype=torch.bfloat16, device=dev)
    gs = torch.empty((S, N, H, dk), dtype=torch.float32, device=dev)
    bs = torch.empty((S, N, H), dtype=torch.float32, device=dev)
    gdr2 = cfg.gates == "gdr2"
    if gdr2:
        es = torch.empty((S, N, H, dk), dtype=torch.float32, device=dev)
        ws = torch.empty((S, N, H, dv), dtype=torch.float32, device=dev)
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(8) as ex:
        for s, d in enumerate(ex.map(lambda i: decode_step_inputs(cfg, i), range(S))):
            qs[s].copy_(torch.from_numpy(d.q))
            ks[s].copy_(torch.from_numpy(d.k))
            vs[s].copy_(torch.from_numpy(d.v))
            gs[s].copy_(torch.from_numpy(d.g))
            bs[s].copy_(torch.from_numpy(d.beta))
            if gdr2:
                es[s].copy_(torch.from_numpy(d.erase))
                ws[s].copy_(torch.from_numpy(d.write))

    def step(s):
        if gdr2:
            kda.gdr2_recurrent_step(qs[s], ks[s], vs[s], gs[s], es[s], ws[s], state, o=o)
        else:
            kda.recurrent_step(qs[s], ks[s], vs[s], gs[s], bs[s], state, o=o)
    s_init = torch.from_numpy(decode_initial_state(cfg)).to(dev)
    state = torch.empty_like(s_init)
    o = torch.empty((N, H, dv), dtype=torch.bfloat16, device=dev)
    log(f"decode inputs generated and resident in {time.time() - t0:.1f}s")
    stream = torch.cuda.current_stream(dev)
    state.copy_(s_init)
    for s in range(min(8, S)):  # warm-up
        step(s)
    times = []
    for _ in range(reps):
        state.copy_(s_init)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for s in range(S):
            step(s)
        ev1.record(stream)
        torch.cuda.synchronize()
        times.append(ev0.elapsed_time(ev1) / 1e3)
    # the same steps captured once in a HIP graph and replayed (state re-initialised outside)
    g = torch.cuda.CUDAGraph()
    state.copy_(s_init)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for s in range(S):
            step(s)
    gtimes = []
    for _ in range(reps):
        state.copy_(s_init)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        g.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        gtimes.append(ev0.elapsed_time(ev1) / 1e3)
    return statistics.median(times), statistics.median(gtimes)


def cpu_baseline(x, max_chains: int):
    """The fp64 oracle as it stands, on the host cores, over a seeded sample of chains of
    the same workload (all tokens of each sampled chain). Reported in tokens/s of the
    metric (head-tokens / H, i.e. positions carrying all heads)."""
    import oracle
    H = x.q.shape[1]
    all_chains = [(n, h) for n in range(x.n_seqs) for h in range(H)]
    rng = np.random.default_rng(2024)
    idx = np.sort(rng.choice(len(all_chains), size=min(max_chains, len(all_chains)),
                             replace=False))
    chains = [all_chains[i] for i in idx]
    head_tokens = sum(x.chain_rows(n, h)[2] for (n, h) in chains)
    threads = oracle.max_threads()
    chains, cargs, ckw = oracle.pack_chains(x.q, x.k, x.v, x.g, x.beta, x.s0, x.cu_seqlens,
                                            chains)
    t0 = time.perf_counter()
    oracle.kda_chains(*cargs, **ckw, threads=threads)
    dt = time.perf_counter() - t0
    # the same recurrence on one thread, over the 8 sampled chains of one head
    one = [(n, 0) for n in range(x.n_seqs)]
    one_tokens = sum(x.chain_rows(n, h)[2] for (n, h) in one)
    _, oargs, okw = oracle.pack_chains(x.q, x.k, x.v, x.g, x.beta, x.s0, x.cu_seqlens, one)
    t1 = time.perf_counter()
    oracle.kda_chains(*oargs, **okw, threads=1)
    dt1 = time.perf_counter() - t1
    return {"value": head_tokens / H / dt, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(chains)} of {len(all_chains)} (sequence, head) chains of the "
                      f"workload, all their tokens ({head_tokens} head-tokens), fp64 token "
                      f"recurrence, {dt:.1f} s",
            "cpu_model": cpu_model(),
            "one_thread": {"value": one_tokens / H / dt1, "unit": "tokens/s", "cores": 1,
                           "sample": f"the {len(one)} chains of head 0 ({one_tokens} "
                                     f"head-tokens), {dt1:.1f} s"}}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_probe(torch):
    """A plain 1 GiB device copy, run only to calibrate the HBM byte counters."""
    dev = torch.device("cuda:0")
    a = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-chains", type=int, default=256)
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--no-gdr2", action="store_true",
                    help="skip the Gated Delta Rule-2 measurements")
    ap.add_argument("--no-gates", action="store_true",
                    help="skip the prologue / epilogue measurements")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward pass")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        return 2

    import torch

    import gated_delta_rule_13_amd as kda
    from kda_workloads import (GDN_B1_H16_T8192, KDA_B2_H16_T4096, KDA_DECODE_N256_H32,
                               KDA_VARLEN_H32_T65536, TINY_KDA_F32, make_chunk_inputs)

    kda.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    cfg = KDA_VARLEN_H32_T65536
    t0 = time.time()
    x = make_chunk_inputs(cfg)
    log(f"generated {cfg.name} in {time.time() - t0:.1f}s; lengths {np.diff(x.cu_seqlens)}")
    if args.copy_probe:
        copy_probe(torch)
    # the smaller prefill workloads (parity-test shapes), scheduled as a caller would, and the
    # B2 H16 T4096 shape in fp32 (the fp32 matrix-core kernel at a size that fills it): made
    # and uploaded here, timed right after the headline forward
    small_cfgs = (TINY_KDA_F32, KDA_B2_H16_T4096, GDN_B1_H16_T8192,
                  KDA_B2_H16_T4096.replace(name="kda_f32_b2_h16_t4096", dtype="f32"))
    small_x = [make_chunk_inputs(c) for c in small_cfgs]
    small_d = [device_inputs(torch, sx) for sx in small_x]
    d = device_inputs(torch, x, cotangents=not args.no_bwd)
    # The backward is timed first, on the same device inputs, and the forward right after it:
    # the host-side input generation leaves the GPU idle for seconds, and a forward timed
    # straight from idle runs its first ~25 calls (~25 ms) in a lower power state (measured
    # 0.95 against 0.88 ms per call); the warmup steps alone (5 x 0.9 ms) do not cover that.
    if not args.no_bwd:
        bms, bwsb = bench_bwd(torch, kda, x, d, args.steps, args.warmup)
    ms, ms_median, ws_bytes = bench_chunk(torch, kda, x, args.steps, args.warmup, d)
    del d
    small = {}
    for c, sx, sd in zip(small_cfgs, small_x, small_d):
        sms, smed, _ = bench_chunk(torch, kda, sx, args.steps, args.warmup, sd)
        sb = chunk_alg_bytes(sx)
        sflops = chunk_alg_flops_per_head_token(c.dk, c.dv) * c.B * c.H * c.T
        speak = MFMA_F32_PEAK_TFLOPS if c.dtype == "f32" else MFMA_BF16_PEAK_TFLOPS
        stf = sflops / (smed / 1e3) / 1e12
        small[c.name] = {"ms_per_step": sms, "ms_per_step_median": smed, "dtype": c.dtype,
                         "tokens_per_s": c.B * c.T / (sms / 1e3),
                         "hbm_gbs": sb / (sms / 1e3) / 1e9,
                         "mfma": {"achieved": stf, "peak": speak, "unit": "TFLOP/s",
                                  "frac": stf / speak, "alg_flops_per_launch": sflops,
                                  "time": "median"}}
        log(f"{c.name}: {sms:.3f} ms/step (median {smed:.3f}), "
            f"{c.B * c.T / sms / 1e3:.2f} M tokens/s, {stf:.1f} TFLOP/s of {speak:.0f}")
    del small_d
    tokens = cfg.T
    value = tokens / (ms / 1e3)
    alg_bytes = chunk_alg_bytes(x)
    alg_flops = chunk_alg_flops_per_head_token(cfg.dk, cfg.dv) * cfg.H * cfg.T
    gbs = alg_bytes / (ms / 1e3) / 1e9
    tflops = alg_flops / (ms / 1e3) / 1e12
    log(f"chunk_fwd: {ms:.3f} ms/step (median {ms_median:.3f}), {value / 1e6:.2f} M tokens/s, "
        f"{gbs:.0f} GB/s, {tflops:.1f} TFLOP/s, workspace {ws_bytes} bytes")
    result = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "ms_per_step_median": ms_median,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "H": cfg.H, "dk": cfg.dk, "dv": cfg.dv,
                   "T": cfg.T, "num_seqs": cfg.num_seqs, "gate": "per-key-channel",
                   "chunk": CHUNK, "state": "fp32", "qkvo": "bf16", "g_beta": "fp32"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic(),
                     "kernel": "kda chunk forward (segment plan: planner, items, segment chain, corrections)",
                     "alg_bytes_per_launch": alg_bytes, "workspace_bytes": ws_bytes},
        "mfma": {"achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": tflops / MFMA_BF16_PEAK_TFLOPS, "alg_flops_per_launch": alg_flops},
    }
    if not args.no_decode:
        dcfg = KDA_DECODE_N256_H32
        sec, gsec = bench_decode(torch, kda, dcfg)
        per_step = decode_alg_bytes_per_step(dcfg.B, dcfg.H, dcfg.dk, dcfg.dv)
        dgbs = per_step * dcfg.T / sec / 1e9
        result["decode"] = {
            "workload": dcfg.name, "steps": dcfg.T, "us_per_step": sec / dcfg.T * 1e6,
            "tokens_per_s": dcfg.B * dcfg.T / sec, "hbm_gbs": dgbs,
            "frac": dgbs / HBM_PEAK_GBS, "alg_bytes_per_step": per_step,
            "graph_us_per_step": gsec / dcfg.T * 1e6}
        log(f"decode: {sec / dcfg.T * 1e6:.1f} us/step, {dgbs:.0f} GB/s")
    if not args.no_gdr2:
        # Gated Delta Rule-2 on the same workloads: vector erase / write gates
        gcfg = cfg.replace(name="gdr2_bf16_varlen_h32_t65536", gates="gdr2")
        t0 = time.time()
        gx = make_chunk_inputs(gcfg)
        log(f"generated {gcfg.name} in {time.time() - t0:.1f}s")
        gd = device_inputs(torch, gx, cotangents=not args.no_bwd)
        if not args.no_bwd:  # timed first, as for KDA above
            gbms, _ = bench_bwd(torch, kda, gx, gd, args.steps, args.warmup)
        gms, gmed, _ = bench_chunk(torch, kda, gx, args.steps, args.warmup, gd)
        del gd
        gbytes = chunk_alg_bytes(gx)
        ggbs = gbytes / (gms / 1e3) / 1e9
        result["gdr2"] = {
            "workload": gcfg.name, "ms_per_step": gms, "ms_per_step_median": gmed,
            "tokens_per_s": gcfg.T / (gms / 1e3),
            "roofline": {"bound": "hbm", "achieved": ggbs, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": ggbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic(MEASURED_TRAFFIC_GDR2),
                         "alg_bytes_per_launch": gbytes}}
        log(f"gdr2 chunk_fwd: {gms:.3f} ms/step, {gcfg.T / gms / 1e3:.2f} M tokens/s, "
            f"{ggbs:.0f} GB/s")
        if not args.no_bwd:
            result["gdr2"]["bwd"] = {"ms_per_step": gbms, "tokens_per_s": gcfg.T / (gbms / 1e3)}
            log(f"gdr2 chunk_bwd: {gbms:.3f} ms/step")
        del gx
        if not args.no_decode:
            gd = KDA_DECODE_N256_H32.replace(name="gdr2_decode_n256_h32", gates="gdr2")
            sec, _ = bench_decode(torch, kda, gd)
            per_step = decode_alg_bytes_per_step(gd.B, gd.H, gd.dk, gd.dv, gdr2=True)
            dgbs = per_step * gd.T / sec / 1e9
            result["gdr2"]["decode"] = {
                "workload": gd.name, "steps": gd.T, "us_per_step": sec / gd.T * 1e6,
                "hbm_gbs": dgbs, "frac": dgbs / HBM_PEAK_GBS, "alg_bytes_per_step": per_step}
            log(f"gdr2 decode: {sec / gd.T * 1e6:.1f} us/step, {dgbs:.0f} GB/s")
    result["small_configs"] = small
    if not args.no_bwd:
        bbytes = bwd_alg_bytes(x)
        bgbs = bbytes / (bms / 1e3) / 1e9
        result["bwd"] = {
            "workload": cfg.name, "ms_per_step": bms, "tokens_per_s": cfg.T / (bms / 1e3),
            "workspace_bytes": bwsb,
            "roofline": {"bound": "hbm", "achieved": bgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": bgbs / HBM_PEAK_GBS, "alg_bytes_per_launch": bbytes,
                         "traffic": measured_traffic(MEASURED_TRAFFIC_BWD, BWD_KERNEL_SRC)}}
        log(f"chunk_bwd: {bms:.3f} ms/step, {cfg.T / bms / 1e3:.2f} M tokens/s, {bgbs:.0f} GB/s")
    if not args.no_gates:
        result["gates"] = dict(workload=cfg.name, **bench_gates(torch, kda, cfg, args.steps,
                                                                 args.warmup))
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(x, args.cpu_chains)
        log(f"cpu baseline: {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
