"""Benchmark: prefill tokens/s of the 3:1 linear:sparse SALA layer group at 256K tokens on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode]

A step is one pass of the hot path over one batch of synthetic input with
everything already resident in HBM:
  3 x linear prefill  (B=1, H=32, N=262144, d=128, chunk 128, slope decay)
  1 x sparse select   (Hq=32, Hkv=2, block 64, top-64 + 1 initial + 2 local)
  1 x sparse prefill  (attention over the selected blocks)
all on one stream.  value = 262144 tokens / step time.

The JSON line also carries:
  roofline      the dominant kernel (block-sparse attention, MFMA-bound):
                algorithmic flops 4*d*Hq*sum_t |A(t)| per launch / its average
                duration from HIP events on its stream over the timed steps
  cpu_baseline  the float64 oracle timed on the host on a bounded sample of the
                same workload, scaled to tokens/s of the whole group
  decode        the 1M-context decode step (3 linear decode + select over 16384
                pooled blocks + attention over 67 blocks, B=4) against HBM peak
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# HBM traffic of one sparse_attn_bf16 launch at the 256K workload, from two
# rocprofv3 --pmc runs of `python bench.py --steps 1 --warmup 0
# --no-cpu-baseline --no-decode` (FETCH_SIZE, then WRITE_SIZE, KiB per
# dispatch), each scaled by what the same counter reads for a plain 1 GiB
# device copy (FETCH_SIZE reads 0.5 GiB -> x2.0; WRITE_SIZE reads 1 GiB ->
# x1.0); summary in profiles/sparse_attn_256K_hbm_traffic.md.  It holds only
# for the kernel sources it was measured on: reported as null otherwise.
TRAFFIC_MEASURED = {
    "sources_sha256": "c13d06fd98b00d768e3a9c2f18b4fdb618d390e5aad7562ecb6f0dc29f0c7810",
    "fetch_kib": 8780152.375, "fetch_scale": 2.0,
    "write_kib": 2097208.03125, "write_scale": 1.0,
}
# Fraction of the cycles in which the MFMA pipes are busy while
# sparse_attn_bf16 runs at 256K (SQ_VALU_MFMA_BUSY_CYCLES over the cycles its
# workgroups are resident; profiles/sparse_attn_and_linear_256K_sq_counters.md).
# That is its MFMA efficiency at the clock it actually runs at, so a clock
# reading that would put the efficiency well above it was not taken while the
# kernel ran.
MFMA_BUSY_MEASURED = 0.569
TRAFFIC_SOURCES = ("hybrid_sparse_linear_amd/csrc/sparse_prefill.hip", "hybrid_sparse_linear_amd/csrc/sala_common.hpp")


class ClockSampler:
    """Samples the GPU shader clock (MHz, through torch.cuda.clock_rate) from
    a host thread while the timed steps run.  The published peaks are quoted
    at 2400 MHz; the median of the busy samples (>= 500 MHz, the lowest busy
    level) is the clock the kernels actually ran at, or None when the clock
    cannot be read."""

    def __init__(self, torch, period_s=0.05):
        import threading
        self.torch, self.period, self.samples, self.error = torch, period_s, [], None
        try:
            torch.cuda.clock_rate(0)  # the first query sets up amd-smi (slow); keep it out of the timed steps
        except Exception as e:
            self.error = repr(e)[:200]
        self.stop = threading.Event()
        self.thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self.stop.is_set():
            try:
                self.samples.append(int(self.torch.cuda.clock_rate(0)))
            except Exception as e:
                self.error = repr(e)[:200]
                return
            self.stop.wait(self.period)

    def __enter__(self):
        self.thread.start()
        return self

    def __exit__(self, *exc):
        self.stop.set()
        self.thread.join()

    def mhz(self):
        busy = sorted(c for c in self.samples if c >= 500)
        return busy[len(busy) // 2] if busy else None


def measured_traffic_bytes():
    """Counter-measured HBM bytes per sparse_attn_bf16 launch, or None when the
    kernel sources differ from the ones the counters were taken on."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(root, rel), "rb") as f:
            h.update(f.read())
    t = TRAFFIC_MEASURED
    if h.hexdigest() != t["sources_sha256"]:
        return None
    return int(1024 * (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--tokens", type=int, default=262144)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-attention comparison")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured-ceiling microkernels")
    ap.add_argument("--no-neighbours", action="store_true", help="skip the fused / unfused neighbour comparison")
    ap.add_argument("--cpu-sample-seconds", type=float, default=20.0)
    return ap.parse_args()


def sparse_flops(idx, N, d, G, block=64):
    """4 * d * sum over query rows of |A(t)|, from the actual selection (host)."""
    import numpy as np
    ix = idx.cpu().numpy()
    B, Hkv, NQB, _ = ix.shape
    total = 0
    for i in range(NQB):
        t0, t1 = i * block, min((i + 1) * block, N)
        rows = t1 - t0
        sel = ix[:, :, i, :]
        valid = (sel >= 0) & (sel <= i)
        n_full = (valid & (sel < i)).sum(axis=-1)            # blocks wholly before the query block
        has_diag = (valid & (sel == i)).any(axis=-1)
        per_bh = n_full * block * rows + has_diag * (rows * (rows + 1) // 2)
        total += int(per_bh.sum())
    return 4.0 * d * G * total


def cpu_baseline(lin_inputs, sp_inputs, idx, seconds):
    """Time the oracle on a bounded sample of the group and scale to tokens/s."""
    cores = len(os.sched_getaffinity(0))
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ.setdefault(var, str(cores))
    import numpy as np
    import torch
    from oracle import linear as OL
    from oracle import sparse as OS
    torch.set_num_threads(cores)

    N = sp_inputs["q"].shape[2]
    H = lin_inputs[0]["q"].shape[1]
    share = seconds / 3.0  # each of the three parts samples until it has used its share
    # linear: chunked form, head after head over the sample's tokens (cost is linear in tokens)
    x = lin_inputs[0]
    n_lin = x["q"].shape[2]
    lin_heads = 0
    t_lin = 0.0
    while lin_heads < H and (lin_heads == 0 or t_lin < share):
        q = x["q"][0, lin_heads].double().cpu().numpy()
        k = x["k"][0, lin_heads].double().cpu().numpy()
        v = x["v"][0, lin_heads].double().cpu().numpy()
        lam = float(x["decay"][lin_heads])
        t0 = time.perf_counter()
        OL.linear_attention_chunked(q, k, v, lam, 128)
        t_lin += time.perf_counter() - t0
        lin_heads += 1
    t_lin_tok_head = t_lin / (n_lin * lin_heads)

    # sparse: rows of query blocks deep in the sequence (67 blocks each), one KV group
    sq, sk, sv = sp_inputs["q"], sp_inputs["k"], sp_inputs["v"]
    Hq, Hkv, d = sq.shape[1], sk.shape[1], sq.shape[3]
    G = Hq // Hkv
    kbar = OS.pool_blocks(sk[0, 0].double().cpu().numpy(), 64)
    nb = kbar.shape[0]
    ix = idx.cpu().numpy()
    # selection: query blocks from the end of the context backwards (pooled
    # query, scores against all blocks, top-k), until the share is used
    sample_blocks = []
    t_sel = 0.0
    for i in range(nb - 1, 66, -1):
        t0 = time.perf_counter()
        qb = sq[0, :G, i * 64:(i + 1) * 64].double().cpu().numpy().reshape(-1, d).mean(axis=0)
        s = (kbar @ qb) / math.sqrt(d)
        OS.select_row(s, i, N, 64, 64, 1, 2)
        t_sel += time.perf_counter() - t0
        sample_blocks.append(i)
        if t_sel >= share:
            break
    t_sel_row = t_sel / len(sample_blocks)
    # restricted softmax: rows of those blocks (67 selected blocks each), both
    # KV groups, three rows per block and head, until the share is used
    rows = [(0, h, i * 64 + r) for i in sample_blocks for h in (0, G) for r in (0, 31, 63)]
    t0 = time.perf_counter()
    n_rows = 0
    for (b, h, t) in rows:
        i = t // 64
        blocks = [int(j) for j in ix[0, h // G, i] if j >= 0]
        toks = np.concatenate([np.arange(j * 64, min((j + 1) * 64, N)) for j in blocks])
        toks = toks[toks <= t]
        ti = torch.from_numpy(toks).to(sk.device)
        kk = sk[0, h // G, ti].double().cpu().numpy()
        vv = sv[0, h // G, ti].double().cpu().numpy()
        logit = (kk @ sq[0, h, t].double().cpu().numpy()) / math.sqrt(d)
        logit -= logit.max()
        p = np.exp(logit)
        (p / p.sum()) @ vv
        n_rows += 1
        if time.perf_counter() - t0 >= share:
            break
    t_att_row = (time.perf_counter() - t0) / n_rows
    nqb = (N + 63) // 64
    total = 3 * H * N * t_lin_tok_head + Hkv * nqb * t_sel_row + Hq * N * t_att_row
    return {"value": N / total, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"float64 oracle on the host, up to {seconds:.0f} s of it: chunked linear form over {n_lin} "
                       f"tokens of {lin_heads} heads ({t_lin_tok_head * 1e6:.2f} us/token/head); selection of "
                       f"{len(sample_blocks)} query blocks at the end of the 256K context ({t_sel_row * 1e3:.2f} ms/row); "
                       f"restricted softmax for {n_rows} query rows of 67 blocks ({t_att_row * 1e3:.2f} ms/row); "
                       f"scaled to 3 linear layers x 32 heads x N + 2 x 4096 selection rows + 32 x N attention rows")}


def measure_ceilings(torch, sala):
    """This GPU's practical ceilings from the two in-repo microkernels: an MFMA
    loop (bf16 16x16x32) and a streaming copy of 1 GiB.  Best of a few reps."""
    wgs, iters = 256 * 2, 20000
    out = torch.empty(wgs * 512, dtype=torch.float32, device="cuda")
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)

    def best(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(reps):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            torch.cuda.synchronize()
            t.append(s.elapsed_time(e) * 1e-3)
        return min(t)

    t_mfma = best(lambda: sala.ceiling_mfma(wgs, iters, out))
    t_copy = best(lambda: sala.ceiling_copy(src, dst))
    mfma = wgs * 8 * iters * 8 * 16384 / t_mfma / 1e12
    copy = 2 * src.numel() * 4 / t_copy / 1e9
    del out, src, dst
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(mfma, 1), "copy_gbs": round(copy, 1),
            "method": "in-repo microkernels: 512 workgroups x 8 waves x 20000 rounds of 8 independent bf16 MFMA "
                      "16x16x32; 1 GiB device copy, one contiguous 16 KiB run per workgroup with nontemporal 16-byte "
                      "loads/stores (read + write bytes); best of 5"}


def bench_dense(torch, sala, sp, group_ms):
    """The full-attention layer the sparse layer replaces: causal attention over
    every earlier token at the same shapes, one timed launch after one warmup."""
    q, k, v = sp["q"], sp["k"], sp["v"]
    B, Hq, N, d = q.shape
    o = torch.empty_like(q)
    sala.dense_prefill(q, k, v, out=o)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    sala.dense_prefill(q, k, v, out=o)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e)
    flops = 4 * d * Hq * B * N * (N + 1) / 2  # QK^T and PV over the causal half
    return {"workload": "dense causal attention, Hq=32, Hkv=2, d=128, N=%d (bf16)" % N, "ms": round(ms, 2),
            "tflop": round(flops / 1e12, 1), "achieved_tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "frac_of_peak": round(flops / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4),
            "group_speedup_vs_4_dense_layers": round(4 * ms / group_ms, 2),
            "note": "attention ops only: the 3:1 group time against four full-attention layers at 256K"}


def bench_neighbours(torch, sala, I, x, N, reps=3):
    """One linear layer at the group shapes with its neighbours (QK RMS norm,
    rotate-half RoPE, output gate): fused into the layer's kernels, against the
    unfused pipeline of standalone kernels (norm+RoPE of q, of k, the plain
    layer, the gate) and the plain layer alone.  Mean of `reps` after a warmup."""
    nb = I.neighbour_inputs(1, 32, N, 128, 4, 0, "cuda")
    q, k, v, dec, o, ws = x["q"], x["k"], x["v"], x["decay"], x["o"], x["ws"]
    qh, kh = torch.empty_like(q), torch.empty_like(k)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps

    def fused():
        sala.linear_prefill_fused(q, k, v, dec, gamma_q=nb["gamma_q"], gamma_k=nb["gamma_k"], rope_base=10000.0,
                                  gate=nb["gate"], out=o, workspace=ws, want_state=False)

    def unfused():
        sala.qk_norm_rope(q, gamma=nb["gamma_q"], rope_base=10000.0, out=qh)
        sala.qk_norm_rope(k, gamma=nb["gamma_k"], rope_base=10000.0, out=kh)
        sala.linear_prefill(qh, kh, v, dec, out=o, workspace=ws, want_state=False)
        sala.output_gate(o, nb["gate"], out=o)

    def plain():
        sala.linear_prefill(q, k, v, dec, out=o, workspace=ws, want_state=False)

    t_f, t_u, t_p = timed(fused), timed(unfused), timed(plain)
    tensor = 32 * N * 128 * 2
    # q, k, v, gate read and o written; the aggregate pass reads k and v again (all but the last segment)
    fused_bytes = 5 * tensor + 2 * tensor * 31 // 32
    del qh, kh, nb
    torch.cuda.empty_cache()
    return {"workload": "one linear layer, H=32, d=128, N=%d, bf16: QK RMS norm + RoPE (base 1e4) + output gate" % N,
            "fused_ms": round(t_f, 3), "unfused_ms": round(t_u, 3), "plain_layer_ms": round(t_p, 3),
            "fused_speedup_vs_unfused": round(t_u / t_f, 3),
            "fused_algorithmic_bytes": fused_bytes,
            "fused_hbm_tbs": round(fused_bytes / (t_f * 1e-3) / 1e12, 3),
            "fused_hbm_frac": round(fused_bytes / (t_f * 1e-3) / (PEAK_HBM_GBS * 1e9), 4)}


def bench_decode(torch, sala, I, reps=20):
    lin, sp = I.workload5_decode("cuda")
    for x in lin:
        x["decay"] = x["decay"].cuda()
        x["o"] = torch.empty_like(x["q"])
    L = sp["L"]
    q = sp["q"]
    q4 = q[:, :, None].contiguous()
    idx, kp = sala.sparse_select(q4, sp["k_cache"])  # pooled cache built once, outside the timed region
    ws_sel = torch.zeros(sala.workspace_bytes("sparse_select", dtype=1, B=4, Hq=32, Hkv=2, d=128, Nq=1, L=L,
                                              block=64, topk=64, n_init=1, n_local=2), dtype=torch.uint8,
                         device="cuda")
    ws_att = torch.empty(sala.workspace_bytes("sparse_decode", dtype=1, B=4, Hq=32, Hkv=2, L=L, d=128, block=64,
                                              n_sel=67), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    # Cold caches between reps: READ a 1 GiB buffer.  Reading leaves L2 and the
    # 256 MB MALL full of clean, unrelated lines.  A 1 GiB write would instead
    # leave up to 256 MB of dirty lines whose write-back the next kernel pays for.
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.zeros((), dtype=torch.float32, device="cuda")

    def step():
        for x in lin:
            sala.linear_decode(x["q"], x["k"], x["v"], x["state"], x["decay"], out=x["o"])
        sala.sparse_select(q4, None, k_pooled=kp, L=L, idx_out=idx, workspace=ws_sel)
        sala.sparse_decode(q, sp["k_cache"], sp["v_cache"], idx[:, :, 0], L=L, out=o, workspace=ws_att)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    o_eager = o.clone()
    # The step is five short kernels; launching them from Python one by one
    # would time the host.  Capture the step once in a HIP graph and replay it.
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    graph.replay()
    torch.cuda.synchronize()
    replay_ok = bool(torch.equal(o, o_eager))  # the sparse output does not depend on the linear states
    times = []
    for _ in range(reps):
        sink.add_(flush.sum())  # evict L2 and MALL with clean lines
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        graph.replay()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e) * 1000.0)
    times.sort()
    us = times[len(times) // 2]
    nbytes = 3 * (2 * 4 * 32 * 128 * 128 * 4) + 4 * 2 * 16384 * 128 * 4 + 4 * 2 * 67 * 64 * 128 * 2 * 2
    out = {"workload": "decode step at L=1048576, B=4: 3 linear decode (H=32, d=128 fp32 state) + select over "
                       "16384 pooled blocks + attention over 64+1+2 blocks (Hq=32, Hkv=2)",
           "us_per_step_median": round(us, 2), "algorithmic_bytes": nbytes,
           "hbm_frac": round(nbytes / (us * 1e-6) / (PEAK_HBM_GBS * 1e9), 4),
           "timing": "HIP events around one replay of the captured step (HIP graph), median of 20 reps, "
                     "1 GiB read between reps", "graph_replay_matches_eager": replay_ok}

    # The same step as a generation loop runs it: the linear layers with QK norm,
    # RoPE at position L-1 and the gate fused in, and the sparse layer appending
    # the token's k, v to the cache and updating its block's pooled key first.
    nb = I.neighbour_inputs(4, 32, 1, 128, 5, 0, "cuda")
    gate = nb["gate"][:, :, 0].contiguous()
    pos = torch.full((4,), L - 1, dtype=torch.int64, device="cuda")
    k_new = sp["k_cache"][:, :, L - 1].clone()
    v_new = sp["v_cache"][:, :, L - 1].clone()
    idx1 = torch.empty((4, 2, 67), dtype=torch.int32, device="cuda")
    o2 = torch.empty_like(q)
    ws_step = torch.empty(sala.workspace_bytes("sparse_decode_step", dtype=1, B=4, Hq=32, Hkv=2, capacity=L, d=128,
                                               block=64, topk=64, n_init=1, n_local=2), dtype=torch.uint8,
                          device="cuda")

    def gen_step():
        for x in lin:
            sala.linear_decode_fused(x["q"], x["k"], x["v"], x["state"], x["decay"], gamma_q=nb["gamma_q"],
                                     gamma_k=nb["gamma_k"], rope_base=10000.0, pos=pos, gate=gate, out=x["o"])
        sala.sparse_decode_step(q, k_new, v_new, sp["k_cache"], sp["v_cache"], kp, L - 1, idx_out=idx1, out=o2,
                                workspace=ws_step)

    for _ in range(3):
        gen_step()
    torch.cuda.synchronize()
    gen_ok = bool(torch.equal(o2, o_eager))  # the appended token equals the cache's last row
    graph2 = torch.cuda.CUDAGraph()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gen_step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph2):
        gen_step()
    graph2.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        sink.add_(flush.sum())
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        graph2.replay()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e) * 1000.0)
    times.sort()
    out["generation_step"] = {
        "workload": "the same step inside a generation loop: fused linear decode (QK RMS norm, RoPE at L-1, gate) "
                    "x3 + sala_sparse_decode_step (append k, v at L-1, pooled-key update, select, attend)",
        "us_per_step_median": round(times[len(times) // 2], 2), "matches_plain_step": gen_ok}
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: libsala has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import hybrid_sparse_linear_amd as sala
    from hybrid_sparse_linear_amd import inputs as I
    torch.cuda.set_device(0)
    N = args.tokens
    lin, sp = I.workload4_group("cuda", N)
    for x in lin:
        x["decay"] = x["decay"].cuda()
        x["o"] = torch.empty_like(x["q"])
        x["ws"] = torch.empty(max(1, sala.workspace_bytes("linear_prefill", dtype=1, B=1, H=32, N=N, d=128,
                                                          chunk=128)), dtype=torch.uint8, device="cuda")
    Hq, Hkv, d = sp["q"].shape[1], sp["k"].shape[1], sp["q"].shape[3]
    nqb = (N + 63) // 64
    idx = torch.empty((1, Hkv, nqb, 67), dtype=torch.int32, device="cuda")
    kp = torch.empty((1, Hkv, nqb, d), dtype=torch.float32, device="cuda")
    ws_sel = torch.zeros(sala.workspace_bytes("sparse_select", dtype=1, B=1, Hq=Hq, Hkv=Hkv, d=d, Nq=N, L=N,
                                              block=64, topk=64, n_init=1, n_local=2), dtype=torch.uint8,
                         device="cuda")
    ws_att = torch.empty(sala.workspace_bytes("sparse_prefill", dtype=1, B=1, Hq=Hq, Hkv=Hkv, N=N, d=d, block=64,
                                              n_sel=67), dtype=torch.uint8, device="cuda")
    o_sp = torch.empty_like(sp["q"])
    stream = torch.cuda.current_stream()
    ev = []

    def step(record=False):
        for x in lin:
            sala.linear_prefill(x["q"], x["k"], x["v"], x["decay"], out=x["o"], workspace=x["ws"], want_state=False)
        sala.sparse_select(sp["q"], sp["k"], k_pooled=kp, idx_out=idx, workspace=ws_sel)
        if record:
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
        sala.sparse_prefill(sp["q"], sp["k"], sp["v"], idx, out=o_sp, workspace=ws_att)
        if record:
            e.record(stream)
            ev.append((s, e))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(record=True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # the sparse kernel's own clock: back-to-back launches for at least 0.6 s
    # (at least ten) with the sampler on
    with ClockSampler(torch, period_s=0.02) as sclock:
        t_clk, n_clk = time.perf_counter() + 0.6, 0
        while n_clk < 10 or time.perf_counter() < t_clk:
            sala.sparse_prefill(sp["q"], sp["k"], sp["v"], idx, out=o_sp, workspace=ws_att)
            torch.cuda.synchronize()
            n_clk += 1
    sclk = sclock.mhz()
    ms = elapsed * 1000.0 / args.steps
    att_ms = sum(s.elapsed_time(e) for s, e in ev) / len(ev)
    flops = sparse_flops(idx, N, d, Hq // Hkv)
    group_flops = 3 * (32 * N * (2 * 128 * 128 + 4 * 128 * 128)) * 1.0 + flops  # algorithmic (causal) counts
    achieved = flops / (att_ms * 1e-3) / 1e12
    sclk_note = None
    if sclk and achieved / (PEAK_BF16_TFLOPS * sclk / 2400.0) > MFMA_BUSY_MEASURED + 0.1:
        # the rate needs a faster clock than the one read: the readings came
        # from between launches (as under a profiler that serialises them) or
        # the driver reported another clock
        sclk_note = ("a reading of %d MHz would put the kernel at %.2f MFMA efficiency, above the %.3f MFMA-busy "
                     "fraction the counters measure: not the kernel's clock" %
                     (sclk, achieved / (PEAK_BF16_TFLOPS * sclk / 2400.0), MFMA_BUSY_MEASURED))
        sclk = None
    traffic = measured_traffic_bytes() if N == 262144 else None
    # unique bytes: Q read and O written once; K and V of the KV heads read once
    alg_bytes = 2 * (Hq * N * d * 2) + 2 * (Hkv * N * d * 2)
    out = {
        "metric": "prefill tokens/s for 3:1 linear:sparse layer group at 256K; % MFMA/HBM peak",
        "value": round(N / (ms / 1000.0), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "SALA 3:1 layer-group prefill, B=1, N=%d: 3 linear layers (H=32, d=128, chunk 128, "
                               "decay exp(-2^(-(h+1)/4))) + 1 block-sparse layer (Hq=32, Hkv=2, d=128, block 64, "
                               "top-64 + 1 initial + 2 local)" % N,
                   "tokens": N, "batch": 1},
        "group_mfma_frac": round(group_flops / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4),
        "roofline": {"kernel": "sparse_attn_bf16", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "traffic_unit": "HBM bytes per launch (counters, N=262144 only)",
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "algorithmic_tflop_per_launch": round(flops / 1e12, 4), "avg_launch_ms": round(att_ms, 4),
                     "sclk_mhz": sclk, "sclk_samples": len(sclock.samples),
                     "frac_at_sclk": None if not sclk else round(achieved / (PEAK_BF16_TFLOPS * sclk / 2400.0), 4)},
    }
    if not args.no_dense:
        out["dense_comparison"] = bench_dense(torch, sala, sp, ms)
    if not args.no_neighbours:
        out["neighbours"] = bench_neighbours(torch, sala, I, lin[0], N)
    if not args.no_decode:
        del lin
        torch.cuda.empty_cache()
        out["decode"] = bench_decode(torch, sala, I)
    if not args.no_ceilings:
        out["ceilings"] = measure_ceilings(torch, sala)
        out["roofline"]["frac_of_measured_ceiling"] = round(achieved / out["ceilings"]["mfma_bf16_tflops"], 4)
    if not args.no_cpu_baseline:
        lin1 = [I.workload2_linear(0, "cuda", N=8192, workload=4)]
        out["cpu_baseline"] = cpu_baseline(lin1, sp, idx, args.cpu_sample_seconds)
    if out["roofline"]["sclk_mhz"] is None and sclock.error:
        out["roofline"]["sclk_error"] = sclock.error
    if sclk_note:
        out["roofline"]["sclk_note"] = sclk_note
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
