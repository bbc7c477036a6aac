"""Benchmark: prefill tokens/s of the 3:1 linear:sparse SALA layer group at 256K tokens on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode] [--no-configs]

A step is one pass of the hot path over one batch of synthetic input with
everything already resident in HBM, through the group entry point
(layer_group_prefill):
  3 x linear prefill  (B=1, H=32, N=262144, d=128, chunk 128, slope decay)
  1 x sparse select   (Hq=32, Hkv=2, block 64, top-64 + 1 initial + 2 local)
  1 x sparse prefill  (attention over the selected blocks)
all on one stream.  value = 262144 tokens / step time.

The JSON line also carries:
  roofline      the dominant kernel (block-sparse attention, MFMA-bound):
                algorithmic flops 4*d*Hq*sum_t |A(t)| per launch / its average
                duration from HIP events on its stream over the timed steps
  group         the whole step's algorithmic flops against the bf16 MFMA peak,
                next to the 40 % target
  cpu_baseline  the float64 oracle timed on the host on a bounded sample of the
                same workload (host copies made before any clock starts; only
                the oracle's own functions are timed), scaled to tokens/s
  configs       the other workloads: the tiny fp32 group, the 32K linear
                prefill, the 128K sparse layer and the 1M-context decode step,
                each with its GPU time, its roofline fraction on its
                algorithmic work and the oracle's rate on the same host
  decode        (also under configs) the 1M-context decode step against HBM
                peak, on summed per-call time and on wall time
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
# workgroups are resident; profiles/sparse_attn_linear_and_backward_256K_sq_counters.md).
# That is its MFMA efficiency at the clock it actually runs at, so a clock
# reading that would put the efficiency well above it was not taken while the
# kernel ran.  Like the traffic figure it holds only for the kernel sources it
# was measured on (same hash); otherwise no clock reading is set aside.
MFMA_BUSY_MEASURED = {"sources_sha256": "c13d06fd98b00d768e3a9c2f18b4fdb618d390e5aad7562ecb6f0dc29f0c7810",
                      "busy": 0.601}
TRAFFIC_SOURCES = ("hybrid_sparse_linear_amd/csrc/sparse_prefill.hip", "hybrid_sparse_linear_amd/csrc/sala_common.hpp")
GROUP_TARGET_FRAC = 0.40   # the group step's target fraction of the bf16 MFMA peak
DECODE_TARGET_FRAC = 0.60  # the 1M decode step's target fraction of the HBM peak


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


def sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic_bytes():
    """Counter-measured HBM bytes per sparse_attn_bf16 launch, or None when the
    kernel sources differ from the ones the counters were taken on."""
    t = TRAFFIC_MEASURED
    if sources_sha256() != t["sources_sha256"]:
        return None
    return int(1024 * (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]))


def measured_mfma_busy():
    """Counter-measured MFMA-busy fraction of sparse_attn_bf16, or None for other sources."""
    m = MFMA_BUSY_MEASURED
    return m["busy"] if sources_sha256() == m["sources_sha256"] else None


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
    ap.add_argument("--no-configs", action="store_true", help="skip the per-workload entries")
    ap.add_argument("--no-backward", action="store_true", help="skip the gradient (training) timings")
    ap.add_argument("--cpu-sample-seconds", type=float, default=8.0,
                    help="oracle time budget of each sampled part of the CPU baselines")
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


def host_cores():
    """(threads the oracle's BLAS actually uses, cores this process may run on)."""
    affinity = len(os.sched_getaffinity(0))
    try:
        import threadpoolctl
        n = max((lib.get("num_threads") or 0) for lib in threadpoolctl.threadpool_info()) or affinity
    except Exception:
        n = int(os.environ.get("OMP_NUM_THREADS", affinity))
    return n, affinity


class HostRows:
    """Host copies (float64, as the tests hand the oracle its inputs) of chosen
    token rows of a GPU tensor [B, H, L, d], made before any clock starts.  The
    oracle's functions index it as they index a full array: x[b, h, tokens]
    (tokens an int or an index array) and x[b, head slice, token slice].  Only
    indexing happens here."""

    def __init__(self, t, rows):
        import numpy as np
        import torch
        self.shape = tuple(t.shape)
        self.rows = {}
        for (b, h), toks in rows.items():
            toks = np.unique(np.asarray(toks, dtype=np.int64))
            data = t[b, h, torch.from_numpy(toks).to(t.device)].double().cpu().numpy()
            self.rows[(int(b), int(h))] = (toks, data)

    def _get(self, b, h, t):
        import numpy as np
        toks, data = self.rows[(int(b), int(h))]
        pos = np.minimum(np.searchsorted(toks, t), len(toks) - 1)
        if not np.all(toks[pos] == t):
            raise KeyError(f"rows of ({b}, {h}) asked for that were not copied")
        return data[pos]

    def __getitem__(self, key):
        import numpy as np
        b, h, t = key
        if isinstance(h, slice):
            ts = np.arange(*t.indices(self.shape[2]))
            return np.stack([self._get(b, hh, ts) for hh in range(*h.indices(self.shape[1]))])
        return self._get(b, h, t)


def oracle_linear_seconds(x, heads, n_tok, chunk=128):
    """Oracle seconds per (token, head) of the chunked linear form, on host float64
    copies of the first n_tok tokens of the given heads (copied before timing)."""
    from oracle import linear as OL
    dec = x["decay"].double().cpu().numpy()
    spent = 0.0
    for h in heads:
        q, k, v = (x[n][0, h, :n_tok].double().cpu().numpy() for n in ("q", "k", "v"))
        t0 = time.perf_counter()
        OL.linear_attention_chunked(q, k, v, float(dec[h]), chunk)
        spent += time.perf_counter() - t0
    return spent / (n_tok * len(heads))


def oracle_sparse_seconds(sp, idx, budget, n_blocks=96):
    """Oracle seconds of the sparse layer's parts on a sample of query blocks at the
    end of the context (each with its full candidate set and 67 selected blocks):
    pooling one KV head's keys, selecting one row (sparse_select_prefill_rows), and
    the restricted softmax of one query row (sparse_attention_prefill_rows).  Host
    copies are made first; the attention part samples rows until `budget` s."""
    import numpy as np
    from oracle import sparse as OS
    q, k, v = sp["q"], sp["k"], sp["v"]
    _, Hq, N, d = q.shape
    Hkv = k.shape[1]
    nqb = (N + 63) // 64
    blocks = list(range(nqb - 1, max(66, nqb - 1 - n_blocks), -1))
    toks = np.concatenate([np.arange(i * 64, min((i + 1) * 64, N)) for i in blocks])
    qrows = HostRows(q, {(0, h): toks for h in range(Hq)})
    kh, vh = k.double().cpu().numpy(), v.double().cpu().numpy()
    ih = idx.cpu().numpy()
    t0 = time.perf_counter()
    for h in range(Hkv):
        OS.pool_blocks(kh[0, h], 64)
    t_pool = (time.perf_counter() - t0) / Hkv
    t0 = time.perf_counter()
    OS.sparse_select_prefill_rows(qrows, kh, blocks, 64, 64, 1, 2)
    t_sel = max(time.perf_counter() - t0 - Hkv * t_pool, 0.0) / (Hkv * len(blocks))
    rng = np.random.default_rng(7)
    rows = [(0, int(h), int(i * 64 + r)) for i in blocks for h in rng.choice(Hq, 4, replace=False)
            for r in rng.choice(64, 4, replace=False)]
    n_rows, spent = 0, 0.0
    while n_rows < len(rows) and (n_rows == 0 or spent < budget):
        part = rows[n_rows:n_rows + 64]
        t0 = time.perf_counter()
        OS.sparse_attention_prefill_rows(qrows, kh, vh, ih, part, 64)
        spent += time.perf_counter() - t0
        n_rows += len(part)
    return {"pool_head_s": t_pool, "select_row_s": t_sel, "attn_row_s": spent / n_rows,
            "select_rows": len(blocks) * Hkv, "attn_rows": n_rows}


def oracle_sparse_layer_seconds(parts, N, Hq, Hkv):
    nqb = (N + 63) // 64
    return Hkv * parts["pool_head_s"] + Hkv * nqb * parts["select_row_s"] + Hq * N * parts["attn_row_s"]


def cpu_baseline(lin, sp, idx, budget):
    """The oracle on the group workload: the chunked linear form over the first
    8192 tokens of all 32 heads of one linear layer, and the sparse layer's
    pooling, selection and restricted softmax on query blocks at the end of the
    context; scaled to the whole group (3 linear layers + 1 sparse layer)."""
    N = sp["q"].shape[2]
    H = lin[0]["q"].shape[1]
    Hq, Hkv = sp["q"].shape[1], sp["k"].shape[1]
    n_tok = 8192
    t_lin = oracle_linear_seconds(lin[0], range(H), n_tok)
    parts = oracle_sparse_seconds(sp, idx, budget)
    total = 3 * H * N * t_lin + oracle_sparse_layer_seconds(parts, N, Hq, Hkv)
    cores, affinity = host_cores()
    return {"value": N / total, "unit": "tokens/s", "cores": cores, "affinity_cores": affinity, "kind": "oracle",
            "sample": (f"float64 oracle functions on host copies made before timing: chunked linear form over "
                       f"{n_tok} tokens x {H} heads ({t_lin * 1e6:.2f} us/token/head); pooling of a KV head "
                       f"({parts['pool_head_s'] * 1e3:.0f} ms); selection of {parts['select_rows']} query-block rows at "
                       f"the end of the context ({parts['select_row_s'] * 1e3:.3f} ms/row); restricted softmax of "
                       f"{parts['attn_rows']} query rows over 67 blocks ({parts['attn_row_s'] * 1e3:.3f} ms/row); "
                       f"scaled to 3 linear layers x {H} heads x N + {Hkv} pooled heads + {Hkv} x {N // 64} "
                       f"selection rows + {Hq} x N attention rows (rows of the first 66 query blocks, which attend "
                       f"fewer blocks, priced as full rows)")}


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
    # q, k, v, gate read and o written (as for the plain layer, the aggregate
    # pass's second read of the keys that reach a segment end is not counted)
    fused_bytes = 5 * tensor
    del qh, kh, nb
    torch.cuda.empty_cache()
    return {"workload": "one linear layer, H=32, d=128, N=%d, bf16: QK RMS norm + RoPE (base 1e4) + output gate" % N,
            "fused_ms": round(t_f, 3), "unfused_ms": round(t_u, 3), "plain_layer_ms": round(t_p, 3),
            "fused_speedup_vs_unfused": round(t_u / t_f, 3),
            "fused_algorithmic_bytes": fused_bytes,
            "fused_hbm_tbs": round(fused_bytes / (t_f * 1e-3) / 1e12, 3),
            "fused_hbm_frac": round(fused_bytes / (t_f * 1e-3) / (PEAK_HBM_GBS * 1e9), 4)}


def events_ms(torch, fn, reps, before=None):
    """Median duration (ms) of fn from HIP events on the current stream; `before`
    runs untimed ahead of each rep."""
    st = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        if before is not None:
            before()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(st)
        fn()
        e.record(st)
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    times.sort()
    return times[len(times) // 2]


def oracle_entry(seconds, tokens):
    cores, affinity = host_cores()
    return {"value": tokens / seconds, "unit": "tokens/s", "cores": cores, "affinity_cores": affinity,
            "kind": "oracle"}


def bench_workload1(torch, sala, I, reps=20):
    """The tiny fp32 group (B=1, 4 heads, d=64, N=2048) through the group entry
    point; the oracle runs the whole workload as the parity tests do."""
    from oracle import linear as OL
    from oracle import sparse as OS
    lin_h = [I.workload1_linear(layer) for layer in range(3)]
    sp_h = I.workload1_sparse()
    lin = [{n: x[n].cuda() for n in ("q", "k", "v", "decay")} for x in lin_h]
    sp = {n: sp_h[n].cuda() for n in ("q", "k", "v")}
    out = {"linear": [torch.empty_like(x["q"]) for x in lin], "sparse": torch.empty_like(sp["q"]),
           "idx": torch.empty((1, 4, 32, 7), dtype=torch.int32, device="cuda"),
           "k_pooled": torch.empty((1, 4, 32, 64), dtype=torch.float32, device="cuda")}
    ws = {"select": torch.empty(sala.workspace_bytes("sparse_select", dtype=0, B=1, Hq=4, Hkv=4, d=64, Nq=2048, L=2048,
                                                     block=64, topk=4, n_init=1, n_local=2), dtype=torch.uint8,
                                device="cuda")}
    fn = lambda: sala.layer_group_prefill(lin, sp, topk=4, chunk=64, out=out, workspaces=ws)  # noqa: E731
    fn()
    ms = events_ms(torch, fn, reps)
    h = lambda t: t.double().numpy()  # noqa: E731
    lh = [(h(x["q"]), h(x["k"]), h(x["v"]), h(x["decay"])) for x in lin_h]
    qh, kh, vh = h(sp_h["q"]), h(sp_h["k"]), h(sp_h["v"])
    t0 = time.perf_counter()
    for q, k, v, dec in lh:
        OL.linear_prefill(q, k, v, dec)
    idx, _, _ = OS.sparse_select_prefill(qh, kh, 64, 4)
    OS.sparse_attention_prefill(qh, kh, vh, idx, 64)
    t_or = time.perf_counter() - t0
    return {"workload": "tiny group, fp32, B=1, N=2048: 3 linear layers (H=4, d=64, chunk 64, decay 1.0/0.99) + "
                        "1 sparse layer (4 heads, top-4 + 1 initial + 2 local)",
            "gpu_ms": round(ms, 4), "tokens_per_s": round(2048 / (ms * 1e-3), 1), "roofline": None,
            "roofline_note": "a correctness workload (fp32, 2048 tokens, the VALU paths): no roofline is claimed",
            "cpu_oracle": dict(oracle_entry(t_or, 2048), sample="the whole workload (quadratic linear form, full "
                                                                "selection, restricted softmax)")}


def bench_workload2(torch, sala, I, budget, reps=20):
    """Linear prefill only, bf16, B=1, H=32, d=128, N=32768, chunk 128 (HBM-bound)."""
    N, H, d = 32768, 32, 128
    x = I.workload2_linear(0, "cuda", N=N)
    x["decay"] = x["decay"].cuda()
    o = torch.empty_like(x["q"])
    ws = torch.empty(max(1, sala.workspace_bytes("linear_prefill", dtype=1, B=1, H=H, N=N, d=d, chunk=128)),
                     dtype=torch.uint8, device="cuda")
    fn = lambda: sala.linear_prefill(x["q"], x["k"], x["v"], x["decay"], out=o, workspace=ws,  # noqa: E731
                                     want_state=False)
    fn()
    ms = events_ms(torch, fn, reps)
    nbytes = 4 * N * H * d * 2
    heads = list(range(0, H, 8))
    t_tok = oracle_linear_seconds(x, heads, N)
    return {"workload": "linear prefill, bf16, B=1, H=32, d=128, N=32768, chunk 128, decay exp(-2^(-(h+1)/4))",
            "gpu_ms": round(ms, 4), "tokens_per_s": round(N / (ms * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(nbytes / (ms * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
                         "algorithmic_bytes": nbytes},
            "cpu_oracle": dict(oracle_entry(H * N * t_tok, N),
                               sample=f"chunked linear form over all {N} tokens of heads {heads} "
                                      f"({t_tok * 1e6:.2f} us/token/head), scaled to {H} heads")}


def bench_workload3(torch, sala, I, budget, reps=10):
    """Sparse layer only, bf16, B=1, Hq=32, Hkv=2, d=128, N=131072: selection
    (HBM-bound) and block-sparse attention (MFMA-bound), timed apart."""
    N = 131072
    sp = I.workload3_sparse(0, "cuda", N=N)
    q, k, v = sp["q"], sp["k"], sp["v"]
    Hq, Hkv, d = q.shape[1], k.shape[1], q.shape[3]
    nqb = N // 64
    idx = torch.empty((1, Hkv, nqb, 67), dtype=torch.int32, device="cuda")
    kp = torch.empty((1, Hkv, nqb, d), dtype=torch.float32, device="cuda")
    o = torch.empty_like(q)
    ws = torch.empty(sala.workspace_bytes("sparse_select", dtype=1, B=1, Hq=Hq, Hkv=Hkv, d=d, Nq=N, L=N, block=64,
                                          topk=64, n_init=1, n_local=2), dtype=torch.uint8, device="cuda")
    sel = lambda: sala.sparse_select(q, k, k_pooled=kp, idx_out=idx, workspace=ws)  # noqa: E731
    att = lambda: sala.sparse_prefill(q, k, v, idx, out=o)  # noqa: E731
    sel()
    att()
    ms_sel = events_ms(torch, sel, reps)
    ms_att = events_ms(torch, att, reps)
    flops = sparse_flops(idx, N, d, Hq // Hkv)
    sel_bytes = Hq * N * d * 2 + Hkv * N * d * 2 + Hkv * nqb * d * 4 + Hkv * nqb * 67 * 4
    parts = oracle_sparse_seconds(sp, idx, budget)
    t_or = oracle_sparse_layer_seconds(parts, N, Hq, Hkv)
    return {"workload": "sparse layer, bf16, B=1, Hq=32, Hkv=2, d=128, N=131072, block 64, top-64 + 1 + 2, "
                        "5% of key blocks shifted",
            "gpu_ms": round(ms_sel + ms_att, 4), "tokens_per_s": round(N / ((ms_sel + ms_att) * 1e-3), 1),
            "roofline": {"kernel": "sparse_attn_bf16", "bound": "mfma",
                         "achieved": round(flops / (ms_att * 1e-3) / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(flops / (ms_att * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4),
                         "algorithmic_tflop": round(flops / 1e12, 4), "ms": round(ms_att, 4)},
            "select_roofline": {"bound": "hbm", "achieved": round(sel_bytes / (ms_sel * 1e-3) / 1e9, 1),
                                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(sel_bytes / (ms_sel * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
                                "algorithmic_bytes": sel_bytes, "ms": round(ms_sel, 4)},
            "cpu_oracle": dict(oracle_entry(t_or, N),
                               sample=f"pooling ({parts['pool_head_s'] * 1e3:.0f} ms/head), {parts['select_rows']} "
                                      f"selection rows ({parts['select_row_s'] * 1e3:.3f} ms/row) and "
                                      f"{parts['attn_rows']} attention rows ({parts['attn_row_s'] * 1e3:.3f} ms/row) "
                                      f"at the end of the context, scaled to the layer")}


def bench_backward(torch, sala, I, x, sp, idx, reps=3):
    """The gradients of one linear layer and of the sparse layer at the group's
    shapes (N=262144), for dL/do ~ N(0, 1/d): sala_linear_prefill_backward
    (HBM-bound: q, k, v, dO read and dq, dk, dv written, 7 tensors of the layer's
    size) and sala_sparse_prefill_backward at the forward's selection
    (MFMA-bound: S, dP, dQ, dK and dV products, 10 d flops per (query row, key)
    pair of the selection).  Mean of `reps` after a warmup."""
    q, k, v = x["q"], x["k"], x["v"]
    B, H, N, d = q.shape
    do = I.normal((B, H, N, d), 4999, 1.0 / math.sqrt(d), I.BF16, "cuda")
    grads = [torch.empty_like(q) for _ in range(3)]
    ws = torch.empty(max(1, sala.workspace_bytes("linear_prefill", dtype=1, B=B, H=H, N=N, d=d, chunk=128)),
                     dtype=torch.uint8, device="cuda")
    lin = lambda: sala.linear_prefill_backward(q, k, v, do, x["decay"], dq=grads[0], dk=grads[1],  # noqa: E731
                                               dv=grads[2], want_dstate=False, workspace=ws, chunk=128)
    lin()
    ms_lin = events_ms(torch, lin, reps)
    # the same gradients in 64-token chunks, where dK and dV come from one pass
    ws64 = torch.empty(max(1, sala.workspace_bytes("linear_prefill", dtype=1, B=B, H=H, N=N, d=d, chunk=64)),
                       dtype=torch.uint8, device="cuda")
    lin64 = lambda: sala.linear_prefill_backward(q, k, v, do, x["decay"], dq=grads[0], dk=grads[1],  # noqa: E731
                                                 dv=grads[2], want_dstate=False, workspace=ws64, chunk=64)
    lin64()
    ms_lin64 = events_ms(torch, lin64, reps)
    del grads, ws, ws64
    sq, sk, sv = sp["q"], sp["k"], sp["v"]
    Hq, Hkv = sq.shape[1], sk.shape[1]
    sdo = I.normal(sq.shape, 5000, 1.0 / math.sqrt(d), I.BF16, "cuda")
    sdq, sdk, sdv = torch.empty_like(sq), torch.empty_like(sk), torch.empty_like(sk)
    sws = torch.empty(sala.workspace_bytes("sparse_prefill_backward", dtype=1, B=B, Hq=Hq, Hkv=Hkv, N=N, d=d,
                                           block=64, n_sel=idx.shape[-1]), dtype=torch.uint8, device="cuda")
    spb = lambda: sala.sparse_prefill_backward(sq, sk, sv, idx, sdo, dq=sdq, dk=sdk, dv=sdv,  # noqa: E731
                                               workspace=sws)
    spb()
    ms_sp = events_ms(torch, spb, reps)
    lin_bytes = 7 * B * H * N * d * 2
    sp_flops = sparse_flops(idx, N, d, Hq // Hkv) * 10.0 / 4.0  # forward's 4 d per pair -> 10 d
    del sdo, sdq, sdk, sdv, sws, do
    torch.cuda.empty_cache()
    return {"workload": "gradients at the group shapes, N=%d: one linear layer (H=32, d=128, slope decay; chunk 128 as "
                        "in the forward, and chunk 64, where dK and dV come from one pass) and the sparse layer at "
                        "its forward selection (Hq=32, Hkv=2, 67 blocks)" % N,
            "linear_layer_ms": round(ms_lin, 3),
            "linear_roofline": {"bound": "hbm", "achieved": round(lin_bytes / (ms_lin * 1e-3) / 1e9, 1),
                                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(lin_bytes / (ms_lin * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
                                "algorithmic_bytes": lin_bytes},
            "linear_layer_chunk64_ms": round(ms_lin64, 3),
            "linear_chunk64_hbm_frac": round(lin_bytes / (ms_lin64 * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
            "sparse_layer_ms": round(ms_sp, 3),
            "sparse_roofline": {"bound": "mfma", "achieved": round(sp_flops / (ms_sp * 1e-3) / 1e12, 1),
                                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                "frac": round(sp_flops / (ms_sp * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4),
                                "algorithmic_tflop": round(sp_flops / 1e12, 3)},
            "group_backward_ms": round(3 * ms_lin + ms_sp, 3),
            "timing": "HIP events, mean of %d after a warmup" % reps}


def decode_floors(torch, sala, flush, sink, reps):
    """What the decode step's launches would cost if each only streamed its bytes:
    per call, the same number of launches of the in-repo streaming microkernels,
    each moving that kernel's bytes (a copy of the 8.4 MB of linear states, read
    and written; a read of the 67.1 MB of pooled keys and an empty launch for the
    selection's merge; reads of the 17.6 MB of selected K, V rows and of the
    4.5 MB of partials for the attention), timed like the calls themselves."""
    MB = 1 << 20
    st_bytes = 4 * 32 * 128 * 128 * 4
    sizes = {"linear_decode": [("copy", st_bytes)], "sparse_select": [("read", 4 * 2 * 16384 * 128 * 4), ("read", 0)],
             "sparse_decode": [("read", 4 * 2 * 67 * 64 * 128 * 2 * 2), ("read", 4 * 32 * 67 * 130 * 4)]}
    pool = torch.empty(2 * st_bytes + 96 * MB, dtype=torch.uint8, device="cuda")
    out_f = torch.empty(96 * MB // 16384 + 1, dtype=torch.float32, device="cuda")
    src_c, dst_c = pool[:st_bytes], pool[st_bytes:2 * st_bytes]
    rd = pool[2 * st_bytes:]

    def launches(name):
        off = 0
        for kind, nb in sizes[name]:
            if kind == "copy":
                sala.ceiling_copy(src_c, dst_c)
            else:
                sala.ceiling_read(rd[off:], out_f, nb)
                off += (nb + MB - 1) // MB * MB
    names = list(sizes)
    per = {n: [] for n in names}
    for _ in range(3):
        for n in names:
            launches(n)
    torch.cuda.synchronize()
    for _ in range(reps):
        sink.add_(flush.sum())
        sink.add_(flush.sum())
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 2)]
        evs[0].record()
        for n, name in enumerate(names):
            launches(name)
            evs[n + 1].record()
        sala.ceiling_read(rd, out_f, 0)
        evs[-1].record()
        torch.cuda.synchronize()
        for n, name in enumerate(names):
            per[name].append(evs[n].elapsed_time(evs[n + 1]) * 1000.0)
        per.setdefault("empty", []).append(evs[-2].elapsed_time(evs[-1]) * 1000.0)
    med = {k: sorted(v)[len(v) // 2] for k, v in per.items()}
    calls = {"linear_decode": med["linear_decode"], "sparse_select": med["sparse_select"],
             "sparse_decode": med["sparse_decode"]}
    return {"method": "streaming microkernels moving each call's bytes in as many launches as the call makes, "
                      "timed like the calls (median of %d)" % reps,
            "empty_launch_us": round(med["empty"], 2),
            "calls_us": {k: round(v, 2) for k, v in calls.items()},
            "us_per_step": round(3 * calls["linear_decode"] + calls["sparse_select"] + calls["sparse_decode"], 2)}


def bench_decode(torch, sala, I, reps=20):
    """The 1M-context decode step (B=4): three linear decode steps, selection over
    16384 pooled blocks per (b, KV head), attention over the 67 selected blocks.
    Timed two ways, with a 1 GiB read between reps to leave L2 and the MALL
    holding unrelated clean lines:
      kernels  the sum of the calls' own durations: HIP events between the calls
               while two 1 GiB reads queued ahead keep the GPU busy, so every
               call is enqueued before the GPU reaches it and the events bracket
               the call's kernels (median per call over the reps)
      wall     one replay of the step captured in a HIP graph (median)."""
    lin, sp = I.workload5_decode("cuda")
    for x in lin:
        x["decay"] = x["decay"].cuda()
        x["o"] = torch.empty_like(x["q"])
    states0 = [x["state"].clone() for x in lin]
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
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.zeros((), dtype=torch.float32, device="cuda")

    calls = [(f"linear_decode[{n}]", (lambda x=x: sala.linear_decode(x["q"], x["k"], x["v"], x["state"], x["decay"],
                                                                     out=x["o"]))) for n, x in enumerate(lin)]
    calls += [("sparse_select", lambda: sala.sparse_select(q4, None, k_pooled=kp, L=L, idx_out=idx, workspace=ws_sel)),
              ("sparse_decode", lambda: sala.sparse_decode(q, sp["k_cache"], sp["v_cache"], idx, out=o,
                                                           workspace=ws_att))]

    def step():
        for _, fn in calls:
            fn()

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    o_eager = o.clone()
    # per-call durations with the GPU kept ahead of the host
    per = {name: [] for name, _ in calls}
    for _ in range(reps):
        sink.add_(flush.sum())
        sink.add_(flush.sum())
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
        evs[0].record()
        for n, (_, fn) in enumerate(calls):
            fn()
            evs[n + 1].record()
        torch.cuda.synchronize()
        for n, (name, _) in enumerate(calls):
            per[name].append(evs[n].elapsed_time(evs[n + 1]) * 1000.0)
    calls_us = {name: sorted(t)[len(t) // 2] for name, t in per.items()}
    us_kernels = sum(calls_us.values())
    floors = decode_floors(torch, sala, flush, sink, reps)
    # the step is five short calls; launching them from Python one by one would
    # time the host, so the wall time comes from one replay of a captured graph
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
    us = events_ms(torch, graph.replay, reps, before=lambda: sink.add_(flush.sum())) * 1000.0
    nbytes = 3 * (2 * 4 * 32 * 128 * 128 * 4) + 4 * 2 * 16384 * 128 * 4 + 4 * 2 * 67 * 64 * 128 * 2 * 2
    frac = lambda t_us: round(nbytes / (t_us * 1e-6) / (PEAK_HBM_GBS * 1e9), 4)  # noqa: E731
    out = {"workload": "decode step at L=1048576, B=4: 3 linear decode (H=32, d=128 fp32 state) + select over "
                       "16384 pooled blocks + attention over 64+1+2 blocks (Hq=32, Hkv=2)",
           "algorithmic_bytes": nbytes,
           "us_per_step_kernels": round(us_kernels, 2), "hbm_frac_kernels": frac(us_kernels),
           "us_per_step_median": round(us, 2), "hbm_frac": frac(us), "target_frac": DECODE_TARGET_FRAC,
           "calls_us": {k: round(v, 2) for k, v in calls_us.items()},
           "roofline": {"bound": "hbm", "achieved": round(nbytes / (us_kernels * 1e-6) / 1e9, 1),
                        "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": frac(us_kernels),
                        "on": "summed call durations"},
           "timing": "kernels: median per call of HIP events between the calls with the GPU kept ahead of the host, "
                     "summed; wall: HIP events around one replay of the captured step, median of %d reps; 1 GiB read "
                     "between reps" % reps, "graph_replay_matches_eager": replay_ok}
    floors["hbm_frac"] = frac(floors["us_per_step"])
    out["floors"] = floors

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
    us2 = events_ms(torch, graph2.replay, reps, before=lambda: sink.add_(flush.sum())) * 1000.0
    out["generation_step"] = {
        "workload": "the same step inside a generation loop: fused linear decode (QK RMS norm, RoPE at L-1, gate) "
                    "x3 + sala_sparse_decode_step (append k, v at L-1, pooled-key update, select, attend)",
        "us_per_step_median": round(us2, 2), "matches_plain_step": gen_ok}

    # the oracle on the same step: host copies first (inputs, the pooled cache, the
    # cached rows of the selected blocks), then the oracle's decode functions
    import numpy as np
    from oracle import linear as OL
    from oracle import sparse as OS
    h = lambda t: t.double().cpu().numpy()  # noqa: E731
    lin_h = [(h(x["q"]), h(x["k"]), h(x["v"]), h(s0), h(x["decay"])) for x, s0 in zip(lin, states0)]
    qh, kbar = h(q), h(kp)
    # rows of every block either side may select (the GPU's picks and, untimed, the oracle's)
    both = np.concatenate([idx[:, :, 0].cpu().numpy(), OS.sparse_select_decode(qh, kbar, L, 64, 64, 1, 2)[0]], -1)
    rows = {(b, kv): np.concatenate([np.arange(j * 64, min((j + 1) * 64, L)) for j in set(both[b, kv].tolist())
                                     if j >= 0]) for b in range(4) for kv in range(2)}
    kr, vr = HostRows(sp["k_cache"], rows), HostRows(sp["v_cache"], rows)
    t0 = time.perf_counter()
    for qq, kk, vv, ss, dec in lin_h:
        OL.linear_decode_batched(qq, kk, vv, ss, dec)
    ridx, _ = OS.sparse_select_decode(qh, kbar, L, 64, 64, 1, 2)
    OS.sparse_attention_decode(qh, kr, vr, ridx, L, 64)
    t_or = time.perf_counter() - t0
    out["tokens_per_s"] = round(4 / (us * 1e-6), 1)
    out["cpu_oracle"] = dict(oracle_entry(t_or, 4), sample="the whole step (3 x linear_decode_batched, "
                                                          "sparse_select_decode over the pooled cache, "
                                                          "sparse_attention_decode); tokens = the B=4 decoded tokens")
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
    Hq, Hkv, d = sp["q"].shape[1], sp["k"].shape[1], sp["q"].shape[3]
    nqb = (N + 63) // 64
    out_bufs = {"linear": [torch.empty_like(x["q"]) for x in lin], "sparse": torch.empty_like(sp["q"]),
                "idx": torch.empty((1, Hkv, nqb, 67), dtype=torch.int32, device="cuda"),
                "k_pooled": torch.empty((1, Hkv, nqb, d), dtype=torch.float32, device="cuda")}
    ws = {"linear": [torch.empty(max(1, sala.workspace_bytes("linear_prefill", dtype=1, B=1, H=32, N=N, d=128,
                                                             chunk=128)), dtype=torch.uint8, device="cuda")
                     for _ in lin],
          "select": torch.zeros(sala.workspace_bytes("sparse_select", dtype=1, B=1, Hq=Hq, Hkv=Hkv, d=d, Nq=N, L=N,
                                                     block=64, topk=64, n_init=1, n_local=2), dtype=torch.uint8,
                                device="cuda")}
    idx, o_sp = out_bufs["idx"], out_bufs["sparse"]
    ev = []

    def step(record=False):
        events = None
        if record:
            events = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            ev.append(events)
        sala.layer_group_prefill(lin, sp, topk=64, n_init=1, n_local=2, chunk=128, workspaces=ws, out=out_bufs,
                                 sparse_events=events)

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
            sala.sparse_prefill(sp["q"], sp["k"], sp["v"], idx, out=o_sp)
            torch.cuda.synchronize()
            n_clk += 1
    sclk = sclock.mhz()
    ms = elapsed * 1000.0 / args.steps
    att_ms = sum(s.elapsed_time(e) for s, e in ev) / len(ev)
    flops = sparse_flops(idx, N, d, Hq // Hkv)
    group_flops = 3 * (32 * N * (2 * 128 * 128 + 4 * 128 * 128)) * 1.0 + flops  # algorithmic (causal) counts
    achieved = flops / (att_ms * 1e-3) / 1e12
    busy = measured_mfma_busy()
    sclk_note = None
    if sclk and busy is not None and achieved / (PEAK_BF16_TFLOPS * sclk / 2400.0) > busy + 0.1:
        # the rate needs a faster clock than the one read: the readings came
        # from between launches (as under a profiler that serialises them) or
        # the driver reported another clock
        sclk_note = ("a reading of %d MHz would put the kernel at %.2f MFMA efficiency, above the %.3f MFMA-busy "
                     "fraction the counters measure: not the kernel's clock" %
                     (sclk, achieved / (PEAK_BF16_TFLOPS * sclk / 2400.0), busy))
        sclk = None
    traffic = measured_traffic_bytes() if N == 262144 else None
    # unique bytes: Q read and O written once; K and V of the KV heads read once
    alg_bytes = 2 * (Hq * N * d * 2) + 2 * (Hkv * N * d * 2)
    group_frac = group_flops / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)
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
        "group": {"bound": "mfma", "achieved": round(group_flops / (ms * 1e-3) / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                  "unit": "TFLOP/s", "frac": round(group_frac, 4), "target_frac": GROUP_TARGET_FRAC,
                  "target_met": bool(group_frac >= GROUP_TARGET_FRAC), "algorithmic_tflop": round(group_flops / 1e12, 3),
                  "note": "the whole step's algorithmic flops over its wall time (the linear third is HBM-bound)"},
        "roofline": {"kernel": "sparse_attn_bf16 (the dominant kernel, not the whole step: see group)",
                     "bound": "mfma",
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
        x0 = dict(lin[0], o=out_bufs["linear"][0], ws=ws["linear"][0])
        out["neighbours"] = bench_neighbours(torch, sala, I, x0, N)
    if not args.no_backward:
        out["backward"] = bench_backward(torch, sala, I, lin[0], sp, idx)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(lin, sp, idx, args.cpu_sample_seconds)
    del lin, out_bufs, ws
    torch.cuda.empty_cache()
    if not args.no_configs:
        cfg = {"1_tiny_group_fp32": bench_workload1(torch, sala, I),
               "2_linear_prefill_32K": bench_workload2(torch, sala, I, args.cpu_sample_seconds)}
        cfg["3_sparse_prefill_128K"] = bench_workload3(torch, sala, I, args.cpu_sample_seconds)
        torch.cuda.empty_cache()
        if not args.no_decode:
            cfg["5_decode_1M"] = bench_decode(torch, sala, I)
        out["configs"] = cfg
    elif not args.no_decode:
        out["configs"] = {"5_decode_1M": bench_decode(torch, sala, I)}
    if not args.no_ceilings:
        out["ceilings"] = measure_ceilings(torch, sala)
        out["roofline"]["frac_of_measured_ceiling"] = round(achieved / out["ceilings"]["mfma_bf16_tflops"], 4)
    if cpu is not None:
        out["cpu_baseline"] = cpu
    if out["roofline"]["sclk_mhz"] is None and sclock.error:
        out["roofline"]["sclk_error"] = sclock.error
    if sclk_note:
        out["roofline"]["sclk_note"] = sclk_note
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
