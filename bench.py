"""Benchmark of the FP8 block-scaled GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload decode|prefill|contiguous|masked|small|prefill_ue8m0|contiguous_ue8m0|mqa|
                                prefill_nn|prefill_tn|prefill_tt|kgrouped|kgrouped_ue8m0]

A step is one pass of the hot path over one batch of synthetic input: for
every GEMM of the workload, quantise the fp32 activations (1x128 scales) and
run the FP8 block-scaled GEMM.  Weights are quantised once (128x128 scales)
before timing, as in inference.  Default workload: the decode-shaped dense
GEMMs, M in {64, 128} x (N, K) in {(2112, 7168), (24576, 1536), (7168, 16384)},
C = 0, bf16 D.

Timing: the W warm-up steps and the K timed steps are each captured as one
HIP graph of consecutive steps (so host launch cost does not stall the GPU);
the timed region is one replay of the K-step graph, bracketed by device
synchronisation.  Weight copies rotate so that every B
is re-read only after more than 512 MB of other traffic (the 256 MB
Infinity Cache cannot serve it).  Per-kernel durations for the roofline are
measured separately with HIP events around graph replays of one GEMM launch
repeated over rotating weight copies.

Workload mqa: one FP8 MQA logits call (the v3.2 indexer's scoring) of 4096
query tokens x 64 heads against 8192 keys with causal ranges, inputs already
E4M3 and resident; value -> TFLOP/s of 2 * H * 128 per computed logit.

Prints ONE JSON line.  `value` is whole-job throughput: decode -> GB/s of
algorithmic HBM traffic (activation read + codes/scales written by the
quantiser, A + B + scales + D read/written by the GEMM); prefill and grouped
-> TFLOP/s of 2*M_valid*N*K.  `roofline` is the dominant kernels' figure:
algorithmic units of one launch of each GEMM of the step over the sum of
their median launch durations.  The decode run also carries `secondary`: the
same figures for the prefill, contiguous and masked workloads, measured in
the same process (--no-secondary skips them).  Dense decode GEMMs get their
split-K scratch from workspaces this script allocates (zeroed once).
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from moe_grouped_gemm_scaled_amd import binding as dg  # noqa: E402
from moe_grouped_gemm_scaled_amd import profiling  # noqa: E402
from moe_grouped_gemm_scaled_amd import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, published
MALL_BYTES = 256 << 20
ROTATE_BYTES = 512 << 20

METRIC = "FP8 GEMM TFLOPS (prefill) and HBM GB/s (decode) as % of MI355X peak"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cdiv(a, b):
    return (a + b - 1) // b


def gemm_bytes(m_valid, N, K, g_active=1, with_c=False):
    """Algorithmic bytes of one GEMM: A + B + sfa + sfb + D (+ C), valid rows only."""
    nkb = K // 128
    b = m_valid * K + g_active * N * K + 4 * m_valid * nkb + 4 * g_active * cdiv(N, 128) * nkb + 2 * m_valid * N
    if with_c:
        b += 2 * m_valid * N
    return b


def quant_bytes(rows, K):
    """fp32 read + E4M3 written + one fp32 scale per 128 elements."""
    return rows * K * 4 + rows * K + 4 * rows * (K // 128)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

class Job:
    """One GEMM of a step: activation quantiser + GEMM, with rotating weight copies."""

    def __init__(self, name, launch, copies, flops, bytes_gemm, bytes_quant):
        self.name = name
        self.launch = launch          # launch(copy_index, with_quant) -> None
        self.copies = copies
        self.flops = flops
        self.bytes_gemm = bytes_gemm
        self.bytes_quant = bytes_quant


def n_copies(weight_bytes):
    return max(2, cdiv(ROTATE_BYTES, max(1, weight_bytes)) + 1)


def make_weights(G, N, K, seed, ue8m0=False):
    xb = torch.from_numpy(synth.normal_f32(seed, synth.STREAM_B, (G, N, K))).cuda()
    b, sfb = dg.quantize_e4m3_128x128(xb, ue8m0=ue8m0)
    del xb
    return b, sfb


def replicate(t, n):
    return [t] + [t.clone() for _ in range(n - 1)]


def dense_jobs(cfgs, ue8m0=False, layout="nt"):
    """layout "nt": activation quantiser + GEMM per shape.  Other layouts: the
    GEMM alone, on operands quantised and stored in that layout beforehand
    (A as [K, M] for tn/tt, B as [K, N] for nn/tn)."""
    jobs = []
    weights = {}
    for cfg in cfgs:
        M, N, K, seed = cfg["M"], cfg["N"], cfg["K"], cfg["seed"]
        key = (M, N, K)           # no sharing between jobs: every GEMM streams its own copies
        if key not in weights:
            b, sfb = make_weights(1, N, K, seed, ue8m0)
            b0 = b[0] if layout[1] == "t" else b[0].t().contiguous()
            nc = n_copies(N * K)
            weights[key] = (replicate(b0, nc), replicate(sfb[0], nc))
        bs, sfbs = weights[key]
        x = torch.from_numpy(synth.normal_f32(seed, synth.STREAM_A, (M, K))).cuda()
        a = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        sfa = torch.zeros((K // 128, dg.get_sf_aligned_size(M)), dtype=torch.float32, device="cuda")
        c = None
        if cfg["with_c"]:
            c = torch.from_numpy(synth.normal_bf16_bits(seed, synth.STREAM_C, (M, N)).view(np.int16)).cuda()
            c = c.view(torch.bfloat16)
        d = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        # split-K scratch owned here, zeroed once, shared by every launch of this
        # job (they run in stream order); None when the shape does not split K
        ws = dg.get_workspace(M, N, K)

        if layout == "nt":
            def launch(ci, with_quant, x=x, a=a, sfa=sfa, bs=bs, sfbs=sfbs, c=c, d=d, ws=ws):
                if with_quant:
                    dg.quantize_e4m3_1x128(x, q=a, sf=sfa, ue8m0=ue8m0)
                dg.fp8_gemm_nt(a, sfa, bs[ci % len(bs)], sfbs[ci % len(bs)], d, c=c, ue8m0=ue8m0, workspace=ws)
            qbytes = quant_bytes(M, K)
        else:
            dg.quantize_e4m3_1x128(x, q=a, sf=sfa)
            a_st = a if layout[0] == "n" else a.t().contiguous()
            torch.cuda.synchronize()

            def launch(ci, with_quant, a_st=a_st, sfa=sfa, bs=bs, sfbs=sfbs, c=c, d=d):
                dg.fp8_gemm(layout, a_st, sfa, bs[ci % len(bs)], sfbs[ci % len(bs)], d, c=c)
            qbytes = 0

        jobs.append(Job(cfg["name"], launch, len(bs), 2.0 * M * N * K,
                        gemm_bytes(M, N, K, with_c=cfg["with_c"]), qbytes))
    return jobs


def contiguous_jobs(ue8m0=False):
    cfg = synth.CONTIGUOUS
    counts = synth.contiguous_counts(cfg)
    m_idx = synth.contiguous_m_indices(counts)
    M_total, N, K, G = m_idx.size, cfg["N"], cfg["K"], cfg["G"]
    b, sfb = make_weights(G, N, K, cfg["seed"], ue8m0)
    nc = n_copies(G * N * K)
    bs, sfbs = replicate(b, nc), replicate(sfb, nc)
    x = torch.from_numpy(synth.normal_f32(cfg["seed"], synth.STREAM_A, (M_total, K))).cuda()
    a = torch.empty((M_total, K), dtype=torch.uint8, device="cuda")
    sfa = torch.zeros((K // 128, M_total), dtype=torch.float32, device="cuda")
    mi = torch.from_numpy(m_idx).cuda()
    d = torch.empty((M_total, N), dtype=torch.bfloat16, device="cuda")
    m_valid = int(counts.sum())

    def launch(ci, with_quant):
        if with_quant:
            dg.quantize_e4m3_1x128(x, q=a, sf=sfa, ue8m0=ue8m0)
        dg.m_grouped_fp8_gemm_nt_contiguous(a, sfa, bs[ci % nc], sfbs[ci % nc], d, mi, ue8m0=ue8m0)

    return [Job(cfg["name"], launch, nc, 2.0 * m_valid * N * K, gemm_bytes(m_valid, N, K, G),
                quant_bytes(M_total, K))], dict(counts=counts.tolist(), M_total=M_total, m_valid=m_valid)


def masked_jobs():
    cfg = synth.MASKED
    mm = synth.masked_counts(cfg)
    G, M_cap, N, K = cfg["G"], cfg["M_cap"], cfg["N"], cfg["K"]
    b, sfb = make_weights(G, N, K, cfg["seed"])
    g_active = int((mm > 0).sum())
    nc = n_copies(g_active * N * K)
    bs, sfbs = replicate(b, nc), replicate(sfb, nc)
    x = torch.from_numpy(synth.normal_f32(cfg["seed"], synth.STREAM_A, (G, M_cap, K))).cuda()
    a = torch.empty((G, M_cap, K), dtype=torch.uint8, device="cuda")
    sfa = torch.zeros((G, K // 128, dg.get_sf_aligned_size(M_cap)), dtype=torch.float32, device="cuda")
    mmt = torch.from_numpy(mm).cuda()
    d = torch.empty((G, M_cap, N), dtype=torch.bfloat16, device="cuda")
    m_valid = int(mm.sum())

    def launch(ci, with_quant):
        if with_quant:
            dg.quantize_e4m3_1x128(x, q=a, sf=sfa)
        dg.m_grouped_fp8_gemm_nt_masked(a, sfa, bs[ci % nc], sfbs[ci % nc], d, mmt, expected_m=M_cap // 2)

    # the activation quantiser runs over the whole padded buffer (counts live on the device)
    return [Job(cfg["name"], launch, nc, 2.0 * m_valid * N * K, gemm_bytes(m_valid, N, K, g_active),
                quant_bytes(G * M_cap, K))], dict(masked_m=mm.tolist(), m_valid=m_valid, g_active=g_active)


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------

def kgrouped_jobs(ue8m0=False):
    """One K-grouped TN contiguous GEMM (MoE weight gradient): operands
    quantised 1x128 along K by the library's quantiser and laid out [K, M],
    [K, N] beforehand; fp32 D, no C."""
    cfg = synth.KGROUPED
    M, N = cfg["M"], cfg["N"]
    ksn = synth.kgrouped_sizes(cfg)
    K = int(ksn.sum())
    G = ksn.size
    xa = torch.from_numpy(synth.normal_f32(cfg["seed"], synth.STREAM_A, (M, K))).cuda()
    qa, sa = dg.quantize_e4m3_1x128(xa, ld_sf=M, ue8m0=ue8m0)
    del xa
    xb = torch.from_numpy(synth.normal_f32(cfg["seed"], synth.STREAM_B, (N, K))).cuda()
    qb, sb = dg.quantize_e4m3_1x128(xb, ld_sf=N, ue8m0=ue8m0)
    del xb
    a, b = qa.t().contiguous(), qb.t().contiguous()
    sfa, sfb = sa.contiguous(), sb.contiguous()
    ks = torch.from_numpy(ksn).cuda()
    d = torch.empty((G, M, N), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    def launch(ci, with_quant):
        dg.k_grouped_fp8_gemm_tn_contiguous(a, sfa, b, sfb, ks, d, ue8m0=ue8m0)

    flops = 2.0 * M * N * K
    nbytes = K * M + K * N + 4 * (K // 128) * (M + N) + 4 * G + 4 * G * M * N
    meta = {"G": G, "M": M, "N": N, "K_total": K, "ks": ksn.tolist()}
    return [Job(cfg["name"], launch, 1, flops, nbytes, 0)], meta


def mqa_jobs():
    """One FP8 MQA logits call (the v3.2 indexer's scoring) over a causal
    prefill chunk; inputs are already E4M3 (as the indexer holds them)."""
    cfg = synth.MQA
    S, S_kv, H, D = cfg["S"], cfg["S_kv"], cfg["H"], cfg["D"]
    qn, kvn, scn, wn = synth.mqa_tensors(cfg["seed"], S, H, S_kv, D)
    ksn, ken = synth.causal_ranges(S, S_kv)
    q, kv, sc, w = (torch.from_numpy(x).cuda() for x in (qn, kvn, scn, wn))
    ks, ke = torch.from_numpy(ksn).cuda(), torch.from_numpy(ken).cuda()
    out = torch.empty((S, S_kv), dtype=torch.float32, device="cuda")

    def launch(ci, with_quant):
        dg.fp8_mqa_logits(q, kv, sc, w, ks, ke, True, logits=out)

    pairs = int(np.sum(np.maximum(np.minimum(ken, S_kv) - np.maximum(ksn, 0), 0)))
    flops = 2.0 * pairs * H * D
    nbytes = S * H * D + S_kv * D + 4 * S_kv + 4 * S * H + 8 * S + 4 * S * S_kv
    meta = {"S": S, "S_kv": S_kv, "H": H, "D": D, "pairs": pairs, "ranges": "causal, query i sees [0, S_kv-S+i+1)"}
    return [Job(cfg["name"], launch, 1, flops, nbytes, 0)], meta


_CAPTURE_STREAM = None


def capture(fn):
    """Capture fn() into a graph on one dedicated stream, after one eager call
    on that stream (first-call set-up such as kernel attributes happens
    outside the capture)."""
    global _CAPTURE_STREAM
    if _CAPTURE_STREAM is None:
        _CAPTURE_STREAM = torch.cuda.Stream()
    s = _CAPTURE_STREAM
    g = torch.cuda.CUDAGraph()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                         # warm: first-call allocations happen outside capture
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


def kernel_durations(jobs, reps=24, trials=9):
    """Duration of one GEMM launch per job: HIP events on the capture stream
    around graph replays of `reps` launches over rotating weight copies
    (quantiser excluded); the median over `trials` replays, and their spread."""
    out = []
    s = _CAPTURE_STREAM
    for j in jobs:
        def body(j=j):
            for r in range(reps):
                j.launch(r, False)
        g = capture(body)
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(trials):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(s):
                e0.record()
                g.replay()
                e1.record()
            e1.synchronize()
            times.append(e0.elapsed_time(e1) / reps)
        out.append((float(np.median(times)), float(min(times)), float(max(times))))
        del g
    return out


def measured_traffic(workload, jobs):
    """HBM bytes moved by one launch of each GEMM of the step, summed, from the
    committed counter summary profiles/hbm_traffic_<workload>.json (FETCH_SIZE
    and WRITE_SIZE runs scaled by a copy of known size).  None when there is no
    summary, when it misses a job, or when the kernel sources have changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    if data.get("source_hash") != profiling.kernel_source_hash():
        return None
    total = 0.0
    for j in jobs:
        t = data.get("jobs", {}).get(j.name)
        if not t:
            return None
        total += t["fetch_bytes"] + t["write_bytes"]
    return round(total)


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------

def _decode_oracle(budget_s):
    """The oracle (at its current thread count) on all rows and a leading
    fraction of the columns of the six decode GEMMs plus the full activation
    quantiser, sized to about budget_s seconds; returns the algorithmic GB/s of
    the whole step with the GEMM time scaled by the column fraction."""
    import oracle
    cfgs = synth.DECODE
    # calibrate the oracle's multiply-add rate on a small slice
    cfg = cfgs[0]
    xa = synth.normal_f32(cfg["seed"], synth.STREAM_A, (cfg["M"], cfg["K"]))
    xb = synth.normal_f32(cfg["seed"], synth.STREAM_B, (256, cfg["K"]))
    a, sfa = oracle.quantize_1x128(xa)
    b, sfb = oracle.quantize_128x128(xb)
    t0 = time.perf_counter()
    oracle.gemm_nt(a, sfa, b[:64], sfb[:1], None)
    rate = cfg["M"] * 64 * cfg["K"] / (time.perf_counter() - t0)
    full_macs = sum(c["M"] * c["N"] * c["K"] for c in cfgs)
    frac = min(1.0, budget_s * rate / full_macs)
    total_bytes, t_full, macs_sample = 0, 0.0, 0
    for cfg in cfgs:
        M, N, K = cfg["M"], cfg["N"], cfg["K"]
        ns = max(128, int(N * frac) // 128 * 128)
        xa = synth.normal_f32(cfg["seed"], synth.STREAM_A, (M, K))
        xb = synth.normal_f32(cfg["seed"], synth.STREAM_B, (ns, K))
        b, sfb = oracle.quantize_128x128(xb)                  # weights: offline, not timed
        t0 = time.perf_counter()
        a, sfa = oracle.quantize_1x128(xa)
        tq = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.gemm_nt(a, sfa, b, sfb, None)
        tg = time.perf_counter() - t0
        t_full += tq + tg * (N / ns)
        macs_sample += M * ns * K
        total_bytes += gemm_bytes(M, N, K) + quant_bytes(M, K)
    sample = (f"all rows of each of the 6 decode GEMMs x the first {frac:.4f} of their columns "
              f"({macs_sample / 1e9:.2f} G multiply-adds of {full_macs / 1e9:.2f} G), plus the full "
              f"activation quantiser; time scaled to the whole step by the column fraction")
    return total_bytes / t_full / 1e9, t_full, sample


def _small_oracle(reps=5):
    """The oracle on the whole dense 128x256x512 problem (quantiser + GEMM),
    median of `reps` runs: (GB/s of its algorithmic bytes, seconds)."""
    import oracle
    cfg = synth.DENSE_SMALL
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    xa = synth.normal_f32(cfg["seed"], synth.STREAM_A, (M, K))
    xb = synth.normal_f32(cfg["seed"], synth.STREAM_B, (N, K))
    b, sfb = oracle.quantize_128x128(xb)
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        a, sfa = oracle.quantize_1x128(xa)
        oracle.gemm_nt(a, sfa, b, sfb, None)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return (gemm_bytes(M, N, K) + quant_bytes(M, K)) / t / 1e9, t


def cpu_baseline(workload, jobs_meta, budget_s=15.0):
    import oracle
    cores = oracle.num_threads()
    if workload == "mqa":
        return cpu_baseline_mqa(jobs_meta, budget_s)
    if workload != "decode":
        return None
    gbs, t_full, sample = _decode_oracle(budget_s)
    small_gbs, small_t = _small_oracle()
    # the same on one thread (the survey's single-core figures for the small
    # dense problem and the decode step), on a smaller sample
    oracle.set_num_threads(1)
    try:
        gbs1, t_full1, sample1 = _decode_oracle(budget_s / 3)
        small_gbs1, small_t1 = _small_oracle()
    finally:
        oracle.set_num_threads(cores)
    return {"value": gbs, "unit": "GB/s", "cores": cores, "kind": "oracle", "sample": sample,
            "seconds_full_step_extrapolated": t_full,
            "single_thread": {"value": gbs1, "unit": "GB/s", "cores": 1, "sample": sample1,
                              "seconds_full_step_extrapolated": t_full1},
            "small_dense_128x256x512": {"all_cores": {"value": small_gbs, "unit": "GB/s", "seconds": small_t,
                                                      "cores": cores},
                                        "single_thread": {"value": small_gbs1, "unit": "GB/s",
                                                          "seconds": small_t1, "cores": 1},
                                        "sample": "the whole problem: quantiser + GEMM, median of 5 runs"}}


def cpu_baseline_mqa(meta, budget_s):
    import oracle
    cfg = synth.MQA
    S, S_kv, H, D = cfg["S"], cfg["S_kv"], cfg["H"], cfg["D"]
    q, kv, sc, w = synth.mqa_tensors(cfg["seed"], S, H, S_kv, D)
    ks, ke = synth.causal_ranges(S, S_kv)
    lens = np.maximum(np.minimum(ke, S_kv) - np.maximum(ks, 0), 0)
    probe = np.arange(S - oracle.num_threads(), S, dtype=np.int32)     # one row per thread
    t0 = time.perf_counter()
    oracle.mqa_logits_rows(q, kv, sc, w, ks, ke, True, probe)
    rate = float(lens[probe].sum()) / (time.perf_counter() - t0)       # computed logits per second
    n = int(min(S, max(8, budget_s * rate / float(lens.mean()))))
    rows = np.unique(np.linspace(0, S - 1, n).round().astype(np.int32))
    t0 = time.perf_counter()
    oracle.mqa_logits_rows(q, kv, sc, w, ks, ke, True, rows)
    t = time.perf_counter() - t0
    t_full = t * float(lens.sum()) / float(lens[rows].sum())
    flops = 2.0 * float(lens.sum()) * H * D
    return {"value": flops / t_full / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": (f"{rows.size} of {S} query rows, evenly spaced ({int(lens[rows].sum())} of "
                       f"{int(lens.sum())} computed logits); time scaled to the whole call by that fraction"),
            "seconds_full_step_extrapolated": t_full}


# ---------------------------------------------------------------------------

WORKLOAD_DESC = {
    "decode": "decode-shaped dense FP8 NT GEMM, M in {64,128} x (N,K) in {(2112,7168),(24576,1536),(7168,16384)}, "
              "1x128/128x128 block scales, C=0, bf16 D",
    "prefill": "prefill-shaped dense FP8 NT GEMM, M=4096 x (N,K) in {(4096,7168),(7168,2048),(24576,1536)}, "
               "C bf16, bf16 D",
    "contiguous": "M-grouped contiguous FP8 GEMM, 8 experts, counts U[1,4096] padded to 128, N=4096, K=7168",
    "masked": "M-grouped masked FP8 GEMM, 16 experts x 256 rows, masked_m U[0,256], N=7168, K=2048",
    "small": "dense FP8 NT GEMM M=128, N=256, K=512",
    "prefill_ue8m0": "prefill-shaped dense FP8 NT GEMM, M=4096 x (N,K) in {(4096,7168),(7168,2048),(24576,1536)}, "
                     "C bf16, bf16 D, power-of-two (UE8M0) block scales",
    "contiguous_ue8m0": "M-grouped contiguous FP8 GEMM, 8 experts, counts U[1,4096] padded to 128, N=4096, K=7168, "
                        "power-of-two (UE8M0) block scales",
    "prefill_nn": "prefill-shaped dense FP8 GEMM in the NN layout (A [M,K], B stored [K,N]), M=4096 x (N,K) in "
                  "{(4096,7168),(7168,2048),(24576,1536)}, C bf16, bf16 D",
    "prefill_tn": "prefill-shaped dense FP8 GEMM in the TN layout (A stored [K,M], B stored [K,N]), M=4096 x (N,K) in "
                  "{(4096,7168),(7168,2048),(24576,1536)}, C bf16, bf16 D",
    "prefill_tt": "prefill-shaped dense FP8 GEMM in the TT layout (A stored [K,M], B [N,K]), M=4096 x (N,K) in "
                  "{(4096,7168),(7168,2048),(24576,1536)}, C bf16, bf16 D",
    "kgrouped": "K-grouped TN contiguous FP8 GEMM (MoE weight gradient), 8 groups of the contiguous workload's "
                "token counts padded to 128 (K_total 17408), M=7168, N=2048, 1x128 scales on both operands, "
                "fp32 D, no C",
    "kgrouped_ue8m0": "K-grouped TN contiguous FP8 GEMM (MoE weight gradient), 8 groups of the contiguous "
                      "workload's token counts padded to 128 (K_total 17408), M=7168, N=2048, power-of-two "
                      "(UE8M0) 1x128 scales on both operands, fp32 D, no C",
    "mqa": "FP8 MQA logits (non-paged, clean_logits): 4096 query tokens x 64 heads x 128 against 8192 keys, "
           "causal ranges, fp32 logits [4096, 8192]",
}

WORKLOADS = list(WORKLOAD_DESC)


def build_jobs(workload):
    """(jobs, bound, meta) of a workload."""
    meta = {}
    if workload == "decode":
        return dense_jobs(synth.DECODE), "hbm", meta
    if workload == "prefill":
        return dense_jobs(synth.PREFILL), "mfma", meta
    if workload == "prefill_ue8m0":
        return dense_jobs(synth.PREFILL, ue8m0=True), "mfma", meta
    if workload in ("prefill_nn", "prefill_tn", "prefill_tt"):
        return dense_jobs(synth.PREFILL, layout=workload[-2:]), "mfma", meta
    if workload == "small":
        return dense_jobs([synth.DENSE_SMALL]), "hbm", meta
    if workload in ("contiguous", "contiguous_ue8m0"):
        jobs, meta = contiguous_jobs(ue8m0=workload.endswith("_ue8m0"))
        return jobs, "mfma", meta
    if workload in ("kgrouped", "kgrouped_ue8m0"):
        jobs, meta = kgrouped_jobs(ue8m0=workload.endswith("_ue8m0"))
        return jobs, "mfma", meta
    if workload == "mqa":
        jobs, meta = mqa_jobs()
        return jobs, "mfma", meta
    jobs, meta = masked_jobs()
    return jobs, "hbm", meta


def step_kind(workload):
    if workload == "mqa":
        return "one fp8_mqa_logits call, inputs resident"
    if workload[-3:] in ("_nn", "_tn", "_tt") or workload.startswith("kgrouped"):
        return "one GEMM per shape, operands quantised and laid out beforehand"
    return "activation quantiser + GEMM per shape; weights pre-quantised"


def run_workload(workload, steps, warmup):
    """Times one workload: returns its measured figures (value, roofline,
    per-GEMM durations) and its job metadata."""
    jobs, bound, meta = build_jobs(workload)
    log(f"workload {workload}: {[j.name for j in jobs]}, copies {[j.copies for j in jobs]}")

    # two graphs: the W warm-up steps and the K timed steps, each captured as
    # one graph of consecutive steps (step s uses weight copy s of every job),
    # so that a replay boundary never sits between two timed steps
    def steps_fn(first, count):
        def fn():
            for s in range(first, first + count):
                for j in jobs:
                    j.launch(s, True)
        return fn

    warm_graph = capture(steps_fn(0, warmup)) if warmup > 0 else None
    timed_graph = capture(steps_fn(warmup, steps))
    configs = []
    with torch.cuda.stream(_CAPTURE_STREAM):       # the stream the graphs were captured on
        for j in jobs:
            j.launch(0, False)
            configs.append(dg.last_config())
    torch.cuda.synchronize()

    with torch.cuda.stream(_CAPTURE_STREAM):
        if warm_graph is not None:
            warm_graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        timed_graph.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / steps
    del warm_graph, timed_graph

    kd = kernel_durations(jobs)
    kms = [k[0] for k in kd]                       # medians
    step_bytes = sum(j.bytes_gemm + j.bytes_quant for j in jobs)
    step_flops = sum(j.flops for j in jobs)
    gemm_bytes_total = sum(j.bytes_gemm for j in jobs)
    gemm_time_s = sum(kms) / 1e3
    per_job = [{"name": j.name, "gemm_us": round(k[0] * 1e3, 3),
                "gemm_us_min_max": [round(k[1] * 1e3, 3), round(k[2] * 1e3, 3)],
                "gemm_GBps": round(j.bytes_gemm / (k[0] / 1e3) / 1e9, 1),
                "gemm_TFLOPs": round(j.flops / (k[0] / 1e3) / 1e12, 1), "config": cfg}
               for j, k, cfg in zip(jobs, kd, configs)]

    traffic = measured_traffic(workload, jobs)
    if bound == "hbm":
        value = step_bytes / (ms_step / 1e3) / 1e9
        unit = "GB/s"
        achieved = gemm_bytes_total / gemm_time_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}
    else:
        value = step_flops / (ms_step / 1e3) / 1e12
        unit = "TFLOP/s"
        achieved = step_flops / gemm_time_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP8_PEAK_TFLOPS, 4), "traffic": traffic}
    # bytes the traffic figure compares with: the algorithmic bytes of the same launches
    roof["algorithmic_bytes"] = round(gemm_bytes_total)
    res = {"workload": workload, "value": round(value, 2), "unit": unit, "steps": steps, "warmup": warmup,
           "ms_per_step": round(ms_step, 5), "roofline": roof,
           "frac_of_peak_step": round(value / (HBM_PEAK_GBS if bound == "hbm" else FP8_PEAK_TFLOPS), 4),
           "per_gemm": per_job}
    del jobs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, meta


def data_desc(workload):
    if workload == "mqa":
        return ("synthetic: seeded uniformly random e4m3 codes for q and kv, kv_scale 2^-9 (1+U[0,1)), "
                "weights N(0,1)/8")
    return ("synthetic: seeded N(0,1) fp32, quantised to e4m3 with 1x128 / 128x128 fp32 scales"
            + (" rounded up to powers of two (UE8M0)" if workload.endswith("_ue8m0") else ""))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=WORKLOADS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="decode only: skip the prefill, contiguous and masked figures in `secondary`")
    ap.add_argument("--secondary-steps", type=int, default=20)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 20 device-to-device copies of MIB MiB each (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: there is no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(20):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_copy": n, "copies": 20}), flush=True)
        return
    dg.lib()

    res, meta = run_workload(args.workload, args.steps, args.warmup)

    # the other half of the metric, from the same process: the compute-bound
    # prefill and contiguous workloads and the HBM-bound masked one
    secondary = []
    if args.workload == "decode" and not args.no_secondary:
        for w in ("prefill", "contiguous", "masked"):
            r, m = run_workload(w, args.secondary_steps, min(args.warmup, 3))
            r["config"] = {"workload": WORKLOAD_DESC[w], "step": step_kind(w), "graph_replay": True,
                           **({"layout": m} if m else {})}
            r["data"] = data_desc(w)
            secondary.append(r)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample")
        cpu = cpu_baseline(args.workload, meta)

    out = {
        "metric": METRIC,
        "value": res["value"],
        "unit": res["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": data_desc(args.workload),
        "config": {"workload": WORKLOAD_DESC[args.workload], "step": step_kind(args.workload),
                   "graph_replay": True, **({"layout": meta} if meta else {})},
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
        "frac_of_peak_step": res["frac_of_peak_step"],
        "per_gemm": res["per_gemm"],
        "secondary": secondary,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
