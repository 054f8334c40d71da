"""Benchmark of the compressed-KV decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama8b|ragged|long] [--fmt F3|F4|F25]

A step is one pass of the whole path over one batch, for every layer: append
the new token of each sequence (FIFO eviction of the oldest hot entry, whose
K and V are quantised into cold codes), decode attention of every query head
over hot fp16 and cold codes, then promotion bookkeeping.  Inputs are
synthetic and drawn on the device with seeded torch generators (the same
distributions as the seeded workload generators); nothing is read from disk.

Prints one JSON line.  value = decode context tokens per second over the whole
step (sequence x layer x live context token, per wall second of the timed
steps, append and promotion included).  The roofline object covers the
split-context attention kernel (the dominant one), timed with HIP events on
the library's stream inside the timed region.  cpu_baseline times the CPU
oracle on a bounded sample of the same workload.

    python bench.py --copy-probe

times a plain device copy of a known size instead (achievable HBM bandwidth,
and the reference kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE).
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0     # MI355X HBM3E peak, GB/s
PEAK_F16_TFLOPS = 2500.0  # MI355X dense fp16 MFMA peak, TFLOP/s
COPY_PROBE_BYTES = 2 << 30
GATE_THRESHOLDS = (None, 4.0, 3.5, 3.0, 2.5, 0.0)  # hot-first gate sweep (None: the plain step)


def record_bytes(d, fmt):
    rb, tb, m = fmt
    return (d // 2) * (rb + tb) // 8 + m // 8 + 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b", choices=["llama8b", "ragged", "long", "tiny", "tinyllama"])
    ap.add_argument("--fmt", default="F3", choices=["F3", "F4", "F25"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--copy-probe", action="store_true", help="time a plain device copy and exit")
    ap.add_argument("--scrub-mb", type=int, default=-1,
                    help="MB written and read before each timed step to evict the MALL (-1: 1024 for the long, "
                         "tiny and tinyllama workloads, whose steps fit in the 256 MB MALL, else 0)")
    ap.add_argument("--no-quality", action="store_true", help="skip the quality block")
    ap.add_argument("--calls", default="step", choices=["step", "separate"],
                    help="step: one tq_decode_step per layer (append, then attention, the query preparation inside "
                         "the append's launch); separate: tq_quantize_append, then tq_decode_attention")
    ap.add_argument("--promote", default="deferred", choices=["deferred", "immediate"],
                    help="deferred: tq_promote_deferred (each layer's promotion runs inside the next layer's append "
                         "launch; the step ends with tq_flush, inside the timed region); immediate: tq_promote")
    return ap.parse_args()


def device_kv(torch, gen, n_tok, hkv, d, scales):
    x = torch.randn((n_tok, hkv, d), generator=gen, device="cuda", dtype=torch.float32)
    return (x * scales).to(torch.float16).contiguous()


def copy_probe(torch, reps=5):
    """Achievable HBM bandwidth of a plain copy: (read + write bytes) / time."""
    n = COPY_PROBE_BYTES // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) / 1e3 / reps
    return dict(bytes_per_copy=2 * COPY_PROBE_BYTES, us_per_copy=s * 1e6, gbs=2 * COPY_PROBE_BYTES / s / 1e9)


CPU_SAMPLE_TOKENS = 8192   # context of each oracle worker's (sequence, layer) sample


def _oracle_worker(args):
    """One oracle (sequence, layer) sample: prefill the first CPU_SAMPLE_TOKENS
    tokens with the oracle's own codec (timed apart: the quantise rate), then
    time decode-attention steps for about budget_s seconds.  BLAS on one
    thread."""
    name, fmt_t, seq, budget_s = args
    from threadpoolctl import threadpool_limits

    from compressed_kv_decode_amd import workloads as wl
    from oracle import params
    from oracle.codec import Format
    from oracle.paging import SeqLayerCache

    w = wl.make(name, fmt=fmt_t) if name == "llama8b" else wl.make(name)
    seq = seq % w.n_seq
    with threadpool_limits(limits=1):
        pi, s = params.rotation(w.head_dim, w.seed), params.sketch(64, w.head_dim, w.seed)
        oc = SeqLayerCache(w.n_kv_heads, w.head_dim, w.window, Format(*(fmt_t or w.formats[0])), pi, s, tau=2.0)
        n = min(CPU_SAMPLE_TOKENS, w.prefill[seq])
        k, v = wl.prefill_kv(w, 0, seq, 0, n)
        tq = time.perf_counter()
        oc.append(k, v)
        tq = time.perf_counter() - tq
        ctx = len(oc.hot) + len(oc.live)
        t0 = time.perf_counter()
        steps = 0
        while True:
            oc.attend(wl.query(w, 0, seq, steps))
            steps += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    return ctx, steps, el, len(oc.live), tq


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(name, fmt_t, budget_s):
    """The CPU oracle, as it stands, on a bounded sample of the workload: one
    process on one core, then a fork pool of N processes (N = the cores this
    process may run on, at most 16), each on its own (sequence, layer 0)
    sample.  Runs before the GPU is initialised, so no child inherits a GPU
    context."""
    import multiprocessing as mp

    ctx1, n1, el1, nq1, tq1 = _oracle_worker((name, fmt_t, 0, budget_s))
    n_cores = max(1, min(16, len(os.sched_getaffinity(0))))
    with mp.get_context("fork").Pool(n_cores) as pool:
        res = pool.map(_oracle_worker, [(name, fmt_t, i, budget_s) for i in range(n_cores)])
    agg = sum(c * n / e for c, n, e, _, _ in res)
    steps_n = sum(r[1] for r in res)
    return dict(value=agg, unit="ctx tokens/s", cores=n_cores, kind="oracle", cpu_model=cpu_model(),
                value_1core=ctx1 * n1 / el1,
                quantize_tokens_per_s=sum(nq / tq for _, _, _, nq, tq in res), quantize_tokens_per_s_1core=nq1 / tq1,
                quantize_sample=f"the {nq1} tokens that go cold in each process's prefill, all kv heads, K and V "
                                f"(1 core: {tq1:.1f} s)",
                sample=f"{name}: per process one (sequence, layer 0) with a {ctx1}-token context (its first "
                       f"{CPU_SAMPLE_TOKENS} tokens: {ctx1 - 512} cold codes + 512 hot), prefill untimed, then "
                       f"about {budget_s:.0f} s of decode-attention steps of all query heads; 1 core: {n1} steps in "
                       f"{el1:.1f} s; {n_cores} processes: {steps_n} steps in total; numpy fp64, BLAS on 1 thread "
                       f"per process")


def read_probe(torch, tqkv, reps=5):
    """Achievable read-only HBM bandwidth: the library's streaming probe over
    a 4 GiB buffer (far beyond the 256 MB MALL)."""
    nbytes = 4 << 30
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(3)
    blocks = 8 * torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(blocks, dtype=torch.int32, device="cuda")
    tqkv.probe_read_bandwidth(buf, sink, blocks)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        tqkv.probe_read_bandwidth(buf, sink, blocks)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / reps
    del buf
    return dict(bytes=nbytes, us=t * 1e6, gbs=nbytes / t / 1e9, blocks=blocks)


def exact_attention_error(torch, q, k_all, v_all, out, g):
    """Error of the compressed-cache output against exact attention over the
    original fp16 keys and values (fp32 arithmetic)."""
    d = q.shape[-1]
    kk = k_all.float().permute(1, 0, 2).contiguous()           # [hkv, N, d]
    vv = v_all.float().permute(1, 0, 2).contiguous()
    qq = q.float().view(kk.shape[0], g, d)                      # [hkv, g, d]
    lg = torch.matmul(qq, kk.transpose(1, 2).contiguous()) / math.sqrt(d)
    ex = torch.matmul(torch.softmax(lg, dim=-1), vv).reshape(-1, d)
    diff = (out.float() - ex)
    return dict(max_abs=float(diff.abs().max()), rel_l2=float(diff.norm() / ex.norm()),
                tokens=int(k_all.shape[0]), heads=int(q.shape[0]))


def quality_block(torch, tqkv, wl):
    """Error of the compressed path against exact attention over the original
    fp16 keys and values (reported, not gated), with the value QJL term on
    and off, on two seeded numpy workloads: one llama8b (sequence 0, layer 0,
    F3, 32768 tokens) and the long-context needle (131072 tokens, F2.5), for
    which the needle's share of the attention and whether it is every head's
    argmax are reported as well, also under the hot-first gate."""
    import numpy as np

    def run(w, fmt, steps, v_qjl, gates=(None,), rotation_kind=0):
        k, v = wl.prefill_kv(w, 0, 0)
        c = tqkv.Cache(n_seq_max=1, n_layers=1, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                       head_dim=w.head_dim, hot_window=w.window, max_context=w.prefill[0], formats=[fmt],
                       seed=w.seed, v_qjl=v_qjl, rotation_kind=rotation_kind)
        kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        c.append(0, [0], [w.prefill[0]], kd, vd)
        e1.record()
        torch.cuda.synchronize()
        prefill_ms = e0.elapsed_time(e1)
        g = w.n_q_heads // w.n_kv_heads
        kk = kd.float().permute(1, 0, 2).contiguous()  # [hkv, N, d]
        vv = vd.float().permute(1, 0, 2).contiguous()
        rows = []
        for gate in gates:
            errs, cos, mass, hit = [], [], [], []
            for t in range(steps):
                qn = wl.query(w, 0, 0, t)
                q = torch.from_numpy(qn[None]).cuda()
                lg = torch.full((1, w.n_q_heads, c.logits_stride), float("nan"), device="cuda")
                out = c.attend(0, [0], q, logits=lg, gate=gate)[0]
                qq = q[0].float().view(w.n_kv_heads, g, w.head_dim)
                el = torch.matmul(qq, kk.transpose(1, 2).contiguous()) / float(np.sqrt(w.head_dim))
                ex = torch.matmul(torch.softmax(el, dim=-1), vv).reshape(-1, w.head_dim)
                d = out - ex
                errs.append((float(d.abs().max()), float(d.norm() / ex.norm())))
                cos.append(float(torch.nn.functional.cosine_similarity(out, ex, dim=1).mean()))
                if w.needle:
                    tok, _, _ = wl.needle(w, 0)
                    lgc = lg[0]
                    col = c.hot_capacity + tok
                    hit.append(float((lgc.argmax(dim=1) == col).float().mean()))
                    p = torch.softmax(lgc.nan_to_num(float("-inf")), dim=1)
                    mass.append(float(p[:, col].mean()))
            r = dict(max_abs=max(e[0] for e in errs), rel_l2=float(np.mean([e[1] for e in errs])),
                     cosine=float(np.mean(cos)), steps=steps)
            if w.needle:
                r.update(needle_argmax_hit_rate=float(np.mean(hit)), needle_mass_mean=float(np.mean(mass)))
            if gate is not None:
                r["gate_threshold"] = gate
            if rotation_kind:
                r["prefill_append_ms"] = prefill_ms
            rows.append(r)
        del c
        return rows[0] if len(rows) == 1 else rows

    w8 = wl.make("llama8b").with_(n_seq=1, n_layers=1, prefill=(32768,), formats=((2, 3, 32),))
    wn = wl.make("long")
    out = {}
    for v_qjl in (1, 0):
        out[f"llama8b_F3_vqjl{v_qjl}"] = run(w8, (2, 3, 32), 2, v_qjl)
        out[f"needle_F2.5_vqjl{v_qjl}"] = run(wn, (2, 2, 64), 4, v_qjl)
        torch.cuda.empty_cache()
    out["needle_F2.5_hot_first_gate"] = run(wn, (2, 2, 64), 4, 1, gates=(6.0, 4.0, 3.0, 2.0))
    # rotation ablation: the randomized Hadamard rotation against the Haar
    # one on the same inputs (both applied as dense matrices, so the append
    # time is the same kernel's)
    w4 = w8.with_(formats=((3, 4, 64),))
    abl = {}
    for name, ww, fmt in (("F3", w8, (2, 3, 32)), ("F4", w4, (3, 4, 64))):
        for kind, label in ((0, "haar"), (1, "hadamard")):
            r = run(ww, fmt, 2, 1, rotation_kind=kind)
            if not kind:
                r["prefill_append_ms"] = None
            abl[f"llama8b_{name}_{label}"] = r
        torch.cuda.empty_cache()
    abl["note"] = ("same llama8b sequence-0 inputs and queries per format; the Haar cache's append is timed "
                   "in the main prefill figures")
    out["rotation_ablation"] = abl
    out["note"] = ("compressed-cache output against fp32 exact attention over the original fp16 K/V (seeded numpy "
                   "inputs: llama8b sequence 0 layer 0, 32768 tokens, random queries; the 131072-token needle, "
                   "needle-aligned queries); needle figures from the debug logits, over all 32 query heads")
    return out


def tensor_cache_block(torch, tqkv, w, steps=8, layers=4):
    """The Tensor Cache cold tier on the same shapes (a few layers): evicted
    tokens are written into the d x d matrices (lambda 0.999, eta 1/128,
    g 0) instead of codes, attention is the hot window plus the gated read.
    Per-layer times of the prefill (matrix writes of every evicted token) and
    of a decode step (append + attention + promotion call)."""
    n_seq, hq, hkv, d = w.n_seq, w.n_q_heads, w.n_kv_heads, w.head_dim
    ctx = max(w.prefill)
    c = tqkv.Cache(n_seq_max=n_seq, n_layers=layers, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, hot_window=w.window,
                   max_context=ctx + steps + 4, formats=[w.formats[0]] * layers, seed=w.seed,
                   cold_tier=tqkv.COLD_TENSOR_CACHE, tc_lambda=0.999, tc_eta=1.0 / 128, tc_gate=0.0)
    seqs = list(range(n_seq))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pre = 0.0
    for l in range(layers):
        k = torch.randn((sum(w.prefill), hkv, d), generator=gen, device="cuda").half()
        v = torch.randn((sum(w.prefill), hkv, d), generator=gen, device="cuda").half()
        torch.cuda.synchronize()
        e0.record()
        c.append(l, seqs, list(w.prefill), k, v)
        e1.record()
        torch.cuda.synchronize()
        pre += e0.elapsed_time(e1)
        del k, v
    sk = [torch.randn((n_seq, hkv, d), generator=gen, device="cuda").half() for _ in range(steps + 2)]
    sq = [torch.randn((n_seq, hq, d), generator=gen, device="cuda").half() for _ in range(steps + 2)]
    out = torch.empty((n_seq, hq, d), dtype=torch.float32, device="cuda")

    def step(t):
        for l in range(layers):
            c.append(l, seqs, [1] * n_seq, sk[t], sk[t])
            c.attend(l, seqs, sq[t], out=out)
            c.promote(l, seqs)

    for t in range(2):
        step(t)
    torch.cuda.synchronize()
    e0.record()
    for t in range(steps):
        step(2 + t)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps / layers
    del c
    return dict(ms_per_layer_step=ms, prefill_ms_per_layer=pre / layers, layers_timed=layers, steps=steps,
                note="per (layer, decode step) over the workload's batch: append with the matrix write of the "
                     "evicted token, attention over the hot window plus sigmoid(g) q A, promotion call (a no-op "
                     "in this tier); compare ms_per_step / layers of the codes tier above")


def multi_query_block(torch, cache, w, n_new=4, reps=3):
    """Chunk / draft verification: the newest n_new hot entries of every
    (sequence, layer) treated as a chunk whose n_new queries attend to the
    whole cache (causal within the chunk), on the bench cache as the timed
    steps left it: one tq_multi_query_attention_batch call per layer over
    every sequence, and for comparison one tq_multi_query_attention call per
    (sequence, layer)."""
    n_seq, L, hq, d = w.n_seq, w.n_layers, w.n_q_heads, w.head_dim
    seqs = list(range(n_seq))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    q = torch.randn((n_new, hq, d), generator=gen, device="cuda").half()
    qb = q.unsqueeze(0).expand(n_seq, n_new, hq, d).contiguous()
    ws = torch.empty(cache.multi_query_batch_workspace_bytes(n_seq), dtype=torch.uint8, device="cuda")
    live = 0
    for l in range(L):
        for s in seqs:
            st = cache.stats(s, l)
            live += st["hot_len"] + st["live_cold"]
    cache.multi_query(0, 0, q)  # first launch of the kernels outside the events
    cache.multi_query_batch(0, seqs, qb, workspace=ws)
    torch.cuda.synchronize()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def batched():
        for l in range(L):
            cache.multi_query_batch(l, seqs, qb, workspace=ws)

    def per_sequence():
        for l in range(L):
            for s in seqs:
                cache.multi_query(l, s, q, workspace=ws)

    ms = timed(batched)
    ms1 = timed(per_sequence)
    return dict(n_new=n_new, ms_per_pass=ms, calls_per_pass=L,
                ctx_tokens_per_s=live / (ms / 1e3), query_ctx_pairs_per_s=live * n_new / (ms / 1e3),
                per_sequence_calls=dict(ms_per_pass=ms1, calls_per_pass=n_seq * L,
                                        ctx_tokens_per_s=live / (ms1 / 1e3)),
                note="one pass = every layer and sequence of the workload with n_new queries each, one batched "
                     "call per layer (per_sequence_calls: one call per sequence and layer); compare "
                     "attention.ms_per_step (one query per sequence) above")


def mips_block(torch, tqkv, n=1 << 20, d=128, n_q=64, k=10, reps=5):
    """Compressed-vector search (the codec's vector-search use): n synthetic
    Gaussian vectors stored as F3 codes in one cache stream, n_q queries,
    top-k by code-domain inner products.  Time per search (HIP events),
    bytes of key tiles read per search against the HBM peak, and recall@k
    against exact fp32 search over the original vectors."""
    fmt = (2, 3, 32)
    c = tqkv.Cache(n_seq_max=1, n_layers=1, n_q_heads=1, n_kv_heads=1, head_dim=d, hot_window=64, max_context=n,
                   formats=[fmt], seed=3)
    g = torch.Generator(device="cuda")
    g.manual_seed(21)
    x = torch.randn((n, 1, d), generator=g, device="cuda").half()
    c.append(0, [0], [n], x, torch.zeros_like(x))
    c.evict(0, [0], 0)
    q = torch.randn((n_q, d), generator=g, device="cuda").half()
    idx, sc = c.mips_search(0, 0, 0, q, k)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        idx, sc = c.mips_search(0, 0, 0, q, k)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / reps
    exact = torch.topk(q.float() @ x[:, 0].float().t(), k, dim=1).indices
    hits = sum(len(set(a.tolist()) & set(b.tolist())) for a, b in zip(idx.cpu(), exact.cpu()))
    groups = (n_q + 7) // 8
    key_bytes = n * (d // 2 * 5 // 8 + 32 // 8 + 4)  # F3 key records
    scanned = groups * key_bytes
    del c, x
    return dict(vectors=n, head_dim=d, format="F3", queries=n_q, k=k, us_per_search=t * 1e6,
                vector_scores_per_s=n * n_q / t, key_bytes_read_per_search=scanned,
                achieved_gbs=scanned / t / 1e9, frac_of_hbm_peak=scanned / t / 1e9 / PEAK_HBM_GBS,
                recall_at_k_vs_exact=hits / (n_q * k),
                note="queries in groups of 8 share one pass over the key tiles; recall on Gaussian data")


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {a.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    fmt_t = {"F3": (2, 3, 32), "F4": (3, 4, 64), "F25": (2, 2, 64)}[a.fmt]
    cpu = None
    if not a.no_cpu_baseline and not a.copy_probe:
        # before the GPU is touched: the pool forks
        cpu = cpu_baseline(a.workload, fmt_t if a.workload == "llama8b" else None, a.cpu_seconds)
    torch.cuda.set_device(0)
    if a.copy_probe:
        print(json.dumps({"copy_probe": copy_probe(torch)}))
        return

    from compressed_kv_decode_amd import tqkv
    from compressed_kv_decode_amd import workloads as wl

    fmt = {"F3": wl.F3, "F4": wl.F4, "F25": wl.F25}[a.fmt]
    if a.workload == "llama8b":
        w = wl.make("llama8b", fmt=fmt)
    else:
        w = wl.make(a.workload)
    total_steps = a.warmup + a.steps
    n_inputs = total_steps + 1  # one more step after the timed region: attention-only rate, error check
    w = w.with_(tau=0.15, sticky=3)  # promotion bookkeeping runs every step
    dev = torch.device("cuda")
    n_seq, L, hq, hkv, d = w.n_seq, w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim
    g = hq // hkv
    cache = tqkv.Cache(n_seq_max=n_seq, n_layers=L, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                       hot_window=w.window, max_context=max(w.prefill) + n_inputs, formats=list(w.formats),
                       seed=w.seed, promote_threshold=w.tau, sticky=w.sticky, v_qjl=w.v_qjl)
    seqs = list(range(n_seq))
    gen = torch.Generator(device="cuda")

    # A small untimed append per distinct format on a scratch cache first: the
    # first launch of each kernel loads its code object and the launcher
    # queries occupancy, host work that would otherwise sit inside the
    # events of the first prefill call.
    fmts_u = list(dict.fromkeys(w.formats))
    scratch = tqkv.Cache(n_seq_max=1, n_layers=len(fmts_u), n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                         hot_window=w.window, max_context=w.window + 64, formats=fmts_u, seed=w.seed,
                         promote_threshold=w.tau, sticky=w.sticky, v_qjl=w.v_qjl)
    sk = torch.randn((w.window + 64, hkv, d), device=dev).half()
    for l in range(len(fmts_u)):
        scratch.append(l, [0], [w.window + 64], sk, sk)
    torch.cuda.synchronize()
    del scratch, sk

    # prefill (untimed for the decode metric; gives the quantiser's rate)
    t_q = 0.0
    q_vectors = 0
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    keep_k = keep_v = None  # sequence 0, layer 0: for the exact-attention check
    for l in range(L):
        sk = torch.from_numpy(wl.channel_scales(w, l, "k")).float().to(dev)
        sv = torch.from_numpy(wl.channel_scales(w, l, "v")).float().to(dev)
        gen.manual_seed(1000 + l)
        tot = sum(w.prefill)
        k = device_kv(torch, gen, tot, hkv, d, sk)
        v = device_kv(torch, gen, tot, hkv, d, sv)
        if l == 0:
            keep_k, keep_v = k[:w.prefill[0]].clone(), v[:w.prefill[0]].clone()
        torch.cuda.synchronize()
        # the GPU spins while the host enqueues the events and the append, so
        # the interval between the events holds GPU work only
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(2_000_000)
        ev0.record()
        cache.append(l, seqs, list(w.prefill), k, v)
        ev1.record()
        torch.cuda.synchronize()
        t_q += ev0.elapsed_time(ev1) / 1e3
        q_vectors += 2 * hkv * sum(max(0, p - w.window) for p in w.prefill)
        del k, v
    # per-step tokens and queries, resident before timing
    gen.manual_seed(7)
    step_k = [[None] * L for _ in range(n_inputs)]
    step_v = [[None] * L for _ in range(n_inputs)]
    step_q = [[None] * L for _ in range(n_inputs)]
    for t in range(n_inputs):
        for l in range(L):
            step_k[t][l] = torch.randn((n_seq, hkv, d), generator=gen, device=dev).half()
            step_v[t][l] = torch.randn((n_seq, hkv, d), generator=gen, device=dev).half()
            step_q[t][l] = torch.randn((n_seq, hq, d), generator=gen, device=dev).half()
    out = torch.empty((n_seq, hq, d), dtype=torch.float32, device=dev)
    out0 = torch.empty((hq, d), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    att_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(L)]
    att_s = []

    deferred = a.promote == "deferred"
    ones = [1] * n_seq

    def step(t, probe):
        # the timed steps record nothing between the calls (an event record
        # costs the stream a few microseconds); the probe step after them does
        # (the probe step makes separate calls, to time the attention alone)
        for l in range(L):
            if a.calls == "step" and not probe:
                cache.step(l, seqs, ones, step_k[t][l], step_v[t][l], step_q[t][l], out=out)
            else:
                cache.append(l, seqs, ones, step_k[t][l], step_v[t][l])
                if probe:
                    att_ev[l][0].record()
                cache.attend(l, seqs, step_q[t][l], out=out)
                if probe:
                    att_ev[l][1].record()
                    if l == 0:
                        out0.copy_(out[0])
            cache.promote(l, seqs, deferred=deferred)
        cache.flush()  # the last layer's promotion, if deferred

    for t in range(a.warmup):
        step(t, False)
    torch.cuda.synchronize()
    cache.profile_read()  # clear
    cache.profile_enable(True)
    scrub_mb = a.scrub_mb if a.scrub_mb >= 0 else (1024 if a.workload in ("long", "tiny", "tinyllama") else 0)
    scrub = torch.empty(scrub_mb << 18, dtype=torch.float32, device=dev) if scrub_mb else None
    if scrub is not None:
        scrub.fill_(0.0)
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, t in enumerate(range(a.warmup, total_steps)):
        if scrub is not None:
            scrub.add_(1.0)  # reads and writes scrub_mb MB: the MALL holds none of the cache afterwards
        step_ev[i][0].record()
        step(t, False)
        step_ev[i][1].record()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    cache.profile_enable(False)
    dec_ms, dec_n = cache.profile_read()
    step_ms = [e0.elapsed_time(e1) for e0, e1 in step_ev]
    if scrub is not None:
        # the host clock would include the scrubs: the timed duration is the
        # sum of the steps' own intervals on the GPU clock
        el = sum(step_ms) / 1e3
        del scrub
    step(total_steps, True)  # probe step
    torch.cuda.synchronize()
    probe_att_ms = sum(att_ev[l][0].elapsed_time(att_ev[l][1]) for l in range(L))

    # live context per (seq, layer) during the timed steps
    st = [cache.stats(s_, l) for s_ in seqs for l in range(L)]
    assert all(x["status"] == 0 for x in st), "device error latched"
    live_now = sum(x["hot_len"] + x["live_cold"] for x in st)  # after the probe step
    ctx_per_step = live_now - n_seq * L - (n_seq * L) * (a.steps - 1) / 2.0  # mean over the timed steps
    ms_per_step = el * 1e3 / a.steps
    value = ctx_per_step / (ms_per_step / 1e3)

    # algorithmic bytes per decode launch (one layer, all sequences)
    per_layer_bytes = [0.0] * L
    hot_l, cold_l = [0] * L, [0] * L
    for l in range(L):
        B = record_bytes(d, w.formats[l])
        hot_l[l] = sum(cache.stats(s_, l)["hot_len"] for s_ in seqs)
        cold_l[l] = sum(cache.stats(s_, l)["live_cold"] for s_ in seqs)
        per_layer_bytes[l] = hot_l[l] * hkv * 4 * d + cold_l[l] * (hkv * 2 * B + 1 / 8) + n_seq * hq * d * (2 + 4)
    alg_bytes = float(np.mean(per_layer_bytes))
    avg_launch_s = dec_ms / 1e3 / max(dec_n, 1)
    achieved = alg_bytes / avg_launch_s / 1e9

    traffic = None
    tf = os.path.join(ROOT, "profiles", "decode_traffic.json")
    src = open(os.path.join(ROOT, "compressed_kv_decode_amd", "csrc", "tq_decode.hip"), "rb").read()
    if os.path.exists(tf):
        try:
            rec = json.load(open(tf))
            if rec.get("source_sha256") == hashlib.sha256(src).hexdigest() and rec.get("workload") == a.workload \
                    and rec.get("fmt") == a.fmt:
                traffic = rec.get("bytes_per_launch")
        except Exception:
            traffic = None

    # error against exact attention over the original fp16 keys and values
    k_all = torch.cat([keep_k[:, :, :]] + [step_k[t][0][0:1] for t in range(n_inputs)], 0)
    v_all = torch.cat([keep_v[:, :, :]] + [step_v[t][0][0:1] for t in range(n_inputs)], 0)
    exact = exact_attention_error(torch, step_q[total_steps][0][0], k_all, v_all, out0, g)
    probe = copy_probe(torch)
    rprobe = read_probe(torch, tqkv)

    # hot-first gate: speed / error trade-off of the attention alone, one pass
    # over every layer per threshold (same cache state and queries as the
    # probe step)
    gate_rows = []
    qg = [step_q[total_steps][l] for l in range(L)]
    ge0, ge1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for theta in GATE_THRESHOLDS:
        torch.cuda.synchronize()
        ge0.record()
        for l in range(L):
            cache.attend(l, seqs, qg[l], out=out, gate=theta)
            if l == 0:
                out0.copy_(out[0])
        ge1.record()
        torch.cuda.synchronize()
        ms = ge0.elapsed_time(ge1)
        err = exact_attention_error(torch, qg[0][0], k_all, v_all, out0, g)
        gate_rows.append(dict(threshold=theta if theta is not None else "off", attention_ms_per_step=ms,
                              ctx_tokens_per_s=live_now / (ms / 1e3), max_abs=err["max_abs"], rel_l2=err["rel_l2"]))

    m_max = max(f[2] for f in w.formats)
    rot_flops = q_vectors * 2.0 * (d * d + m_max * d)
    fnames = [n for f in w.formats for n, g in (("F3", wl.F3), ("F4", wl.F4), ("F25", wl.F25)) if g == f]
    fmt_label = fnames[0] if len(set(fnames)) == 1 else "/".join(sorted(set(fnames))) + " by layer"
    line = {
        "metric": "compressed-KV decode attn ctx tokens/s + HBM GB/s vs peak; quantize tok/s",
        "value": value,
        "unit": "ctx tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded on-device Gaussian K/V with the workload's outlier channels; no weights)",
        "config": {
            "workload": (f"{w.name}: {n_seq} seqs x {L} layers, {hq} q / {hkv} kv heads, head_dim {d}, "
                         f"context {max(w.prefill)}+ ({w.window} hot fp16 + rest cold {fmt_label}), decode step = "
                         f"append+evict+quantize, attention, promotion (tau {w.tau}, sticky {w.sticky})"),
            "n_seq": n_seq, "layers": L, "q_heads": hq, "kv_heads": hkv, "head_dim": d,
            "format": fmt_label, "hot_window": w.window, "promote": a.promote, "calls": a.calls,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic,
            "traffic_source": ("stored: profiles/decode_traffic.json, rocprofv3 FETCH_SIZE + WRITE_SIZE of this "
                               "workload and format, taken on the same k_decode source (sha256 match); not "
                               "measured in this run" if traffic is not None else None),
            "kernel": "k_decode (split-context attention over hot fp16 + cold codes)",
            "alg_bytes_per_launch": alg_bytes,
            "avg_launch_us": avg_launch_s * 1e6,
            "launches": dec_n,
            "achievable_copy_gbs": probe["gbs"],
            "achievable_read_gbs": rprobe["gbs"],
            "frac_of_read_probe": achieved / rprobe["gbs"],
        },
        "step_ms": {"median": float(np.median(step_ms)), "p10": float(np.percentile(step_ms, 10)),
                    "p90": float(np.percentile(step_ms, 90))},
        "attention": {
            "ctx_tokens_per_s": live_now / (probe_att_ms / 1e3),
            "ms_per_step": probe_att_ms,
            "note": "tq_decode_attention calls (query prep, split-context kernel, combine) of one step after the "
                    "timed region, bracketed by events",
        },
        "quantize": {
            "vectors_per_s": q_vectors / t_q,
            "tokens_per_s": q_vectors / (2 * hkv) / t_q,
            "rotation_sketch_tflops": rot_flops / t_q / 1e12,
            "mfma_frac_of_f16_peak": rot_flops / t_q / 1e12 / PEAK_F16_TFLOPS,
            "note": "prefill appends (all layers): rotation + pair codes + sketch + packing, HIP events "
                    "around each append call queued behind a GPU spin (no host time inside); "
                    "flops = 2 (d^2 + m d) per vector (algorithmic, the hi/lo split doubles the issue)",
        },
        "hot_first_gate": dict(rows=gate_rows, note="tq_decode_attention_gated over every layer (attention only), "
                               "threshold on the best hot logit <q,k>/sqrt(d) of every head of a kv group; error "
                               "of sequence 0 layer 0 against exact attention"),
        "error_vs_exact_fp16": dict(exact, note="sequence 0, layer 0, the step after the timed region, fp32 exact "
                                                "attention over the original fp16 K/V"),
        "context_tokens_per_step": ctx_per_step,
        "mall_scrub_mb_per_step": scrub_mb,
        "hot_per_layer": float(np.mean(hot_l)), "live_cold_per_layer": float(np.mean(cold_l)),
    }
    if not a.no_quality:
        line["quality"] = quality_block(torch, tqkv, wl)
        line["tensor_cache_tier"] = tensor_cache_block(torch, tqkv, w)
        line["compressed_mips"] = mips_block(torch, tqkv)
        line["multi_query"] = multi_query_block(torch, cache, w)
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line))


if __name__ == "__main__":
    main()
