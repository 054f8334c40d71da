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


def record_bytes(d, fmt):
    rb, tb, m = fmt
    return (d // 2) * (rb + tb) // 8 + m // 8 + 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b", choices=["llama8b", "ragged", "long"])
    ap.add_argument("--fmt", default="F3", choices=["F3", "F4", "F25"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-probe", action="store_true", help="time a plain device copy and exit")
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


def cpu_baseline(w, fmt, budget_s):
    """The CPU oracle, as it stands, on a bounded sample of the workload:
    prefill one (sequence, layer) to its full context with the oracle's own
    codec (untimed), then time its decode-attention step over that context
    until about budget_s seconds of attention have run.  BLAS limited to one
    thread."""
    from threadpoolctl import threadpool_limits

    from compressed_kv_decode_amd import workloads as wl
    from oracle import params
    from oracle.codec import Format
    from oracle.paging import SeqLayerCache

    with threadpool_limits(limits=1):
        pi, s = params.rotation(w.head_dim, w.seed), params.sketch(64, w.head_dim, w.seed)
        oc = SeqLayerCache(w.n_kv_heads, w.head_dim, w.window, Format(*fmt), pi, s, tau=2.0)
        k, v = wl.prefill_kv(w, 0, 0)
        oc.append(k, v)
        ctx = len(oc.hot) + len(oc.live)
        t0 = time.perf_counter()
        n = 0
        while True:
            oc.attend(wl.query(w, 0, 0, n))
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    return dict(value=ctx * n / el, unit="ctx tokens/s", cores=1, kind="oracle",
                sample=f"1 sequence x 1 layer of the workload, {ctx}-token context ({len(oc.live)} cold codes), "
                       f"{n} decode-attention steps of {w.n_q_heads} query heads in {el:.1f} s (prefill untimed); "
                       f"numpy fp64, BLAS on 1 thread")


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


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {a.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

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

    def step(t, probe):
        # the timed steps record nothing between the calls (an event record
        # costs the stream a few microseconds); the probe step after them does
        for l in range(L):
            cache.append(l, seqs, [1] * n_seq, step_k[t][l], step_v[t][l])
            if probe:
                att_ev[l][0].record()
            cache.attend(l, seqs, step_q[t][l], out=out)
            if probe:
                att_ev[l][1].record()
                if l == 0:
                    out0.copy_(out[0])
            cache.promote(l, seqs)

    for t in range(a.warmup):
        step(t, False)
    torch.cuda.synchronize()
    cache.profile_read()  # clear
    cache.profile_enable(True)
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_ev[0].record()
    for i, t in enumerate(range(a.warmup, total_steps)):
        step(t, False)
        step_ev[i + 1].record()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    cache.profile_enable(False)
    dec_ms, dec_n = cache.profile_read()
    step_ms = [step_ev[i].elapsed_time(step_ev[i + 1]) for i in range(a.steps)]
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
            "format": fmt_label, "hot_window": w.window,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic,
            "kernel": "k_decode (split-context attention over hot fp16 + cold codes)",
            "alg_bytes_per_launch": alg_bytes,
            "avg_launch_us": avg_launch_s * 1e6,
            "launches": dec_n,
            "achievable_copy_gbs": probe["gbs"],
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
        "error_vs_exact_fp16": dict(exact, note="sequence 0, layer 0, the step after the timed region, fp32 exact "
                                                "attention over the original fp16 K/V"),
        "context_tokens_per_step": ctx_per_step,
        "hot_per_layer": float(np.mean(hot_l)), "live_cold_per_layer": float(np.mean(cold_l)),
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, w.formats[0], a.cpu_seconds)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
