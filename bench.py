"""Benchmark of the deferred-RoPE paged attention hot path on one MI355X.

One step = one pass over the whole path on synthetic, HBM-resident inputs:
  decode pass : kvcache_append of the 64 new tokens, then lazyattn_decode over
                the Llama-3.1-8B-shaped batch (64 x 8193 tokens, 32 q / 8 KV
                heads, d_h 128, bf16, documents of 256..2048 tokens);
  prefill pass: kvcache_append of the 4 x 2048 prompt tokens, then
                lazyattn_prefill against 6144 cached document tokens each.
Prints one JSON line.  `value` is the decode pass's KV throughput (logical K+V
bytes of the attended tokens / decode-pass time); the prefill attention
TFLOP/s rides along.  After the timed steps, the metric's other two decode
workloads (Llama-3.1-70B-shaped decode, and the Zipf-skewed document-reuse
mix) are each timed the same way as a decode pass of their own, with their
own roofline and oracle baseline (keys "llama70b_decode", "zipf_reuse_decode";
the Zipf mix through the planned decode, which runs the readers of each
shared document together).
Kernel durations come from HIP events recorded on the stream the library
launches on (torch's current stream).  Before the W counted warm-up steps,
untimed steps run until the clock has settled (the prefill kernel's time
stops changing; "clock_settle" in the record keeps the cold figures;
--no-settle skips this).
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "decode KV GB/s (% HBM peak) + prefill attn TFLOP/s, 8B-shape lazy-RoPE"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")
DECODE_SOURCES = ["position_agnostic_kv_amd/csrc/decode.hip", "position_agnostic_kv_amd/csrc/common.h"]
PREFILL_SOURCES = ["position_agnostic_kv_amd/csrc/prefill.hip", "position_agnostic_kv_amd/csrc/common.h"]


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(name, sources):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, or None
    if it is missing or the kernel source changed since the counters were taken."""
    path = os.path.join(PROFILES, f"{name}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(sources):
        return None
    return rec.get("traffic_bytes_per_launch")


def decode_algorithmic_bytes(case):
    """K+V of every attended token once, plus q in, out, table words and
    lengths (and one fill count per block when documents end mid-block)."""
    esz = 2
    d, hq, hkv = case.head_dim, case.num_q_heads, case.num_kv_heads
    tokens = int(case.layout.total_lens.sum())
    kv = tokens * hkv * d * 2 * esz
    qo = case.batch * hq * d * esz * 2
    nblk = int(sum(-(-int(n) // 16) for n in case.seq_lens))
    table = nblk * (4 if case.block_fill is None else 5) + case.batch * 8
    return kv, kv + qo + table


def host_threads():
    """Host cores this process may run on (the oracle's BLAS thread count)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


class SampleParity:
    """Element-wise error of the GPU output against the oracle on the rows the
    CPU baseline computed (bf16 tolerances: 2e-2 max-abs, 5e-3 mean-abs)."""

    def __init__(self):
        self.max_abs, self.sum_abs, self.count = 0.0, 0.0, 0

    def add(self, got, want):
        err = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(want, dtype=np.float64))
        self.max_abs = max(self.max_abs, float(err.max()))
        self.sum_abs += float(err.sum())
        self.count += err.size

    def record(self, what):
        mean = self.sum_abs / max(self.count, 1)
        return {"max_abs": self.max_abs, "mean_abs": mean, "elements": self.count,
                "tolerance": {"max_abs": 2e-2, "mean_abs": 5e-3},
                "within_tolerance": bool(self.max_abs <= 2e-2 and mean <= 5e-3),
                "sample": f"{what}: the GPU output of the timed steps against the float64 oracle on the "
                          f"CPU baseline's sample"}


def cpu_baseline_decode(case, dc, seconds, out=None):
    """The oracle, single-threaded, on whole (sequence, KV head) groups of the
    same workload until `seconds` of CPU work; scaled to GB/s of K+V.  With
    the GPU output `out` of the same inputs, also returns its error against
    the oracle on those groups (else None)."""
    from threadpoolctl import threadpool_limits
    import oracle
    import workloads as W
    import torch
    lay = case.layout
    q = W.to_float(case.q, case.dtype)
    g = case.num_q_heads // case.num_kv_heads
    done_bytes, groups, t_used = 0, 0, 0.0
    par = SampleParity()
    nthr = host_threads()
    with threadpool_limits(nthr):
        for b in range(case.batch):
            nb = -(-int(case.seq_lens[b]) // 16)
            ids = (lay.table[b, :nb] & 0xFFFF).astype(np.int64)
            sel = torch.from_numpy(ids).to(dc.k_pool.device)
            kp = W.to_float(dc.k_pool.index_select(0, sel), case.dtype)
            vp = W.to_float(dc.v_pool.index_select(0, sel), case.dtype)
            row = ((lay.table[b, :nb] & 0xFFFF0000) | np.arange(nb, dtype=np.uint32)).astype(np.uint32)
            for kvh in range(case.num_kv_heads):
                t0 = time.perf_counter()
                k_hat, v_hat = oracle.materialize_sequence(kp, vp, row, int(case.seq_lens[b]), kvh,
                                                           case.rope_theta)
                qr = oracle.rope(q[b, kvh * g:(kvh + 1) * g], int(case.q_pos[b]), case.rope_theta)
                p = oracle.softmax(case.scale * (qr @ k_hat.T))
                o = p @ v_hat
                t_used += time.perf_counter() - t0
                if out is not None:
                    par.add(W.to_float(out[b, kvh * g:(kvh + 1) * g], case.dtype), o)
                done_bytes += int(case.seq_lens[b]) * case.head_dim * 2 * 2
                groups += 1
                if t_used >= seconds:
                    break
            if t_used >= seconds:
                break
    base = {"value": done_bytes / t_used / 1e9, "unit": "GB/s", "cores": nthr, "kind": "oracle",
            "sample": f"{groups} (sequence, KV head) groups of {case.name} "
                      f"({groups * g} query heads, {done_bytes // (case.head_dim * 4)} tokens x KV heads), "
                      f"{t_used:.1f} s, float64 numpy, {nthr} BLAS threads"}
    return base, (par.record(f"{groups * g} query heads of {case.name}") if out is not None else None)


def cpu_baseline_prefill(case, dc, seconds, out=None):
    """The oracle on the prompt rows of (sequence, head) pairs of the prefill
    workload, head by head, until `seconds` of CPU work; with the GPU output
    `out`, also its error against the oracle on those rows (else None)."""
    from threadpoolctl import threadpool_limits
    import oracle
    import workloads as W
    import torch
    lay = case.layout
    g = case.num_q_heads // case.num_kv_heads
    q = W.to_float(case.q, case.dtype)
    plen = case.max_q_len
    flops, t_used, rows_done, heads = 0, 0.0, 0, 0
    par = SampleParity()
    nthr = host_threads()
    with threadpool_limits(nthr):
        for b in range(case.batch):
            nb = -(-int(case.seq_lens[b]) // 16)
            ids = (lay.table[b, :nb] & 0xFFFF).astype(np.int64)
            sel = torch.from_numpy(ids).to(dc.k_pool.device)
            kp = W.to_float(dc.k_pool.index_select(0, sel), case.dtype)
            vp = W.to_float(dc.v_pool.index_select(0, sel), case.dtype)
            row = ((lay.table[b, :nb] & 0xFFFF0000) | np.arange(nb, dtype=np.uint32)).astype(np.uint32)
            kv_len = int(case.seq_lens[b])
            cached = kv_len - plen
            q0 = int(case.cu_q_lens[b])
            for h in range(case.num_q_heads):
                for r0 in range(0, plen, 128):
                    rows = np.arange(r0, min(plen, r0 + 128))
                    t0 = time.perf_counter()
                    o = oracle.prefill_rows(q[q0 + rows, h], rows, plen, int(lay.tail_pos[b]), kp, vp, row,
                                            kv_len, h // g, case.scale, case.rope_theta)
                    t_used += time.perf_counter() - t0
                    if out is not None:
                        idx = torch.from_numpy(q0 + rows).to(out.device)
                        par.add(W.to_float(out[:, h].index_select(0, idx), case.dtype), o)
                    flops += 4 * case.head_dim * int(np.sum(cached + rows + 1))
                    rows_done += len(rows)
                heads += 1
                if t_used >= seconds:
                    break
            if t_used >= seconds:
                break
    base = {"value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": nthr, "kind": "oracle",
            "sample": f"{rows_done} prompt rows ({heads} (sequence, head) pairs) of llama8b_prefill, "
                      f"{t_used:.1f} s, float64 numpy, {nthr} BLAS threads"}
    return base, (par.record(f"{rows_done} prompt rows of llama8b_prefill") if out is not None else None)


def overhead_main(args):
    """Cost of laziness: the lazy kernels against the non-lazy baseline
    (lazyattn_*_eager: keys taken as already rotated to absolute positions,
    offsets ignored, the query rotated once) on identical inputs.  Launches
    alternate lazy / eager so clock drift hits both alike; medians of
    `args.steps` launches each.  Also a documents-per-sequence sweep of the 8B
    decode shape (1, 16, 64 documents per 8192-token sequence).  One JSON line."""
    import torch
    import position_agnostic_kv_amd as pak
    import workloads as W
    from workloads.device import DeviceInputs

    pak.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def ab(run_lazy, run_eager):
        for _ in range(args.warmup):
            run_lazy()
            run_eager()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for e in ev:
            e[0].record()
            run_lazy()
            e[1].record()
            run_eager()
            e[2].record()
        torch.cuda.synchronize()
        lazy = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
        eager = float(np.median([e[1].elapsed_time(e[2]) for e in ev]))
        return {"lazy_ms": round(lazy, 4), "eager_ms": round(eager, 4),
                "overhead_pct": round(100.0 * (lazy - eager) / eager, 3)}

    def decode_ab(case):
        W.materialize_torch(case, dev)
        d = DeviceInputs(case, dev)
        pak.kvcache_append(d.k_pool, d.v_pool, d.k_new, d.v_new, d.slots)
        out = torch.empty_like(d.q)
        kw = dict(scale=case.scale, rope_theta=case.rope_theta, out=out)
        r = ab(lambda: pak.lazyattn_decode(d.q, d.q_pos, d.k_pool, d.v_pool, d.table, d.seq_lens, **kw),
               lambda: pak.lazyattn_decode_eager(d.q, d.q_pos, d.k_pool, d.v_pool, d.table, d.seq_lens, **kw))
        docs = [len(x) for x in case.layout.doc_spans]
        r["docs_per_seq"] = round(float(np.mean(docs)), 2)
        r["offset_changes_per_seq"] = round(float(np.mean(docs)) + 1, 2)  # + the new token's block
        del d, out
        case.q = case.k_pool = case.v_pool = case.k_new = case.v_new = None
        torch.cuda.empty_cache()
        return r

    res = {"metric": "lazy vs eager (non-lazy baseline) kernel time, same inputs", "unit": "ms",
           "steps": args.steps, "warmup": args.warmup, "data": "synthetic"}
    res["decode_llama8b"] = decode_ab(W.llama8b_decode())
    pcase = W.llama8b_prefill()
    W.materialize_torch(pcase, dev)
    pd = DeviceInputs(pcase, dev)
    pak.kvcache_append(pd.k_pool, pd.v_pool, pd.k_new, pd.v_new, pd.slots)
    pout = torch.empty_like(pd.q)
    pkw = dict(scale=pcase.scale, rope_theta=pcase.rope_theta, out=pout)
    res["prefill_llama8b"] = ab(
        lambda: pak.lazyattn_prefill(pd.q, pd.cu, pd.q_pos_start, pd.k_pool, pd.v_pool, pd.table,
                                     pd.seq_lens, pcase.max_q_len, **pkw),
        lambda: pak.lazyattn_prefill_eager(pd.q, pd.cu, pd.q_pos_start, pd.k_pool, pd.v_pool, pd.table,
                                           pd.seq_lens, pcase.max_q_len, **pkw))
    del pd, pout
    torch.cuda.empty_cache()
    sweep = {}
    for label, blocks in (("1_doc", (512, 512)), ("16_docs", (32, 32)), ("64_docs", (8, 8))):
        sweep[label] = decode_ab(W.decode_case(2, 64, 32, 8, 128, 8192, blocks, name=f"sweep_{label}"))
    res["decode_docs_sweep"] = sweep
    print(json.dumps(res), flush=True)


def fp8_decode_algorithmic_bytes(case):
    """decode_algorithmic_bytes with one byte per K/V element."""
    kv, total = decode_algorithmic_bytes(case)
    return kv // 2, total - kv // 2


# 8-bit pools timed by --shapes: (code generator, k_scale, v_scale) per format
POOL8_FORMATS = {"fp8": ("e4m3_codes_torch", 0.25, 0.125), "int8": ("int8_codes_torch", 0.01, 0.005)}


def _pool8(case, d, fmt):
    """Random 8-bit pools of the case's shape on the GPU, with the step's new
    rows quantised in by the format's append; returns (k, v, k_scale, v_scale)."""
    import position_agnostic_kv_amd as pak
    import workloads as W
    gen, ks, vs = POOL8_FORMATS[fmt]
    shape = tuple(d.k_pool.shape)
    k8 = getattr(W, gen)(shape, d.k_pool.device, case.seed + 5000)
    v8 = getattr(W, gen)(shape, d.k_pool.device, case.seed + 6000)
    getattr(pak, f"kvcache_append_{fmt}")(k8, v8, d.k_new, d.v_new, d.slots, ks, vs)
    return k8, v8, ks, vs


def fp8_decode_shape(case, d, out, ws, timed, fmt="fp8"):
    """Time lazyattn_decode_fp8 (or _int8) on the case's layout with an 8-bit
    pool of random codes (E4M3: k_scale 0.25, v_scale 0.125; int8: 0.01,
    0.005); the step's new rows are quantised in by the format's append
    first."""
    import torch
    import position_agnostic_kv_amd as pak
    k8, v8, ks, vs = _pool8(case, d, fmt)
    fn = getattr(pak, f"lazyattn_decode_{fmt}")
    med, p10, p90 = timed(lambda: fn(d.q, d.q_pos, k8, v8, d.table, d.seq_lens, ks, vs, scale=case.scale,
                                     rope_theta=case.rope_theta, out=out, workspace=ws))
    kv, alg = fp8_decode_algorithmic_bytes(case)
    del k8, v8
    torch.cuda.empty_cache()
    return {"ms_p50": round(med, 4), "ms_p10": round(p10, 4), "ms_p90": round(p90, 4),
            "kv_bytes_logical": kv, "gbps_logical": round(kv / (med * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(alg / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "tokens_per_s": round(float(case.layout.total_lens.sum()) / (med * 1e-3), 0)}


def fp8_prefill_shape(case, d, out, timed, fmt="fp8"):
    """Time lazyattn_prefill_fp8 (or _int8: widening pass and prefill) on the
    case's layout with an 8-bit pool of random codes; the prompts' rows are
    quantised in by the format's append first."""
    import torch
    import position_agnostic_kv_amd as pak
    k8, v8, ks, vs = _pool8(case, d, fmt)
    ws = torch.empty(pak.prefill_fp8_workspace_size(case.batch, d.table.shape[1], case.num_kv_heads),
                     dtype=torch.uint8, device=d.k_pool.device)
    fn = getattr(pak, f"lazyattn_prefill_{fmt}")
    med, p10, p90 = timed(lambda: fn(d.q, d.cu, d.q_pos_start, k8, v8, d.table, d.seq_lens, case.max_q_len, ks,
                                     vs, scale=case.scale, rope_theta=case.rope_theta, out=out, workspace=ws))
    del k8, v8, ws
    torch.cuda.empty_cache()
    fl = case.attention_flops()
    return {"ms_p50": round(med, 4), "ms_p10": round(p10, 4), "ms_p90": round(p90, 4),
            "tflops": round(fl / (med * 1e-3) / 1e12, 1),
            "frac_of_bf16_peak": round(fl / (med * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}


def shapes_main(args):
    """Kernel time of every decode workload (8B, 70B, Zipf mix, 8B with
    documents of any token count, 8B with ALiBi, and GQA 4 against
    multi-query groups of 32 and 64 at equal K/V bytes) and of the 8B prefill (RoPE,
    ALiBi, documents of any token count), each on its own HBM-resident
    inputs: medians and p10/p90 of
    `args.steps` launches after `args.warmup`.  One JSON line."""
    import torch
    import position_agnostic_kv_amd as pak
    import workloads as W
    from workloads.device import DeviceInputs

    pak.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for e in ev:
            e[0].record()
            fn()
            e[1].record()
        torch.cuda.synchronize()
        x = np.array([e[0].elapsed_time(e[1]) for e in ev])
        return float(np.median(x)), float(np.percentile(x, 10)), float(np.percentile(x, 90))

    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.int16, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    res = {"metric": "kernel time per workload (decode: K+V GB/s; prefill: attention TFLOP/s)",
           "steps": args.steps, "warmup": args.warmup, "data": "synthetic", "peak_hbm_gbps": HBM_PEAK_GBPS,
           "peak_bf16_tflops": BF16_PEAK_TFLOPS}
    for name in ("llama8b_decode", "llama70b_decode", "zipf_reuse_decode", "llama8b_decode_ragged",
                 "decode_g4_equal_bytes", "decode_g32_equal_bytes", "decode_g64_equal_bytes"):
        case = W.make(name)
        W.materialize_torch(case, dev)
        d = DeviceInputs(case, dev)
        pak.kvcache_append(d.k_pool, d.v_pool, d.k_new, d.v_new, d.slots)
        out = torch.empty_like(d.q)
        wsb = pak.decode_workspace_size(case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim,
                                        case.layout.table.shape[1], 0)
        ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=dev)
        med, p10, p90 = timed(lambda: pak.lazyattn_decode(d.q, d.q_pos, d.k_pool, d.v_pool, d.table, d.seq_lens,
                                                          scale=case.scale, rope_theta=case.rope_theta,
                                                          out=out, workspace=ws, block_fill=d.fill))
        kv, alg = decode_algorithmic_bytes(case)
        phys = int(case.k_pool.numel()) * 2 * 2 if name == "zipf_reuse_decode" else None
        r = {"ms_p50": round(med, 4), "ms_p10": round(p10, 4), "ms_p90": round(p90, 4),
             "kv_bytes_logical": kv, "gbps_logical": round(kv / (med * 1e-3) / 1e9, 1),
             "frac_of_hbm_peak": round(alg / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
             "batch": case.batch, "q_heads": case.num_q_heads, "kv_heads": case.num_kv_heads}
        if phys is not None:
            r["pool_bytes_physical"] = phys
        if d.fill is not None:
            r["table_slots_per_token"] = round(float(case.seq_lens.sum() / case.layout.total_lens.sum()), 4)
        res[name] = r
        if name == "zipf_reuse_decode":  # the planned decode: shared documents read together
            res[name + "_planned"] = planned_decode_shape(case, d, out, timed)
        if name in ("llama8b_decode", "llama70b_decode"):  # the same geometry over an 8-bit (E4M3) pool
            res[name + "_fp8"] = fp8_decode_shape(case, d, out, ws, timed)
            if name == "llama8b_decode":  # and over an int8 pool
                res[name + "_int8"] = fp8_decode_shape(case, d, out, ws, timed, "int8")
        if name == "llama8b_decode":  # the same inputs read with ALiBi biases instead of RoPE
            import oracle
            tab = torch.from_numpy(W.block_frame_table(case.layout).view(np.int32)).to(dev)
            sl = torch.from_numpy(oracle.alibi_slopes(case.num_q_heads).astype(np.float32)).to(dev)
            med, p10, p90 = timed(lambda: pak.lazyattn_decode_alibi(d.q, d.q_pos, d.k_pool, d.v_pool, tab,
                                                                    d.seq_lens, sl, out=out, workspace=ws))
            res["llama8b_decode_alibi"] = {"ms_p50": round(med, 4), "ms_p10": round(p10, 4),
                                           "ms_p90": round(p90, 4),
                                           "gbps_logical": round(kv / (med * 1e-3) / 1e9, 1),
                                           "frac_of_hbm_peak": round(alg / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        del d, out, ws
        case.q = case.k_pool = case.v_pool = case.k_new = case.v_new = None
        torch.cuda.empty_cache()
    case = W.llama8b_prefill()
    W.materialize_torch(case, dev)
    d = DeviceInputs(case, dev)
    pak.kvcache_append(d.k_pool, d.v_pool, d.k_new, d.v_new, d.slots)
    out = torch.empty_like(d.q)
    med, p10, p90 = timed(lambda: pak.lazyattn_prefill(d.q, d.cu, d.q_pos_start, d.k_pool, d.v_pool, d.table,
                                                       d.seq_lens, case.max_q_len, scale=case.scale,
                                                       rope_theta=case.rope_theta, out=out))
    fl = case.attention_flops()
    res["llama8b_prefill"] = {"ms_p50": round(med, 4), "ms_p10": round(p10, 4), "ms_p90": round(p90, 4),
                              "attention_flops": fl, "tflops": round(fl / (med * 1e-3) / 1e12, 1),
                              "frac_of_bf16_peak": round(fl / (med * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    res["llama8b_prefill_fp8"] = fp8_prefill_shape(case, d, out, timed)  # the same shape over an 8-bit pool
    res["llama8b_prefill_int8"] = fp8_prefill_shape(case, d, out, timed, "int8")  # and over an int8 pool
    import oracle
    tab = torch.from_numpy(W.block_frame_table(case.layout).view(np.int32)).to(dev)
    sl = torch.from_numpy(oracle.alibi_slopes(case.num_q_heads).astype(np.float32)).to(dev)
    med, p10, p90 = timed(lambda: pak.lazyattn_prefill_alibi(d.q, d.cu, d.q_pos_start, d.k_pool, d.v_pool, tab,
                                                             d.seq_lens, case.max_q_len, sl, out=out))
    res["llama8b_prefill_alibi"] = {"ms_p50": round(med, 4), "ms_p10": round(p10, 4), "ms_p90": round(p90, 4),
                                    "tflops": round(fl / (med * 1e-3) / 1e12, 1),
                                    "frac_of_bf16_peak": round(fl / (med * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    # the same inputs through the precise prefill (twice the Q.K^T products;
    # the rate counts the algorithmic FLOPs only)
    med, p10, p90 = timed(lambda: pak.lazyattn_prefill_precise(d.q, d.cu, d.q_pos_start, d.k_pool, d.v_pool,
                                                               d.table, d.seq_lens, case.max_q_len,
                                                               scale=case.scale, rope_theta=case.rope_theta,
                                                               out=out))
    res["llama8b_prefill_precise"] = {"ms_p50": round(med, 4), "ms_p10": round(p10, 4), "ms_p90": round(p90, 4),
                                      "tflops": round(fl / (med * 1e-3) / 1e12, 1),
                                      "frac_of_bf16_peak": round(fl / (med * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    del d, out
    case.q = case.k_pool = case.v_pool = case.k_new = case.v_new = None
    torch.cuda.empty_cache()
    # documents of any token count: a document's partly filled last block
    # costs MFMA work on its masked slots
    case = W.make("llama8b_prefill_ragged")
    W.materialize_torch(case, dev)
    d = DeviceInputs(case, dev)
    pak.kvcache_append(d.k_pool, d.v_pool, d.k_new, d.v_new, d.slots)
    out = torch.empty_like(d.q)
    med, p10, p90 = timed(lambda: pak.lazyattn_prefill(d.q, d.cu, d.q_pos_start, d.k_pool, d.v_pool, d.table,
                                                       d.seq_lens, case.max_q_len, scale=case.scale,
                                                       rope_theta=case.rope_theta, out=out, block_fill=d.fill))
    fl = case.attention_flops()
    res["llama8b_prefill_ragged"] = {"ms_p50": round(med, 4), "ms_p10": round(p10, 4), "ms_p90": round(p90, 4),
                                     "attention_flops": fl, "tflops": round(fl / (med * 1e-3) / 1e12, 1),
                                     "frac_of_bf16_peak": round(fl / (med * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                                     "table_slots_per_token": round(float(case.seq_lens.sum()
                                                                          / case.layout.total_lens.sum()), 4)}
    print(json.dumps(res), flush=True)


# --shapes launches each kernel on these workloads, in this order, warmup +
# steps times each (other kernels in between); the profile summary splits a
# kernel's dispatches into consecutive runs accordingly.  Value: (profile
# file stem, kernel source files, algorithmic bytes of one launch).
SHAPES_DISPATCH_ORDER = {
    "lazyattn::decode_mma16_kernel<4, 0>": ["llama8b_decode", "zipf_reuse_decode", "llama8b_decode_ragged",
                                            "decode_g4_equal_bytes"],
    # the planned decode (shared documents read together), on the Zipf mix
    "lazyattn::decode_planned_kernel<4>": ["zipf_reuse_decode_planned"],
    "lazyattn::decode_mma16_wide_kernel<2, 0>": ["decode_g32_equal_bytes"],
    "lazyattn::decode_mma16_wide_kernel<4, 0>": ["decode_g64_equal_bytes"],
    "lazyattn::decode_mma16_kernel<4, 2>": ["llama8b_decode_alibi"],
    "lazyattn::decode_mma16_kernel<8, 0>": ["llama70b_decode"],
    "lazyattn::decode_mma8_kernel<4, 0>": ["llama8b_decode_fp8"],
    "lazyattn::decode_int8_kernel<4>": ["llama8b_decode_int8"],
    "lazyattn::decode_mma8_kernel<8, 0>": ["llama70b_decode_fp8"],
    # the 8-bit prefill: the widening pass, then the bf16 kernel on the widened copy
    "lazyattn::prefill_kernel<128, 4, 0, false>": ["llama8b_prefill", "llama8b_prefill_fp8", "llama8b_prefill_int8",
                                            "llama8b_prefill_ragged"],
    "lazyattn::widen_fp8_kernel": ["llama8b_prefill_fp8_widen"],
    "lazyattn::widen_int8_kernel": ["llama8b_prefill_int8_widen"],
    "lazyattn::prefill_kernel<128, 4, 2, false>": ["llama8b_prefill_alibi"],
    # the precise prefill (query as bf16 hi + lo, tiles cut at document ends)
    "lazyattn::prefill_kernel<128, 4, 0, true>": ["llama8b_prefill_precise"],
}
PROFILE_STEMS = {
    "llama8b_decode": "decode_llama8b", "zipf_reuse_decode": "decode_zipf",
    "zipf_reuse_decode_planned": "decode_zipf_planned",
    "llama8b_decode_ragged": "decode_llama8b_ragged", "llama8b_decode_alibi": "decode_llama8b_alibi",
    "llama70b_decode": "decode_llama70b", "llama8b_decode_fp8": "decode_llama8b_fp8",
    "llama70b_decode_fp8": "decode_llama70b_fp8", "llama8b_prefill": "prefill_llama8b",
    "llama8b_prefill_ragged": "prefill_llama8b_ragged", "llama8b_prefill_alibi": "prefill_llama8b_alibi",
    "llama8b_prefill_fp8": "prefill_llama8b_fp8", "llama8b_prefill_fp8_widen": "widen_llama8b_fp8",
    "llama8b_decode_int8": "decode_llama8b_int8", "llama8b_prefill_int8": "prefill_llama8b_int8",
    "llama8b_prefill_int8_widen": "widen_llama8b_int8", "llama8b_prefill_precise": "prefill_llama8b_precise",
    "decode_g4_equal_bytes": "decode_g4_equal_bytes",
    "decode_g32_equal_bytes": "decode_g32_equal_bytes", "decode_g64_equal_bytes": "decode_g64_equal_bytes",
}


def planned_decode_shape(case, d, out, timed):
    """--shapes: the planned decode (lazyattn_decode_planned) on a decode
    workload's inputs; the plan is built once on the host, outside the
    timing."""
    import position_agnostic_kv_amd as pak
    import torch

    t0 = time.perf_counter()
    plan = pak.decode_plan(d.table, d.seq_lens, case.num_q_heads, case.num_kv_heads)
    plan_ms = (time.perf_counter() - t0) * 1e3
    wsb = pak.decode_planned_workspace_size(case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim,
                                            plan.max_items_per_seq)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=d.q.device)
    med, p10, p90 = timed(lambda: pak.lazyattn_decode_planned(d.q, d.q_pos, d.k_pool, d.v_pool, d.table,
                                                              d.seq_lens, plan, scale=case.scale,
                                                              rope_theta=case.rope_theta, out=out, workspace=ws))
    kv, alg = decode_algorithmic_bytes(case)
    return {"ms_p50": round(med, 4), "ms_p10": round(p10, 4), "ms_p90": round(p90, 4),
            "gbps_logical": round(kv / (med * 1e-3) / 1e9, 1),
            "pool_bytes_physical": int(d.k_pool.numel()) * 2 * 2,
            "plan": {"items": plan.num_items, "max_items_per_seq": plan.max_items_per_seq,
                     "host_build_ms": round(plan_ms, 2)}}


def _profile_workload_bytes(name):
    """(description, algorithmic bytes of one launch) of a --shapes workload."""
    import workloads as W
    pool = "E4M3" if "_fp8" in name else "int8" if "_int8" in name else None
    if name.endswith("_widen"):
        case = W.make("llama8b_prefill")
        slots = int(sum(-(-int(n) // W.BLOCK) for n in case.seq_lens)) * case.num_kv_heads
        total = slots * (2 * 2048 + 2 * 4096)
        return (f"{name}: the {slots} visible (block, KV head) slots of llama8b_prefill over an {pool} pool, "
                f"widened once to bf16; algorithmic = 2 x 2 KiB of codes read + 2 x 4 KiB bf16 written per "
                f"slot"), total
    base = (name.replace("_fp8", "").replace("_int8", "").replace("_alibi", "").replace("_planned", "")
            .replace("_precise", ""))
    case = W.make(base)
    if case.kind == "decode":
        kv, total = decode_algorithmic_bytes(case)
        if pool:
            kv, total = fp8_decode_algorithmic_bytes(case)
        desc = (f"{name}: {case.batch} seqs, {int(case.layout.total_lens.sum())} tokens attended, "
                f"{case.num_q_heads} q / {case.num_kv_heads} KV heads, d_h {case.head_dim}, "
                f"{pool + ' pool, bf16 q' if pool else 'bf16'}; algorithmic = K+V once + q, out, "
                f"table words")
        return desc, total
    toks = int(case.layout.total_lens.sum())
    rows = int(case.cu_q_lens[-1])
    total = toks * case.num_kv_heads * case.head_dim * 2 * 2 + 2 * rows * case.num_q_heads * case.head_dim * 2
    desc = (f"{name}: {case.batch} seqs, {toks} K/V tokens ({rows} prompt rows), {case.num_q_heads} q / "
            f"{case.num_kv_heads} KV heads, d_h {case.head_dim}, "
            f"{'bf16 copy widened from an ' + pool + ' pool' if pool else 'bf16'}; "
            f"algorithmic = K+V once + q + out")
    return desc, total


def _rocpd_rows(root, query):
    """Rows of a query over every rocprofv3 result database (rocpd SQLite) under root."""
    import sqlite3
    rows = []
    for dirpath, _, files in os.walk(root):
        for fn in sorted(files):
            if fn.endswith("_results.db"):
                con = sqlite3.connect(os.path.join(dirpath, fn))
                rows.extend(con.execute(query).fetchall())
                con.close()
    if not rows:
        raise SystemExit(f"no rocprofv3 results under {root}")
    return rows


def _kernel_key(name):
    name = name.replace("(anonymous namespace)::", "").split("(")[0].strip()
    return name[5:] if name.startswith("void ") else name


def pmc_summary_main(args):
    """Write profiles/*_pmc.json and profiles/decode_shapes_kernel_trace.md
    from the rocprofv3 result databases of three runs of `bench.py --shapes --steps S
    --warmup W --copy-calibration` (FETCH_SIZE, WRITE_SIZE, kernel trace).
    Counters are per dispatch; each is scaled by what it reads for the
    calibration dispatches at the start of the run (a 1 GiB fill for
    WRITE_SIZE, a 1 GiB device copy for FETCH_SIZE)."""
    fetch_dir, write_dir, trace_dir = args.pmc_summary
    per_run = args.steps + args.warmup
    known = 1 << 30

    def counters(root, counter):
        vals = {}
        for disp, kname, cname, value in _rocpd_rows(
                root, "select dispatch_id, kernel_name, counter_name, value from counters_collection"):
            if cname != counter:
                continue
            prev = vals.get(int(disp), (_kernel_key(kname), 0.0))
            vals[int(disp)] = (prev[0], prev[1] + float(value))
        return [vals[k] for k in sorted(vals)]

    fetch = counters(fetch_dir, "FETCH_SIZE")
    write = counters(write_dir, "WRITE_SIZE")
    first_copy = next(v for n, v in fetch if "copyBuffer" in n or "copy" in n.lower())
    first_fill = next(v for n, v in write if "Fill" in n)
    fetch_scale = known / (first_copy * 1024)
    write_scale = known / (first_fill * 1024)

    durs = {}
    for name, start, end in sorted(_rocpd_rows(trace_dir, "select name, start, end from kernels"),
                                   key=lambda r: int(r[1])):
        durs.setdefault(_kernel_key(name), []).append((int(end) - int(start)) / 1000.0)

    def runs(seq, kernel):
        vals = [v for n, v in seq if n == kernel]
        return [vals[i * per_run:(i + 1) * per_run] for i in range(len(vals) // per_run)]

    cmd_base = f"python -u bench.py --shapes --steps {args.steps} --warmup {args.warmup} --copy-calibration"
    cal = {"known_bytes": known, "copy_fetch_kib": round(first_copy, 3), "fetch_scale": round(fetch_scale, 5),
           "fill_write_kib": round(first_fill, 3), "write_scale": round(write_scale, 5),
           "note": "1 GiB device copy read back by FETCH_SIZE; 1 GiB fill by WRITE_SIZE"}
    for kernel, names in SHAPES_DISPATCH_ORDER.items():
        fr, wr = runs(fetch, kernel), runs(write, kernel)
        tr = [durs.get(kernel, [])[i * per_run:(i + 1) * per_run] for i in range(len(names))]
        if len(fr) != len(names) or len(wr) != len(names):
            print(f"skip {kernel}: {len(fr)}/{len(wr)} runs for {len(names)} workloads", file=sys.stderr)
            continue
        for name, f_run, w_run, t_run in zip(names, fr, wr, tr):
            desc, alg = _profile_workload_bytes(name)
            f_kib = float(np.mean(f_run[args.warmup:]))
            w_kib = float(np.mean(w_run[args.warmup:]))
            traffic = int(round(f_kib * 1024 * fetch_scale + w_kib * 1024 * write_scale))
            src = PREFILL_SOURCES if "prefill" in kernel or "widen" in kernel else DECODE_SOURCES
            rec = {"kernel": kernel.replace("lazyattn::", ""), "workload": desc, "source_files": src,
                   "source_hash": source_hash(src), "fetch_kib_per_dispatch": round(f_kib, 3),
                   "write_kib_per_dispatch": round(w_kib, 3), "dispatches": len(f_run) - args.warmup,
                   "copy_calibration": cal, "traffic_bytes_per_launch": traffic, "algorithmic_bytes": alg,
                   "traffic_over_algorithmic": round(traffic / alg, 4),
                   "trace_avg_duration_us": round(float(np.mean(t_run[args.warmup:])), 1) if t_run else None,
                   "commands": [f"rocprofv3 --pmc FETCH_SIZE -d {fetch_dir} -o run -- {cmd_base}",
                                f"rocprofv3 --pmc WRITE_SIZE -d {write_dir} -o run -- {cmd_base}",
                                f"rocprofv3 --kernel-trace --stats -d {trace_dir} -o run -- {cmd_base}",
                                f"python bench.py --pmc-summary {fetch_dir} {write_dir} {trace_dir} "
                                f"--steps {args.steps} --warmup {args.warmup}"]}
            path = os.path.join(PROFILES, f"{PROFILE_STEMS[name]}_pmc.json")
            with open(path, "w") as f:
                json.dump(rec, f, indent=1)
                f.write("\n")
            print(f"{path}: traffic/algorithmic {rec['traffic_over_algorithmic']}, "
                  f"{rec['trace_avg_duration_us']} us")

    # kernel-trace summary: every kernel, then the per-workload runs
    lines = ["# rocprofv3 kernel trace: bench.py --shapes (every decode workload, the 8-bit pool, ALiBi; "
             "8B prefill, ALiBi and ragged prefill)", "",
             "Command (GPU box, from the repository root):", "",
             f"    rocprofv3 --kernel-trace --stats -d {trace_dir} -o run -- {cmd_base}", "",
             f"Summarised by `python bench.py --pmc-summary {fetch_dir} {write_dir} {trace_dir} "
             f"--steps {args.steps} --warmup {args.warmup}`.  Torch's fill, copy and random kernels are input "
             "generation or the counter calibration, outside the timed work.", "",
             "kernel | calls | avg us | total us | %", "---|---|---|---|---"]
    tot = sum(sum(v) for v in durs.values())
    for k, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{k[:90]} | {len(v)} | {np.mean(v):.1f} | {sum(v):.1f} | {100 * sum(v) / tot:.1f}")
    lines += ["", f"Per workload ({args.warmup} warm-up + {args.steps} timed dispatches each; the timed ones):", "",
              "kernel | workload | median us | min us | max us", "---|---|---|---|---"]
    for kernel, names in SHAPES_DISPATCH_ORDER.items():
        v = durs.get(kernel, [])
        for i, name in enumerate(names):
            run = v[i * per_run:(i + 1) * per_run][args.warmup:]
            if run:
                lines.append(f"{kernel.replace('lazyattn::', '')} | {name} | {np.median(run):.1f} | "
                             f"{min(run):.1f} | {max(run):.1f}")
    with open(os.path.join(PROFILES, "decode_shapes_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote profiles/decode_shapes_kernel_trace.md")


ACTIVITY_COUNTERS = ["GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                     "SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_LDS_IDX_ACTIVE",
                     "SQ_LDS_BANK_CONFLICT", "SQ_BUSY_CU_CYCLES"]
MI355X_XCDS, MI355X_CUS, MI355X_SIMDS = 8, 256, 1024


def activity_summary_main(args):
    """Write profiles/decode_prefill_shapes_activity.md from one rocprofv3 run
    of `bench.py --shapes` with ACTIVITY_COUNTERS: per kernel and workload the
    clock, MFMA utilisation (rocprofv3's MfmaUtil: MFMA-busy cycles over GPU
    cycles x SIMDs), the bf16 MFMA FLOPs the counters saw against the
    algorithmic ones, VALU busy, MFMA/VALU co-issue and LDS utilisation.  The
    per-dispatch GRBM_GUI_ACTIVE is summed over the 8 XCDs, so it is divided
    by 8 to get GPU cycles."""
    root = args.activity_summary
    per_run = args.steps + args.warmup
    vals, names, durs = {}, {}, {}
    for disp, kname, cname, value, start, end in _rocpd_rows(
            root, "select dispatch_id, kernel_name, counter_name, value, start, end from counters_collection"):
        d = int(disp)
        vals.setdefault(d, {})
        vals[d][cname] = vals[d].get(cname, 0.0) + float(value)
        names[d] = _kernel_key(kname)
        durs[d] = (int(end) - int(start)) * 1e-9
    order = sorted(vals)
    cmd = (f"rocprofv3 --pmc {' '.join(ACTIVITY_COUNTERS)} -d {root} -o run -- python -u bench.py --shapes "
           f"--steps {args.steps} --warmup {args.warmup}")
    lines = ["# rocprofv3 activity counters: bench.py --shapes", "", "Command (GPU box, from the repository root):",
             "", f"    {cmd}", "", f"Summarised by `python bench.py --activity-summary {root} --steps {args.steps} "
             f"--warmup {args.warmup}` (means over the {args.steps} timed dispatches of each workload; the "
             "dispatches run serialised under counter collection).", "",
             "* clock = GRBM_GUI_ACTIVE / 8 XCDs / dispatch time;",
             "* MFMA util = SQ_VALU_MFMA_BUSY_CYCLES / (GPU cycles x 1024 SIMDs), rocprofv3's MfmaUtil;",
             "* MFMA TFLOP/s = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / dispatch time; counted/alg = those FLOPs over the "
             "algorithmic ones (masked keys inside computed tiles count as work done);",
             "* VALU busy = SQ_ACTIVE_INST_VALU (quad-cycles) / (GPU cycles x 256 CUs), rocprofv3's VALUBusy; "
             "co-issue = SQ_VALU_MFMA_COEXEC_CYCLES / (GPU cycles x 1024 SIMDs);",
             "* LDS util = SQ_LDS_IDX_ACTIVE / (GPU cycles x 256 CUs), rocprofv3's LdsUtil; conflicts = "
             "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE.", "",
             "kernel | workload | us | clock GHz | MFMA util | MFMA TFLOP/s | counted/alg | VALU busy | co-issue "
             "| LDS util | LDS conflict cycles",
             "---|---|---|---|---|---|---|---|---|---|---"]
    for kernel, wl in SHAPES_DISPATCH_ORDER.items():
        ds = [d for d in order if names[d] == kernel]
        for i, name in enumerate(wl):
            run = ds[i * per_run:(i + 1) * per_run][args.warmup:]
            if not run:
                continue

            def mean(c):
                return float(np.mean([vals[d].get(c, 0.0) for d in run]))
            t = float(np.mean([durs[d] for d in run]))
            cyc = mean("GRBM_GUI_ACTIVE") / MI355X_XCDS
            flops = mean("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512
            alg = None
            if "prefill" in kernel:
                import workloads as W
                alg = W.make(name.replace("_alibi", "").replace("_fp8", "").replace("_int8", "")
                         .replace("_precise", "")).attention_flops()
            lds = mean("SQ_LDS_IDX_ACTIVE")
            lines.append(
                f"{kernel.replace('lazyattn::', '')} | {name} | {t * 1e6:.1f} | {cyc / t / 1e9:.3f} | "
                f"{100 * mean('SQ_VALU_MFMA_BUSY_CYCLES') / (cyc * MI355X_SIMDS):.1f} % | {flops / t / 1e12:.1f} | "
                f"{'' if alg is None else f'{flops / alg:.3f}'} | "
                f"{100 * mean('SQ_ACTIVE_INST_VALU') / (cyc * MI355X_CUS):.1f} % | "
                f"{100 * mean('SQ_VALU_MFMA_COEXEC_CYCLES') / (cyc * MI355X_SIMDS):.1f} % | "
                f"{100 * lds / (cyc * MI355X_CUS):.1f} % | "
                f"{100 * mean('SQ_LDS_BANK_CONFLICT') / lds if lds else 0:.1f} %")
    path = os.path.join(PROFILES, "decode_prefill_shapes_activity.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {path}")


def trace_summary_main(args):
    """Write profiles/decode_prefill_llama8b_kernel_trace.md from the rocprofv3
    kernel trace of the default bench step (`bench.py --steps S --warmup W
    --no-cpu-baseline`): per-kernel calls and durations."""
    trace_dir = args.trace_summary
    durs = {}
    rows = sorted(((_kernel_key(n), int(a), int(b)) for n, a, b in
                   _rocpd_rows(trace_dir, "select name, start, end from kernels")), key=lambda r: r[1])
    for key, start, end in rows:
        durs.setdefault(key, []).append((end - start) / 1000.0)
    # the timed steps: the last K prefill dispatches, each with the decode dispatch before it
    pf_key, dec_key = "lazyattn::prefill_kernel<128, 4, 0, false>", "lazyattn::decode_mma16_kernel<4, 0>"
    pf_idx = [i for i, r in enumerate(rows) if r[0] == pf_key][-args.steps:]
    timed_pf = [(rows[i][2] - rows[i][1]) / 1000.0 for i in pf_idx]
    timed_dec = []
    for i in pf_idx:
        j = max(k for k in range(i) if rows[k][0] == dec_key)
        timed_dec.append((rows[j][2] - rows[j][1]) / 1000.0)
    cmd = (f"rocprofv3 --kernel-trace --stats -d {trace_dir} -o run -- python -u bench.py --steps {args.steps} "
           f"--warmup {args.warmup} --no-cpu-baseline")
    lines = ["# rocprofv3 kernel trace: bench.py step (8B decode + 8B prefill)", "",
             "Command (GPU box, from the repository root):", "", f"    {cmd}", "",
             f"Summarised by `python bench.py --trace-summary {trace_dir} --steps {args.steps} --warmup "
             f"{args.warmup}`.  Each step is kvcache_append + lazyattn_decode, then kvcache_append + "
             "lazyattn_prefill.  Torch's fill, copy and random kernels are input generation or the copy roof, "
             "outside the timed step.", "",
             f"The {len(pf_idx)} timed steps (the last {len(pf_idx)} dispatches of `{pf_key}`, each with the "
             f"`{dec_key}` dispatch before it; the bench line's kernel times cover the same dispatches):", "",
             "kernel | calls | avg us | median us", "---|---|---|---",
             f"{dec_key} | {len(timed_dec)} | {np.mean(timed_dec):.1f} | {np.median(timed_dec):.1f}",
             f"{pf_key} | {len(timed_pf)} | {np.mean(timed_pf):.1f} | {np.median(timed_pf):.1f}", "",
             "Every dispatch of the run (the settling steps, warm-up and timed steps, then the other decode "
             "workloads' passes):", "",
             "kernel | calls | avg us | median us | total us | %", "---|---|---|---|---|---"]
    tot = sum(sum(v) for v in durs.values())
    for k, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{k[:90]} | {len(v)} | {np.mean(v):.1f} | {np.median(v):.1f} | {sum(v):.1f} | "
                     f"{100 * sum(v) / tot:.1f}")
    path = os.path.join(PROFILES, "decode_prefill_llama8b_kernel_trace.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {path}")


def cache_sim_main(args):
    """Hit rates of the host pool manager under a KV budget (CPU only, no GPU).

    A Zipf-skewed RAG trace (the recipe of zipf_reuse_decode: a 1000-document
    catalogue of 16*U{16..128} tokens, rank-i probability ~ i^-1.2, U{4..8}
    distinct documents per request in random order, a 64-token prompt) is
    placed request by request and released, for each cache-key policy.  The
    budget is 1 GB of KV in two readings: the whole Llama-3.1-8B model
    (32 layers x 8 KV heads x 128 dims x K,V x bf16 = 128 KiB per token: 512
    blocks) and one layer of it (4 KiB per token: 16384 blocks).  A request
    that does not fit counts as all misses.  One JSON line."""
    from position_agnostic_kv_amd import cache as C

    rng = np.random.default_rng(5)
    catalogue, zipf_s, prompt = 1000, 1.2, 64
    lens = 16 * rng.integers(16, 129, size=catalogue)
    p = 1.0 / np.arange(1, catalogue + 1) ** zipf_s
    p /= p.sum()
    trace = []
    for _ in range(args.cache_requests):
        k = int(rng.integers(4, 9))
        ids = rng.choice(catalogue, size=k, replace=False, p=p)
        trace.append(([int(x) for x in ids], [int(lens[x]) for x in ids]))
    res = {"metric": "document-token hit rate of the KV pool manager", "unit": "fraction",
           "requests": len(trace), "data": "synthetic Zipf trace",
           "trace": "1000 docs of 16*U{16..128} tokens, p(rank i) ~ i^-1.2, U{4..8} docs/request, 64-token prompt"}
    for label, blocks in (("1GB_whole_8B_model_512_blocks", 512), ("1GB_one_8B_layer_16384_blocks", 16384)):
        row = {}
        for mode in ("agnostic", "aware", "prefix"):
            m = C.CacheManager(blocks, mode)
            hit = total = unplaced = 0
            t0 = time.perf_counter()
            for ids, ls in trace:
                total += sum(ls)
                try:
                    _, miss, rid = m.acquire(ids, ls, prompt)
                except C.CacheError:
                    unplaced += 1
                    continue
                hit += sum(L for L, x in zip(ls, miss) if not x)
                m.release(rid)
            row[mode] = {"hit_rate": round(hit / total, 4), "unplaced_requests": unplaced,
                         "evicted": m.stats()["evicted"],
                         "us_per_request": round((time.perf_counter() - t0) / len(trace) * 1e6, 2)}
        row["agnostic_over_aware"] = round(row["agnostic"]["hit_rate"] / max(row["aware"]["hit_rate"], 1e-9), 2)
        row["agnostic_over_prefix"] = round(row["agnostic"]["hit_rate"] / max(row["prefix"]["hit_rate"], 1e-9), 2)
        res[label] = row
    print(json.dumps(res), flush=True)


def decode_workload_line(name, args, dev):
    """The default step's decode pass (kvcache_append of the new tokens, then
    lazyattn_decode) on another decode workload of the same metric, timed the
    same way (W warm-up passes, then K timed ones, HIP events on the launch
    stream): its own K+V rate, kernel-time percentiles, roofline and oracle
    baseline.  On the Zipf mix the record is the planned decode's
    (lazyattn_decode_planned: the readers of each shared document run
    together), with the per-sequence decode's figures beside it.  Inputs are
    dropped afterwards."""
    import torch
    import position_agnostic_kv_amd as pak
    import workloads as W
    from workloads.device import DeviceInputs

    case = W.make(name)
    W.materialize_torch(case, dev)
    d = DeviceInputs(case, dev)
    wsb = pak.decode_workspace_size(case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim,
                                    case.layout.table.shape[1], args.split_blocks)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(d.q)

    def one(ev=None):
        if ev is not None:
            ev[0].record()
        pak.kvcache_append(d.k_pool, d.v_pool, d.k_new, d.v_new, d.slots)
        if ev is not None:
            ev[1].record()
        pak.lazyattn_decode(d.q, d.q_pos, d.k_pool, d.v_pool, d.table, d.seq_lens, scale=case.scale,
                            rope_theta=case.rope_theta, split_blocks=args.split_blocks, out=out, workspace=ws)
        if ev is not None:
            ev[2].record()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for k in range(args.steps):
            fn(events[k])
        torch.cuda.synchronize()
        return (float(np.mean([e[0].elapsed_time(e[2]) for e in events])),
                np.array([e[1].elapsed_time(e[2]) for e in events]))

    pass_ms, kx = timed(one)
    kernel_ms = float(np.mean(kx))
    kv, alg = decode_algorithmic_bytes(case)
    g = case.num_q_heads // case.num_kv_heads
    kname = f"lazyattn::decode_mma16_kernel<{min(g, 16)}, 0>"
    stem = {"llama70b_decode": "decode_llama70b", "zipf_reuse_decode": "decode_zipf"}[name]
    per_seq = None
    if name == "zipf_reuse_decode":
        # shared documents: the planned decode (the host plan is built once,
        # outside the timing, as a scheduler builds the block table)
        per_seq = {"path": "lazyattn_decode", "decode_pass_ms": round(pass_ms, 4),
                   "decode_kernel_ms": round(kernel_ms, 4),
                   "value": round(kv / (pass_ms * 1e-3) / 1e9, 2),
                   "traffic": measured_traffic(stem, DECODE_SOURCES)}
        t0 = time.perf_counter()
        plan = pak.decode_plan(d.table, d.seq_lens, case.num_q_heads, case.num_kv_heads)
        plan_ms = (time.perf_counter() - t0) * 1e3
        pws = torch.empty(max(pak.decode_planned_workspace_size(case.batch, case.num_q_heads, case.num_kv_heads,
                                                                case.head_dim, plan.max_items_per_seq), 1),
                          dtype=torch.uint8, device=dev)

        def planned(ev=None):
            if ev is not None:
                ev[0].record()
            pak.kvcache_append(d.k_pool, d.v_pool, d.k_new, d.v_new, d.slots)
            if ev is not None:
                ev[1].record()
            pak.lazyattn_decode_planned(d.q, d.q_pos, d.k_pool, d.v_pool, d.table, d.seq_lens, plan,
                                        scale=case.scale, rope_theta=case.rope_theta, out=out, workspace=pws)
            if ev is not None:
                ev[2].record()

        pass_ms, kx = timed(planned)
        kernel_ms = float(np.mean(kx))
        stem = "decode_zipf_planned"
        kname = f"lazyattn::decode_planned_kernel<{g}>"
    rec = {
        "value": round(kv / (pass_ms * 1e-3) / 1e9, 2), "unit": "GB/s",
        "config": {"batch": case.batch, "q_heads": case.num_q_heads, "kv_heads": case.num_kv_heads,
                   "head_dim": case.head_dim, "tokens_attended": int(case.layout.total_lens.sum()),
                   "kv_bytes": kv},
        "decode_pass_ms": round(pass_ms, 4), "decode_kernel_ms": round(kernel_ms, 4),
        "decode_kernel_ms_pct": {"p10": round(float(np.percentile(kx, 10)), 4),
                                 "p50": round(float(np.median(kx)), 4),
                                 "p90": round(float(np.percentile(kx, 90)), 4)},
        "roofline": {"kernel": kname, "bound": "hbm", "achieved": round(alg / (kernel_ms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(alg / (kernel_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(stem, DECODE_SOURCES), "algorithmic_bytes": alg},
    }
    if name == "zipf_reuse_decode":
        phys = int(d.k_pool.numel()) * 2 * 2
        rec["path"] = "lazyattn_decode_planned"
        rec["plan"] = {"items": plan.num_items, "max_items_per_seq": plan.max_items_per_seq,
                       "host_build_ms": round(plan_ms, 2),
                       "note": "built on the host from the block table and lengths, outside the timing; valid "
                               "while sequences grow into blocks appended to their rows"}
        rec["roofline"]["note"] = ("algorithmic bytes count every attended token once per sequence; the plan "
                                   "runs the readers of each shared document together so the L2 serves the "
                                   "repeats, so the logical rate exceeds the HBM peak")
        rec["pool_bytes_physical"] = phys
        rec["physical_pool_gbps"] = round(phys / (kernel_ms * 1e-3) / 1e9, 1)
        rec["per_sequence_decode"] = per_seq
    if not args.no_cpu_baseline:
        rec["cpu_baseline"], rec["parity_sample"] = cpu_baseline_decode(case, d, args.cpu_seconds, out)
    del d, out, ws
    case.q = case.k_pool = case.v_pool = case.k_new = case.v_new = None
    torch.cuda.empty_cache()
    return rec


def clock_settle(step, chunk=10, min_steps=40, max_steps=400, tol=0.005):
    """Untimed steps, before the counted warm-up, until the clock has settled.

    From idle (and again after as little as 0.2 s without work) MI355X takes
    about 30-40 steps of this workload (40-50 ms) to reach its steady clock: in
    that stretch the prefill kernel, which is power-limited, runs up to 25 %
    slower, while the memory-bound decode kernel does not change.  Steps run
    in chunks of `chunk` until the chunk mean of the prefill kernel's time
    moves by less than `tol` (at least `min_steps`, at most `max_steps`).
    Returns the step count and the chunk means, so the cold figures stay in
    the record."""
    import torch

    means, done = [], 0
    while done < max_steps:
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(chunk)]
        for e in ev:
            step(e)
        torch.cuda.synchronize()
        means.append(float(np.mean([e[3].elapsed_time(e[4]) for e in ev])))
        done += chunk
        if done >= min_steps and abs(means[-1] - means[-2]) <= tol * means[-2]:
            break
    return {"steps": done, "prefill_kernel_ms_per_10_steps": [round(m, 4) for m in means],
            "note": "untimed steps before the counted warm-up, run until the prefill kernel's time "
                    "stops changing (the GPU's clock ramps up from idle); --no-settle skips them"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--split-blocks", type=int, default=0)
    ap.add_argument("--no-settle", action="store_true",
                    help="skip the untimed steps that bring the clock to its steady state before the warm-up")
    ap.add_argument("--overhead", action="store_true",
                    help="time the lazy kernels against the non-lazy baseline instead (one JSON line)")
    ap.add_argument("--shapes", action="store_true",
                    help="time every decode workload and the prefill separately instead (one JSON line)")
    ap.add_argument("--cache-sim", action="store_true",
                    help="hit rates of the host pool manager on a Zipf trace (CPU only; one JSON line)")
    ap.add_argument("--cache-requests", type=int, default=5000)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for rocprofv3 counter scaling)")
    ap.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "TRACE_DIR"),
                    help="summarise rocprofv3 output of --shapes runs into profiles/ (no GPU)")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR",
                    help="summarise the rocprofv3 kernel trace of a default bench run into profiles/ (no GPU)")
    ap.add_argument("--activity-summary", metavar="PMC_DIR",
                    help="summarise a rocprofv3 --pmc run of --shapes with the activity counters (no GPU)")
    args = ap.parse_args()

    if args.activity_summary:
        activity_summary_main(args)
        return
    if args.trace_summary:
        trace_summary_main(args)
        return
    if args.pmc_summary:
        pmc_summary_main(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    if args.overhead:
        overhead_main(args)
        return
    if args.shapes:
        shapes_main(args)
        return
    if args.cache_sim:
        cache_sim_main(args)
        return

    import torch
    import position_agnostic_kv_amd as pak
    import workloads as W
    from workloads.device import DeviceInputs

    pak.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    dcase = W.llama8b_decode()
    pcase = W.llama8b_prefill()
    W.materialize_torch(dcase, dev)
    W.materialize_torch(pcase, dev)
    dd = DeviceInputs(dcase, dev)
    pd = DeviceInputs(pcase, dev)
    ws_bytes = pak.decode_workspace_size(dcase.batch, dcase.num_q_heads, dcase.num_kv_heads,
                                         dcase.head_dim, dcase.layout.table.shape[1], args.split_blocks)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    dout = torch.empty_like(dd.q)
    pout = torch.empty_like(pd.q)

    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.int16, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        pak.kvcache_append(dd.k_pool, dd.v_pool, dd.k_new, dd.v_new, dd.slots)
        if ev is not None:
            ev[1].record()
        pak.lazyattn_decode(dd.q, dd.q_pos, dd.k_pool, dd.v_pool, dd.table, dd.seq_lens,
                            scale=dcase.scale, rope_theta=dcase.rope_theta,
                            split_blocks=args.split_blocks, out=dout, workspace=ws)
        if ev is not None:
            ev[2].record()
        pak.kvcache_append(pd.k_pool, pd.v_pool, pd.k_new, pd.v_new, pd.slots)
        if ev is not None:
            ev[3].record()
        pak.lazyattn_prefill(pd.q, pd.cu, pd.q_pos_start, pd.k_pool, pd.v_pool, pd.table, pd.seq_lens,
                             pcase.max_q_len, scale=pcase.scale, rope_theta=pcase.rope_theta, out=pout)
        if ev is not None:
            ev[4].record()

    settle = None if args.no_settle else clock_settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def mean_ms(i, j):
        return float(np.mean([e[i].elapsed_time(e[j]) for e in events]))

    def pct_ms(i, j):
        x = np.array([e[i].elapsed_time(e[j]) for e in events])
        return {"p10": round(float(np.percentile(x, 10)), 4), "p50": round(float(np.median(x)), 4),
                "p90": round(float(np.percentile(x, 90)), 4)}

    # measured copy roof (outside the timed region): a plain 2 GiB device copy
    # (torch's copy kernel), bytes read + written per second
    csrc = torch.empty(1 << 30, dtype=torch.int16, device=dev).fill_(1)
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    cev = [torch.cuda.Event(enable_timing=True) for _ in range(11)]
    cev[0].record()
    for i in range(10):
        cdst.copy_(csrc)
        cev[i + 1].record()
    torch.cuda.synchronize()
    copy_ms = float(np.median([cev[i].elapsed_time(cev[i + 1]) for i in range(10)]))
    copy_gbps = 2 * csrc.numel() * 2 / (copy_ms * 1e-3) / 1e9
    del csrc, cdst

    decode_pass_ms = mean_ms(0, 2)
    decode_kernel_ms = mean_ms(1, 2)
    prefill_kernel_ms = mean_ms(3, 4)
    prefill_pass_ms = mean_ms(2, 4)
    step_ms = mean_ms(0, 4)

    kv_bytes, dec_alg_bytes = decode_algorithmic_bytes(dcase)
    value = kv_bytes / (decode_pass_ms * 1e-3) / 1e9
    dec_achieved = dec_alg_bytes / (decode_kernel_ms * 1e-3) / 1e9
    flops = pcase.attention_flops()
    pf_tflops = flops / (prefill_kernel_ms * 1e-3) / 1e12

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llama8b_decode + llama8b_prefill",
            "decode": {"batch": dcase.batch, "tokens_per_seq": int(dcase.seq_lens[0]), "q_heads": 32,
                       "kv_heads": 8, "head_dim": 128, "kv_bytes": kv_bytes, "docs_tokens": "256..2048"},
            "prefill": {"batch": pcase.batch, "cached_tokens": 6144, "prompt_tokens": 2048, "q_heads": 32,
                        "kv_heads": 8, "head_dim": 128, "attention_flops": flops, "q_tile": 128},
        },
        "decode_pass_ms": round(decode_pass_ms, 4),
        "decode_kernel_ms": round(decode_kernel_ms, 4),
        "prefill_pass_ms": round(prefill_pass_ms, 4),
        "prefill_kernel_ms": round(prefill_kernel_ms, 4),
        "prefill_tflops": round(pf_tflops, 2),
        "decode_kernel_ms_pct": pct_ms(1, 2),
        "prefill_kernel_ms_pct": pct_ms(3, 4),
        "copy_roof": {"gbps": round(copy_gbps, 1), "bytes_moved": 2 * (1 << 31),
                      "note": "context only: torch's 2 GiB device-to-device copy, bytes read + written "
                              "per second, median of 10 (a read+write stream, not the read-only "
                              "pattern of decode)"},
        "wall_s_timed": round(wall, 3),
        "clock_settle": settle,
        "roofline": {
            "kernel": "lazyattn::decode_mma16_kernel<4, 0>",
            "bound": "hbm",
            "achieved": round(dec_achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(dec_achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic("decode_llama8b", DECODE_SOURCES),
            "algorithmic_bytes": dec_alg_bytes,
        },
        "roofline_prefill": {
            "kernel": "lazyattn::prefill_kernel<128, 4, 0, false>",
            "bound": "mfma",
            "achieved": round(pf_tflops, 2),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(pf_tflops / BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic("prefill_llama8b", PREFILL_SOURCES),
            "algorithmic_flops": flops,
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"], res["parity_sample"] = cpu_baseline_decode(dcase, dd, args.cpu_seconds, dout)
        res["cpu_baseline_prefill"], res["parity_sample_prefill"] = cpu_baseline_prefill(
            pcase, pd, args.cpu_seconds, pout)
    # the metric's other decode workloads, each timed as its own pass after the steps above
    del dd, pd, ws, dout, pout
    dcase.q = dcase.k_pool = dcase.v_pool = dcase.k_new = dcase.v_new = None
    pcase.q = pcase.k_pool = pcase.v_pool = pcase.k_new = pcase.v_new = None
    torch.cuda.empty_cache()
    for name in ("llama70b_decode", "zipf_reuse_decode"):
        res[name] = decode_workload_line(name, args, dev)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
