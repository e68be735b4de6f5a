"""Benchmark of the exact paged attention path on one MI355X.

One step is one pass of the whole path over one batch of the mixed long-context workload
(120 decode requests with contexts in [4096, 32768] plus 8 prefill requests of 2048 query
tokens, 64 q / 8 kv heads, head_size 128, bf16, block_size 64, a 2048-token prefix shared by
all requests), through both of its layer passes (pass 0 causal, pass 1 causal with a
4096-token sliding window), each with its own q and KV cache. Per pass the batch is sent to
the library as its decode rows (split-KV kernel + LSE merge) and its prefill rows (prefill
kernel), on one stream, with HIP events between the calls so that the kernels' durations are
measured inside the timed region.

Prints one JSON line. ``value`` is the fraction of the MI355X roofline reached by the whole
step, in percent: (prefill flops / 2.5 PFLOP/s + decode bytes / 8 TB/s) / step time, where
flops and bytes are algorithmic (visible (query, key) pairs only; K/V bytes each request must
read, the shared prefix counted once per layer). ``roofline`` describes the dominant kernel
(prefill, bf16 MFMA). ``cpu_baseline`` times the CPU oracle on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_FLOPS = 2.5e15     # MI355X dense bf16 MFMA
PEAK_HBM_BYTES = 8.0e12      # MI355X HBM3E
METRIC = "prefill attn TFLOP/s + decode KV GB/s at 1 MI355X, % of roofline"


def algorithmic_work(batch, causal, window):
    """(prefill flops, decode unique bytes, decode logical bytes) of one layer pass.

    Prefill flops: 4 * head_size per visible (query, key) pair and q head. Decode bytes: the
    K and V rows of every visible key of every kv head, plus q, out, lse and the block-table
    entries of the visible blocks. 'logical' counts each request's keys; 'unique' counts the
    shared-prefix keys once (the prefix is the same physical blocks for every request)."""
    import oracle  # only for the visible-pair count of the definition
    nd = batch.num_decodes
    d, hq, hkv = batch.head_size, batch.num_heads, batch.num_kv_heads
    pairs = oracle.flops_visible_pairs(batch.query_lens[nd:], batch.seq_lens[nd:], causal, window)
    prefill_flops = 4.0 * d * hq * pairs
    row = 2 * hkv * d * 2                                   # K + V bytes of one token
    S = batch.shared_prefix_blocks * batch.block_size
    shared_seen = np.zeros(S, dtype=bool)
    logical_tok = private_tok = bt_entries = 0
    for r in range(nd):
        sl = int(batch.seq_lens[r])
        lo = max(0, sl - window) if window > 0 else 0
        logical_tok += sl - lo
        private_tok += sl - max(lo, S)
        if lo < S:
            shared_seen[lo:min(sl, S)] = True
        bt_entries += -(-sl // batch.block_size) - lo // batch.block_size
    extra = nd * (hq * d * 2 * 2 + hq * 4) + bt_entries * 4   # q + out (bf16), lse, table
    unique = (private_tok + int(shared_seen.sum())) * row + extra
    logical = logical_tok * row + extra
    return prefill_flops, unique, logical


CPU_DECODE_STEP = 2      # every 2nd decode request ...
CPU_PREFILL_ROWS = 20    # ... and 20 query rows of each prefill request: 10-15 s of oracle


def cpu_baseline(batch, layers, seed):
    """Time the oracle on a bounded sample: every CPU_DECODE_STEP-th decode request and
    CPU_PREFILL_ROWS evenly spaced query rows of each prefill request, for every layer pass;
    scale to the metric's unit (percent of the MI355X roofline the CPU reaches on that
    sample)."""
    import torch
    import gen
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    cpu_model = host_cpu_model()
    nd = batch.num_decodes
    dec = list(range(0, nd, CPU_DECODE_STEP))
    pre = list(range(nd, batch.num_seqs))
    floor_s = 0.0
    cpu_s = 0.0
    for li, (q, kv) in enumerate(layers):
        causal, window = batch.passes[li]
        sub, qs, kvs = gen.subset(batch, dec + pre, q, kv)
        qsl = sub.query_start_loc
        rows = list(range(len(dec)))
        for i in range(len(dec), sub.num_seqs):
            ql = int(sub.query_lens[i])
            rows += [int(qsl[i]) + x for x in np.linspace(0, ql - 1, CPU_PREFILL_ROWS).astype(int)]
        qn = qs.to(torch.float32).numpy()
        kvn = kvs.to(torch.float32).numpy()
        t0 = time.perf_counter()
        oracle.attention(qn, kvn, sub.block_table, qsl, sub.seq_lens, sub.scale, causal, window,
                         rows=rows)
        cpu_s += time.perf_counter() - t0
        # roofline floor of the sampled work on the GPU
        d, hq = sub.head_size, sub.num_heads
        flops = 0.0
        for i in range(len(dec), sub.num_seqs):
            ql, sl = int(sub.query_lens[i]), int(sub.seq_lens[i])
            pos = (sl - ql) + np.linspace(0, ql - 1, CPU_PREFILL_ROWS).astype(int)
            lo = np.maximum(pos - window + 1, 0) if window > 0 else 0
            flops += 4.0 * d * hq * float(np.sum(pos + 1 - lo))
        byts = 0.0
        for i in range(len(dec)):
            sl = int(sub.seq_lens[i])
            lo = max(0, sl - window) if window > 0 else 0
            byts += (sl - lo) * 2 * sub.num_kv_heads * d * 2
        floor_s += flops / PEAK_BF16_FLOPS + byts / PEAK_HBM_BYTES
    return {"value": 100.0 * floor_s / cpu_s, "unit": "% of MI355X roofline", "cores": threads,
            "kind": "oracle", "seconds": round(cpu_s, 3), "cpu_model": cpu_model,
            "host_logical_cpus": os.cpu_count(),
            "threads_note": "cores = the BLAS thread pool the fp64 matrix products ran on (the "
                            "rest of the oracle is single-threaded numpy)",
            "sample": f"fp64 numpy oracle; per layer pass: decode requests {dec[0]}..{dec[-1]} "
                      f"step {CPU_DECODE_STEP} ({len(dec)} of {nd}) and {CPU_PREFILL_ROWS} evenly "
                      f"spaced query rows of each of the {len(pre)} prefill requests, all "
                      f"{batch.num_heads} q heads; value = GPU-roofline time of that work / CPU "
                      f"time"}


def host_cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (the box the oracle runs on)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mixed_pass_traffic.json")
# the dominant kernel (one launch of a mixed layer pass) is built from these sources
KERNEL_SRCS = [os.path.join(ROOT, "exact_softmax_attention_paged_amd", "csrc", f)
               for f in ("prefill_bf16.hip", "decode_core.hpp")]
DOMINANT_KERNEL = "mixed_bf16_kernel<128, true, false>"
COPY_BYTES = 1 << 30


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def pmc_probe(dev):
    """Workload for the traffic counters: three plain 1 GiB device copies (the calibration
    kernel of known size), then one bench step. Run under rocprofv3 --pmc FETCH_SIZE, then
    --pmc WRITE_SIZE."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def record_traffic(fetch_csv, write_csv, command):
    """Turn two rocprofv3 counter_collection.csv files into profiles/mixed_pass_traffic.json:
    per-dispatch FETCH_SIZE and WRITE_SIZE (KiB) of the attention kernels, scaled by the bytes
    the same counters report for the plain 1 GiB copy."""
    import csv
    import re

    def per_kernel(path, counter):
        acc = {}
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            acc.setdefault(name, []).append(float(row["Counter_Value"]))
        return acc

    out = {"source_sha256_16": kernel_source_hash(), "command": command}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        acc = per_kernel(path, counter)
        # the calibration copies are the runtime's device-to-device copy kernel
        copy = sorted(v for n, vals in acc.items() if "rocclr_copyBuffer" in n for v in vals)
        pre = {re.sub(r"\(attn::.*$", "", n.replace("void ", "").replace(
            "attn::(anonymous namespace)::", "")): vals for n, vals in acc.items()
            if "attn::" in n}
        copy_kib = copy[len(copy) // 2]
        expected_kib = COPY_BYTES / 1024.0
        factor = expected_kib / copy_kib
        out[counter] = {"copy_kib_per_dispatch": copy_kib, "copy_expected_kib": expected_kib,
                        "scale": factor,
                        "kib_per_dispatch": {k: sum(v) / len(v) for k, v in pre.items()}}
    # per launch of the dominant kernel (the one launch of layer pass 0, causal)
    f_kib = out["FETCH_SIZE"]["kib_per_dispatch"]
    w_kib = out["WRITE_SIZE"]["kib_per_dispatch"]
    key = DOMINANT_KERNEL
    out["kernel"] = key
    out["traffic_bytes_per_launch"] = (f_kib[key] * out["FETCH_SIZE"]["scale"] +
                                       w_kib[key] * out["WRITE_SIZE"]["scale"]) * 1024.0
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    json.dump(out, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(out, indent=1))


def recorded_traffic():
    """HBM bytes per launch of the dominant kernel from profiles/mixed_pass_traffic.json, or
    None when the record is missing or was taken on a different kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def _time_ms(fn, reps, warmup=3):
    """Mean duration of fn() over reps calls, by HIP events on torch's current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def cascade_report(dev, seed):
    """Cascade attention (attn_cascade_fwd) against the plain call on batches whose requests
    share a prefix: decode batches with long shared prefixes, and layer pass 0 of the mixed
    long-context workload. One JSON line per batch: both times, the speedup, the K/V bytes a
    per-request read would touch ('logical') and the largest output difference."""
    import torch
    import exact_softmax_attention_paged_amd as A
    import gen
    rng = np.random.default_rng(seed)
    cases = []
    for nd, pre, lo, hi in ((120, 2048, 4096, 32768), (256, 4096, 4224, 6144),
                            (256, 8192, 8448, 12288), (64, 16384, 16896, 20480)):
        sl = rng.integers(lo, hi, size=nd, endpoint=True)
        b = gen.make_batch(f"{nd} decodes, ctx U[{lo},{hi}], {pre}-token shared prefix",
                           num_heads=64, num_kv_heads=8, head_size=128, block_size=64,
                           dtype="bf16", query_lens=[1] * nd, seq_lens=sl, passes=[(True, 0)],
                           seed=seed, shared_prefix_blocks=pre // 64)
        cases.append(b)
    cases.append(gen.config(5, seed=seed))
    for b in cases:
        q, kv = gen.make_tensors(b, seed, dev)
        bt, qsl, sl = (torch.from_numpy(x).to(dev) for x in (b.block_table, b.query_start_loc,
                                                             b.seq_lens))
        P = b.shared_prefix_blocks * b.block_size
        desc = A.make_desc(num_seqs=b.num_seqs, num_tokens=b.num_tokens,
                           num_decodes=b.num_decodes, max_query_len=b.max_query_len,
                           max_seq_len=b.max_seq_len, num_heads=b.num_heads,
                           num_kv_heads=b.num_kv_heads, head_size=b.head_size,
                           num_blocks=b.num_blocks, block_size=b.block_size,
                           max_blocks_per_seq=b.max_blocks_per_seq, dtype=A.ATTN_BF16)
        out = torch.empty_like(q)
        lse = torch.empty(b.num_tokens, b.num_heads, dtype=torch.float32, device=dev)
        wsp = torch.empty(max(A.attn_workspace_bytes(desc), 1), dtype=torch.uint8, device=dev)
        wsc = torch.empty(A.attn_cascade_workspace_bytes(desc, P), dtype=torch.uint8, device=dev)
        causal = b.passes[0][0]
        reps = 5 if b.num_tokens > 1000 else 20
        tp = _time_ms(lambda: A.attn_varlen_fwd(desc, q, kv, bt, qsl, sl, b.scale, causal, 0,
                                                out, lse, wsp), reps)
        ref = out.clone()
        tc = _time_ms(lambda: A.attn_cascade_fwd(desc, q, kv, bt, qsl, sl, P, b.scale, causal,
                                                 out, lse, wsc), reps)
        diff = (out.float() - ref.float()).abs().max().item()
        logical = int(b.seq_lens[:b.num_decodes].astype(np.int64).sum()) * 2 * b.num_kv_heads * \
            b.head_size * 2
        print(json.dumps({"report": "cascade", "batch": b.name, "common_prefix_len": P,
                          "plain_ms": round(tp, 4), "cascade_ms": round(tc, 4),
                          "speedup": round(tp / tc, 3), "decode_kv_gb_logical": logical / 1e9,
                          "max_abs_diff_vs_plain": diff}), flush=True)


def kv_write_report(dev, seed):
    """KV-cache write (attn_kv_cache_write) throughput. Algorithmic bytes per token: its K and
    V rows read once and written once (4 * num_kv_heads * head_size * 2 bytes in bf16) plus
    its 8-byte slot. One JSON line per shape, against the 8 TB/s HBM roofline."""
    import torch
    import exact_softmax_attention_paged_amd as A
    import gen
    b = gen.config(5, seed=seed)
    hkv, d, bs, nb = b.num_kv_heads, b.head_size, b.block_size, b.num_blocks
    cache = torch.zeros((2, nb, bs, hkv, d), dtype=torch.bfloat16, device=dev)
    rng = np.random.default_rng(seed)
    for T, what in ((b.num_tokens, "the mixed workload's 16504 new tokens"),
                    (262144, "262144 new tokens")):
        slots = torch.from_numpy(rng.permutation(nb * bs)[:T].astype(np.int64)).to(dev)
        key = torch.randn(T, hkv, d, device=dev).to(torch.bfloat16)
        val = torch.randn(T, hkv, d, device=dev).to(torch.bfloat16)
        desc = A.make_desc(num_seqs=1, num_tokens=T, num_decodes=0, max_query_len=1,
                           max_seq_len=bs, num_heads=hkv, num_kv_heads=hkv, head_size=d,
                           num_blocks=nb, block_size=bs, max_blocks_per_seq=1,
                           dtype=A.ATTN_BF16)
        ms = _time_ms(lambda: A.attn_kv_cache_write(desc, key, val, slots, cache), 50)
        byts = T * (4 * hkv * d * 2 + 8)
        print(json.dumps({"report": "kv-write", "shape": f"{what}, {hkv} kv heads, d {d}, "
                          f"bf16, block 64, {nb} blocks", "tokens": T, "ms": round(ms, 5),
                          "bytes": byts, "gbps": round(byts / (ms / 1e3) / 1e9, 1),
                          "frac_of_8tbps": round(byts / (ms / 1e3) / PEAK_HBM_BYTES, 4)}),
              flush=True)


def fp8_decode_report(dev, seed):
    """Decode over an E4M3 cache (attn_fp8_decode_fwd) against the bf16 cache
    (attn_varlen_fwd) on the paged GQA decode workload (256 requests, contexts U[512, 8192],
    32 q / 8 kv heads, d 128, block 16) and on the mixed workload's 120 decode requests
    (pass 0), with the library's default partition (partition_tokens 0: the batch-adapted
    length for bf16, capped at 1024 keys for E4M3) and 512, 1024, 2048, 4096 and 8192 keys. Algorithmic bytes: each request's visible K and V once (2 bytes per element in
    bf16, 1 in E4M3) plus q, out, lse and the block-table entries. One JSON line per
    workload, cache type and partition length."""
    import torch
    import exact_softmax_attention_paged_amd as A
    import gen
    for k in (4, 5):
        b = gen.config(k, seed=seed)
        nd = b.num_decodes
        if nd != b.num_seqs:          # the decode requests only
            b = gen.subset_meta(b, list(range(nd)))
        q = gen.make_q(b, seed, dev)
        kv = gen.make_kv(b, seed, dev)
        rng = np.random.default_rng(seed)
        codes = torch.from_numpy(rng.integers(0, 256, size=tuple(kv.shape), dtype=np.uint8))
        codes[(codes & 0x7F) == 0x7F] = 0
        codes = codes.to(dev)
        bt, qsl, sl = (torch.from_numpy(x).to(dev) for x in (b.block_table, b.query_start_loc,
                                                             b.seq_lens))
        out = torch.empty_like(q)
        lse = torch.empty(b.num_tokens, b.num_heads, dtype=torch.float32, device=dev)
        keys = int(b.seq_lens.astype(np.int64).sum())
        extra = nd * (b.num_heads * b.head_size * 2 * 2 + b.num_heads * 4) + \
            int(sum(-(-int(x) // b.block_size) for x in b.seq_lens)) * 4
        runs = []
        descs = {pt: A.make_desc(num_seqs=b.num_seqs, num_tokens=b.num_tokens, num_decodes=nd,
                                 max_query_len=1, max_seq_len=b.max_seq_len,
                                 num_heads=b.num_heads, num_kv_heads=b.num_kv_heads,
                                 head_size=b.head_size, num_blocks=b.num_blocks,
                                 block_size=b.block_size,
                                 max_blocks_per_seq=b.max_blocks_per_seq, dtype=A.ATTN_BF16,
                                 partition_tokens=pt)
                 for pt in (0, 512, 1024, 2048, 4096, 8192)}
        # one workspace large enough for the shortest partitions (the most partials)
        ws = torch.empty(max(max(A.attn_workspace_bytes(dd),
                                 A.attn_fp8_decode_workspace_bytes(dd)) for dd in descs.values()),
                         dtype=torch.uint8, device=dev)
        for pt, d_pt in descs.items():
            used = A.attn_decode_partition_tokens(d_pt)
            runs.append(("bf16", pt, used, 2, lambda d_pt=d_pt: A.attn_varlen_fwd(
                d_pt, q, kv, bt, qsl, sl, b.scale, True, 0, out, lse, ws)))
            # the E4M3 default caps the partition at 1024 keys
            runs.append(("e4m3", pt, min(used, 1024) if pt == 0 else used,
                         1, lambda d_pt=d_pt: A.attn_fp8_decode_fwd(
                             d_pt, q, codes, bt, qsl, sl, b.scale, 0.0125, 0.02, 0, out, lse,
                             ws)))
        for name, pt, used, elem, fn in runs:
            ms = _time_ms(fn, 20)
            byts = keys * 2 * b.num_kv_heads * b.head_size * elem + extra
            print(json.dumps({"report": "fp8-decode", "workload": gen.CONFIG_NAMES[k] +
                              (" (its 120 decode requests)" if k == 5 else ""), "cache": name,
                              "partition_tokens": pt, "partition_tokens_used": used,
                              "ms": round(ms, 4), "bytes": byts,
                              "gbps": round(byts / (ms / 1e3) / 1e9, 1),
                              "frac_of_8tbps": round(byts / (ms / 1e3) / PEAK_HBM_BYTES, 4),
                              "tokens_per_s": round(keys / (ms / 1e3), 1)}), flush=True)


def schedule_report(dev, seed):
    """Prefill calls with the device-built work schedule (attn_varlen_fwd_scheduled) against
    the plain grid (attn_varlen_fwd), on the prefill workloads and on a skewed varlen batch.
    The schedule is built once per batch and mask (outside the timed calls, as it would be
    reused by every layer); its build time is reported separately."""
    import torch
    import exact_softmax_attention_paged_amd as A
    import gen
    rng = np.random.default_rng(seed)
    cases = []
    for k in (2, 3):
        b = gen.config(k)
        cases.append((gen.CONFIG_NAMES[k], b, b.passes[0], k))
    b5 = gen.config(5, seed=seed)
    b5p = gen.subset_meta(b5, list(range(b5.num_decodes, b5.num_seqs)))
    for li, pas in enumerate(b5.passes):
        cases.append((f"mixed-long-context prefill requests, pass {li}", b5p, pas, 5))
    sl = rng.integers(64, 8192, size=24, endpoint=True)
    bsk = gen.make_batch("skewed", num_heads=32, num_kv_heads=8, head_size=128, block_size=16,
                         dtype="bf16", query_lens=sl, seq_lens=sl, passes=[(True, 0)],
                         seed=seed)
    cases.append(("skewed varlen causal: 24 requests, ql = sl ~ U[64, 8192], 32q/8kv, d128",
                  bsk, (True, 0), seed))
    for name, b, (causal, window), s in cases:
        q = gen.make_q(b, s, dev)
        kv = gen.make_kv(b, s, dev)
        bt, qsl, sl_d = (torch.from_numpy(x).to(dev) for x in (b.block_table,
                                                               b.query_start_loc, b.seq_lens))
        desc = A.make_desc(num_seqs=b.num_seqs, num_tokens=b.num_tokens,
                           num_decodes=b.num_decodes, max_query_len=b.max_query_len,
                           max_seq_len=b.max_seq_len, num_heads=b.num_heads,
                           num_kv_heads=b.num_kv_heads, head_size=b.head_size,
                           num_blocks=b.num_blocks, block_size=b.block_size,
                           max_blocks_per_seq=b.max_blocks_per_seq, dtype=A.ATTN_BF16)
        out = torch.empty_like(q)
        lse = torch.empty(b.num_tokens, b.num_heads, dtype=torch.float32, device=dev)
        sched = torch.empty(A.attn_schedule_bytes(desc) // 4, dtype=torch.int32, device=dev)
        reps = 5 if b.num_tokens > 10000 else 50
        t_build = _time_ms(lambda: A.attn_build_schedule(desc, qsl, sl_d, causal, window, sched),
                           reps)
        tp = _time_ms(lambda: A.attn_varlen_fwd(desc, q, kv, bt, qsl, sl_d, b.scale, causal,
                                                window, out, lse, None), reps)
        ts = _time_ms(lambda: A.attn_varlen_fwd_scheduled(desc, q, kv, bt, qsl, sl_d, b.scale,
                                                          causal, window, out, lse, None, sched),
                      reps)
        import oracle  # visible-pair count of the definition, for the flop rate
        f = 4.0 * b.head_size * b.num_heads * oracle.flops_visible_pairs(
            b.query_lens, b.seq_lens, causal, window)
        print(json.dumps({"report": "schedule", "batch": name, "causal": causal,
                          "window": window, "plain_ms": round(tp, 4),
                          "scheduled_ms": round(ts, 4), "speedup": round(tp / ts, 3),
                          "schedule_build_ms": round(t_build, 4),
                          "plain_tflops": round(f / (tp / 1e3) / 1e12, 1),
                          "scheduled_tflops": round(f / (ts / 1e3) / 1e12, 1)}), flush=True)


COLD_ROTATION_BYTES = 512 << 20


def configs_report(dev, seed):
    """Every workload (the tiny fp32 case, the BERT-large-shaped encoder, the GPT-2-shaped
    varlen prefill, the paged GQA decode, the mixed long-context batch) through one plain
    attn_varlen_fwd call per layer pass, with the library's default decode partition, and the
    paged GQA decode again at its stated 512-token partitions (each decode-only line also
    times attn_varlen_fwd_prescheduled with the decode schedule built ahead, and the build;
    each bf16 prefill-only line attn_varlen_fwd_scheduled with the prefill schedule built
    ahead, and the build). One JSON line per (workload,
    pass, partition): mean call time by HIP events with the inputs hot in the caches, the
    algorithmic prefill TFLOP/s and decode GB/s of that call, and its % of the MI355X roofline,
    (prefill flops / MFMA peak + decode bytes / 8 TB/s) / call time, the MFMA peak being fp32
    (157.3 TFLOP/s) for the fp32 case and bf16 otherwise. The three small prefill workloads are
    also timed cold: the calls rotate over enough copies of q, the cache and the outputs (at
    least 512 MiB, twice the 256 MiB last-level cache) that no call finds its inputs in a cache.
    The seed argument is unused: workload k has seed k."""
    import torch
    import exact_softmax_attention_paged_amd as A
    import gen
    del seed
    for k in (1, 2, 3, 4, 5):
        b = gen.config(k)
        fp32 = b.dtype == "f32"
        parts = [0, 512] if k == 4 else [0]
        bt, qsl, sl = (torch.from_numpy(x).to(dev) for x in (b.block_table, b.query_start_loc,
                                                             b.seq_lens))
        for pt in parts:
            desc = A.make_desc(num_seqs=b.num_seqs, num_tokens=b.num_tokens,
                               num_decodes=b.num_decodes, max_query_len=b.max_query_len,
                               max_seq_len=b.max_seq_len, num_heads=b.num_heads,
                               num_kv_heads=b.num_kv_heads, head_size=b.head_size,
                               num_blocks=b.num_blocks, block_size=b.block_size,
                               max_blocks_per_seq=b.max_blocks_per_seq,
                               dtype=A.ATTN_F32 if fp32 else A.ATTN_BF16, partition_tokens=pt)
            ws = torch.empty(max(A.attn_workspace_bytes(desc), 1), dtype=torch.uint8, device=dev)
            for li, (causal, window) in enumerate(b.passes):
                q, kv = gen.make_tensors(b, k, dev, layer=li)
                out = torch.empty_like(q)
                lse = torch.empty(b.num_tokens, b.num_heads, dtype=torch.float32, device=dev)
                reps = 10 if b.num_tokens > 10000 else 100
                t = _time_ms(lambda: A.attn_varlen_fwd(desc, q, kv, bt, qsl, sl, b.scale,
                                                       causal, window, out, lse, ws), reps)
                flops, dec_unique, dec_logical = algorithmic_work(b, causal, window)
                peak = 157.3e12 if fp32 else PEAK_BF16_FLOPS
                rec = {"report": "configs", "workload": gen.CONFIG_NAMES[k], "pass": li,
                       "causal": causal, "window": window, "dtype": b.dtype,
                       "partition_tokens": pt if b.num_decodes else None,
                       "partition_tokens_used": A.attn_decode_partition_tokens(desc)
                       if b.num_decodes else None,
                       "call_ms": round(t, 4), "prefill_gflop": round(flops / 1e9, 3)}
                rec.update(_rates(t, flops, dec_unique if b.num_decodes else 0, peak))
                if b.num_decodes == b.num_seqs:
                    # the decode schedule built once ahead (a batch builds it once for all
                    # its layers) and the call that reads it instead of building its own
                    ds = torch.empty(A.attn_decode_schedule_bytes(desc, window) // 4,
                                     dtype=torch.int32, device=dev)
                    tb = _time_ms(lambda: A.attn_build_decode_schedule(desc, sl, window, ds),
                                  reps)
                    tp = _time_ms(lambda: A.attn_varlen_fwd_prescheduled(
                        desc, q, kv, bt, qsl, sl, b.scale, causal, window, out, lse, ws,
                        decode_schedule=ds), reps)
                    pre = {"call_ms": round(tp, 4), "schedule_build_ms": round(tb, 4)}
                    pre.update(_rates(tp, 0, dec_unique, peak))
                    rec["prescheduled"] = pre
                if b.num_decodes == 0 and not fp32:
                    # the prefill work schedule built once ahead (once per batch and mask for
                    # all its layers) and the call that dispatches its grid from it
                    ps = torch.empty(A.attn_schedule_bytes(desc) // 4, dtype=torch.int32,
                                     device=dev)
                    tb = _time_ms(lambda: A.attn_build_schedule(desc, qsl, sl, causal, window,
                                                                ps), reps)
                    ts = _time_ms(lambda: A.attn_varlen_fwd_scheduled(
                        desc, q, kv, bt, qsl, sl, b.scale, causal, window, out, lse, ws, ps),
                        reps)
                    sch = {"call_ms": round(ts, 4), "schedule_build_ms": round(tb, 4)}
                    sch.update(_rates(ts, flops, 0, peak))
                    rec["scheduled"] = sch
                if k <= 3:
                    rec["cold"] = _cold_rates(A, b, desc, k, li, causal, window, bt, qsl, sl,
                                              ws, flops, peak, dev)
                print(json.dumps(rec), flush=True)
                del q, kv, out, lse
            del ws
        torch.cuda.empty_cache()


def _rates(ms, flops, dec_bytes, peak):
    sec = ms / 1e3
    return {"prefill_tflops": round(flops / sec / 1e12, 1) if flops else None,
            "decode_gb_unique": round(dec_bytes / 1e9, 4) if dec_bytes else None,
            "decode_gbps": round(dec_bytes / sec / 1e9, 1) if dec_bytes else None,
            "pct_of_roofline": round(100 * (flops / peak + dec_bytes / PEAK_HBM_BYTES) / sec, 2)}


def _cold_rates(A, b, desc, k, li, causal, window, bt, qsl, sl, ws, flops, peak, dev):
    """Mean call time over calls that each use the next of N copies of the inputs and outputs
    (N copies >= COLD_ROTATION_BYTES), after one warm-up pass over all copies."""
    import torch
    import gen
    q0, kv0 = gen.make_tensors(b, k, dev, layer=li)
    per_set = (q0.numel() * 2 + kv0.numel()) * q0.element_size() + b.num_tokens * b.num_heads * 4
    n = max(2, -(-COLD_ROTATION_BYTES // per_set))
    sets = [(q0.clone(), kv0.clone(), torch.empty_like(q0),
             torch.empty(b.num_tokens, b.num_heads, dtype=torch.float32, device=dev))
            for _ in range(n)]
    del q0, kv0

    def call(i):
        q, kv, out, lse = sets[i % n]
        A.attn_varlen_fwd(desc, q, kv, bt, qsl, sl, b.scale, causal, window, out, lse, ws)
    for i in range(n):
        call(i)
    torch.cuda.synchronize()
    reps = 4 * n
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    res = {"input_sets": n, "rotation_mib": round(n * per_set / 2**20, 1), "call_ms": round(ms, 4)}
    res.update(_rates(ms, flops, 0, peak))
    del sets
    torch.cuda.empty_cache()
    return res


_probes = None


def probes():
    """libattn_probes.so (include/attn_probes.h): the HBM read stream and MFMA loop probes."""
    global _probes
    if _probes is None:
        import ctypes
        import torch  # noqa: F401  (the HIP runtime torch uses, loaded first)
        path = os.path.join(ROOT, "exact_softmax_attention_paged_amd", "libattn_probes.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build with "
                               "`python -m exact_softmax_attention_paged_amd.build`")
        L = ctypes.CDLL(path)
        vp, i32, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64
        L.attn_probe_read_stream.argtypes = [vp, u64, vp, i32, i32, vp]
        L.attn_probe_read_stream.restype = i32
        L.attn_probe_mfma_loop.argtypes = [vp, vp, i32, i32, vp]
        L.attn_probe_mfma_loop.restype = i32
        L.attn_probe_lds_read.argtypes = [vp, vp, i32, i32, i32, vp]
        L.attn_probe_lds_read.restype = i32
        _probes = L
    return _probes


def mfma_probe(dev, workgroups=256, iters=20000, reps=3):
    """Run the MFMA loop probe: returns (TFLOP/s, mean shader clock in MHz under that load)."""
    import ctypes
    import torch
    clocks = torch.zeros(4 * workgroups, dtype=torch.int64, device=dev)
    sink = torch.zeros(8 * workgroups, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def run():
        assert probes().attn_probe_mfma_loop(clocks.data_ptr(), sink.data_ptr(), workgroups,
                                             iters, stream) == 0
    ms = _time_ms(run, reps, warmup=1)
    c = clocks.view(workgroups, 4).cpu().numpy().astype(np.float64)
    mhz = float(np.median((c[:, 1] - c[:, 0]) / np.maximum(c[:, 3] - c[:, 2], 1.0) * 100.0))
    flops = workgroups * 8.0 * iters * 4 * 32768
    return flops / (ms / 1e3) / 1e12, mhz


def lds_probe(dev, transposing, workgroups=256, iters=4000, reps=3):
    """Run the LDS read probe: returns (bytes per shader clock per CU, shader clock in MHz,
    TB/s over the whole chip)."""
    import ctypes
    import torch
    clocks = torch.zeros(4 * workgroups, dtype=torch.int64, device=dev)
    sink = torch.zeros(512 * workgroups, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def run():
        assert probes().attn_probe_lds_read(clocks.data_ptr(), sink.data_ptr(), workgroups,
                                            iters, int(transposing), stream) == 0
    ms = _time_ms(run, reps, warmup=1)
    c = clocks.view(workgroups, 4).cpu().numpy().astype(np.float64)
    cycles = float(np.median(c[:, 1] - c[:, 0]))
    mhz = float(np.median((c[:, 1] - c[:, 0]) / np.maximum(c[:, 3] - c[:, 2], 1.0) * 100.0))
    per_wg = 8.0 * iters * 8 * (512 if transposing else 1024)
    return per_wg / cycles, mhz, workgroups * per_wg / (ms / 1e3) / 1e12


def ceilings_report(dev):
    """What this device delivers outside the attention kernels, beside the spec peaks the
    roofline fractions use. Own probes (libattn_probes.so, the instruction forms the kernels
    use): a 4 GiB HBM read stream of 16-byte loads (plain, and non-temporal as the decode
    kernel's K/V loads) at several grid sizes, and back-to-back
    v_mfma_f32_32x32x16_bf16 (8 waves per workgroup, 4 independent accumulators per wave) with
    the shader clock under that load. Vendor paths beside them: a bf16 GEMM through torch.mm
    (8192 x 8192 x 8192, contiguous operands) and a 4 GiB device-to-device copy (read + write
    bytes). Last, the LDS read rate per CU of the prefill kernel's two LDS read forms
    (ds_read_b128 for its K operands, ds_read_b64_tr_b16 for its V^T operands; one workgroup of
    8 waves per CU, 8 reads in flight per wave). One JSON line each."""
    import ctypes
    import torch
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    src = torch.ones(1 << 30, device=dev, dtype=torch.int32)           # 4 GiB
    for nt, wgs in [(0, w) for w in (1024, 2048, 4096, 8192, 16384)] + \
            [(1, w) for w in (1024, 4096, 16384)]:
        sink = torch.empty(wgs * 256, device=dev, dtype=torch.int32)
        ms = _time_ms(lambda: probes().attn_probe_read_stream(
            src.data_ptr(), src.numel() * 4, sink.data_ptr(), wgs, nt, stream), 10)
        byts = src.numel() * 4.0
        print(json.dumps({"report": "ceilings", "what": f"own HBM read stream, 4 GiB, 16-byte "
                          f"{'non-temporal ' if nt else ''}loads, {wgs} workgroups x 256 threads",
                          "ms": round(ms, 4), "gbps": round(byts / (ms / 1e3) / 1e9, 1),
                          "frac_of_spec": round(byts / (ms / 1e3) / PEAK_HBM_BYTES, 4)}),
              flush=True)
    del src
    for wgs in (256, 512):
        tflops, mhz = mfma_probe(dev, wgs, 20000)
        print(json.dumps({"report": "ceilings", "what": f"own v_mfma_f32_32x32x16_bf16 loop, "
                          f"{wgs} workgroups x 8 waves, 4 independent accumulators per wave",
                          "tflops": round(tflops, 1),
                          "frac_of_spec": round(tflops * 1e12 / PEAK_BF16_FLOPS, 4),
                          "shader_clock_mhz": round(mhz, 1),
                          "frac_of_peak_at_that_clock": round(
                              tflops * 1e12 / (PEAK_BF16_FLOPS * mhz / 2400.0), 4)}),
              flush=True)
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    ms = _time_ms(lambda: torch.mm(a, b, out=c), 20)
    flops = 2.0 * n * n * n
    print(json.dumps({"report": "ceilings", "what": "bf16 GEMM 8192^3 (torch.mm)",
                      "ms": round(ms, 4), "tflops": round(flops / (ms / 1e3) / 1e12, 1),
                      "frac_of_spec": round(flops / (ms / 1e3) / PEAK_BF16_FLOPS, 4)}),
          flush=True)
    del a, b, c
    src = torch.empty(1 << 30, device=dev, dtype=torch.int32)
    dst = torch.empty_like(src)
    ms = _time_ms(lambda: dst.copy_(src), 20)
    byts = 2.0 * src.numel() * 4
    print(json.dumps({"report": "ceilings", "what": "4 GiB device copy (read + write)",
                      "ms": round(ms, 4), "gbps": round(byts / (ms / 1e3) / 1e9, 1),
                      "frac_of_spec": round(byts / (ms / 1e3) / PEAK_HBM_BYTES, 4)}),
          flush=True)
    del src, dst
    for tr in (0, 1):
        bpc, mhz, tbps = lds_probe(dev, tr)
        print(json.dumps({"report": "ceilings", "what": "own LDS read loop, 256 workgroups x 8 "
                          "waves, " + ("ds_read_b64_tr_b16 (8 bytes per lane)" if tr else
                                       "ds_read_b128 (16 bytes per lane)"),
                          "bytes_per_clock_per_cu": round(bpc, 1), "shader_clock_mhz": round(mhz, 1),
                          "tbps_chip": round(tbps, 1)}), flush=True)


def mixed_step(batch, layers, dev):
    """The timed step's launch configuration: at the start of the step, the decode work
    schedule of each distinct window (it depends only on the decode rows' seq_lens, so one
    build serves every pass with that window); per layer pass, the decode rows (split-KV
    kernel + LSE merge, their own descriptor, reading the prebuilt schedule) and the prefill
    rows (prefill kernel, query starts rebased to 0). Within a pass the two row sets are independent, so the decode call goes to
    a second stream (default priority) forked from torch's current stream at the start of the
    pass and joined back at its end, while the prefill call runs on the current stream: the
    HBM-bound decode kernels then run beside the MFMA-bound prefill kernel on the CUs its
    workgroups leave free. Passes do not overlap (a model's next layer needs this one's
    output). Returns step(ev=None) and the out / lse tensors it writes (one per
    pass); with ev, step records ev[pass][0..1] around the decode call on the decode stream
    and ev[pass][2..3] around the prefill call on the current stream."""
    import torch
    import exact_softmax_attention_paged_amd as A
    nd = batch.num_decodes
    tok0 = int(batch.query_start_loc[nd])
    bt = torch.from_numpy(batch.block_table).to(dev)
    sl = torch.from_numpy(batch.seq_lens).to(dev)
    qsl_np = batch.query_start_loc
    qsl_dec = torch.from_numpy(qsl_np[:nd + 1].copy()).to(dev)
    qsl_pre = torch.from_numpy((qsl_np[nd:] - qsl_np[nd]).astype(np.int32)).to(dev)
    bt_dec, bt_pre = bt[:nd].contiguous(), bt[nd:].contiguous()
    sl_dec, sl_pre = sl[:nd].contiguous(), sl[nd:].contiguous()
    common = dict(num_heads=batch.num_heads, num_kv_heads=batch.num_kv_heads,
                  head_size=batch.head_size, num_blocks=batch.num_blocks,
                  block_size=batch.block_size, max_blocks_per_seq=batch.max_blocks_per_seq,
                  dtype=A.ATTN_BF16)
    desc_dec = A.make_desc(num_seqs=nd, num_tokens=nd, num_decodes=nd, max_query_len=1,
                           max_seq_len=int(batch.seq_lens[:nd].max()), **common)
    desc_pre = A.make_desc(num_seqs=batch.num_seqs - nd, num_tokens=batch.num_tokens - tok0,
                           num_decodes=0, max_query_len=int(batch.query_lens[nd:].max()),
                           max_seq_len=int(batch.seq_lens[nd:].max()), **common)
    # one decode workspace per pass; one decode work schedule per distinct window, built once
    # per step (batch) at its start and read by every pass with that window
    wss = [torch.empty(A.attn_workspace_bytes(desc_dec), dtype=torch.uint8, device=dev)
           for _ in layers]
    windows = sorted({w for _, w in batch.passes})
    scheds = {w: torch.empty(max(A.attn_decode_schedule_bytes(desc_dec, w) // 4, 1),
                             dtype=torch.int32, device=dev) for w in windows}
    outs = [torch.empty_like(q) for q, _ in layers]
    lses = [torch.empty(batch.num_tokens, batch.num_heads, dtype=torch.float32, device=dev)
            for _ in layers]
    stream = torch.cuda.current_stream(dev)
    dec_stream = torch.cuda.Stream(dev)        # default priority
    fork, join = torch.cuda.Event(), torch.cuda.Event()

    def step(ev=None):
        fork.record(stream)
        dec_stream.wait_event(fork)
        for w in windows:
            A.attn_build_decode_schedule(desc_dec, sl_dec, w, scheds[w], dec_stream)
        for li, (q, kv) in enumerate(layers):
            causal, window = batch.passes[li]
            # a layer pass starts when the previous one has ended on both streams (a model's
            # next layer needs this layer's output); within it the row sets overlap
            fork.record(stream)
            dec_stream.wait_event(fork)
            if ev is not None:
                ev[li][0].record(dec_stream)
            A.attn_varlen_fwd_prescheduled(desc_dec, q[:nd], kv, bt_dec, qsl_dec, sl_dec,
                                           batch.scale, causal, window, outs[li][:nd],
                                           lses[li][:nd], wss[li],
                                           decode_schedule=scheds[window], stream=dec_stream)
            if ev is not None:
                ev[li][1].record(dec_stream)
                ev[li][2].record(stream)
            A.attn_varlen_fwd(desc_pre, q[tok0:], kv, bt_pre, qsl_pre, sl_pre, batch.scale,
                              causal, window, outs[li][tok0:], lses[li][tok0:], None, stream)
            if ev is not None:
                ev[li][3].record(stream)
            join.record(dec_stream)
            stream.wait_event(join)            # the pass ends when both row sets are done

    def prefill_call(li):
        """Layer pass li's prefill-rows call alone, on the current stream."""
        q, kv = layers[li]
        causal, window = batch.passes[li]
        A.attn_varlen_fwd(desc_pre, q[tok0:], kv, bt_pre, qsl_pre, sl_pre, batch.scale,
                          causal, window, outs[li][tok0:], lses[li][tok0:], None, stream)

    def decode_call(li):
        """Layer pass li's decode-rows call alone (its window's schedule built by the last
        step), on the current stream."""
        q, kv = layers[li]
        causal, window = batch.passes[li]
        A.attn_varlen_fwd_prescheduled(desc_dec, q[:nd], kv, bt_dec, qsl_dec, sl_dec,
                                       batch.scale, causal, window, outs[li][:nd],
                                       lses[li][:nd], wss[li], decode_schedule=scheds[window],
                                       stream=stream)

    step.prefill_call = prefill_call
    step.decode_call = decode_call

    return step, outs, lses


def mixed_one_launch_step(batch, layers, dev):
    """The mixed workload with one launch per layer pass (attn_varlen_fwd_mixed): at the start
    of the step the prefill work schedule of each distinct (causal, window) is built (one
    small kernel each, serving every pass with that mask); per pass one launch takes the
    decode rows (one wave per request and kv head group, no split-KV partitions) and the
    prefill rows. Returns step(ev=None) and the out / lse tensors (one per pass); with ev,
    step records ev[pass][0..1] around the pass's launch."""
    import torch
    import exact_softmax_attention_paged_amd as A
    bt, qsl, sl = (torch.from_numpy(x).to(dev) for x in (batch.block_table,
                                                         batch.query_start_loc, batch.seq_lens))
    desc = A.make_desc(num_seqs=batch.num_seqs, num_tokens=batch.num_tokens,
                       num_decodes=batch.num_decodes, max_query_len=batch.max_query_len,
                       max_seq_len=batch.max_seq_len, num_heads=batch.num_heads,
                       num_kv_heads=batch.num_kv_heads, head_size=batch.head_size,
                       num_blocks=batch.num_blocks, block_size=batch.block_size,
                       max_blocks_per_seq=batch.max_blocks_per_seq, dtype=A.ATTN_BF16)
    masks = sorted(set(batch.passes))
    scheds = {m: torch.empty(A.attn_schedule_bytes(desc) // 4, dtype=torch.int32, device=dev)
              for m in masks}
    outs = [torch.empty_like(q) for q, _ in layers]
    lses = [torch.empty(batch.num_tokens, batch.num_heads, dtype=torch.float32, device=dev)
            for _ in layers]

    def step(ev=None):
        for m in masks:
            A.attn_build_schedule(desc, qsl, sl, m[0], m[1], scheds[m])
        for li, (q, kv) in enumerate(layers):
            causal, window = batch.passes[li]
            if ev is not None:
                ev[li][0].record()
            A.attn_varlen_fwd_mixed(desc, q, kv, bt, qsl, sl, batch.scale, causal, window,
                                    outs[li], lses[li], scheds[(causal, window)])
            if ev is not None:
                ev[li][1].record()

    return step, outs, lses


def mixed_launch_report(dev, seed, steps=10, warmup=3):
    """The mixed workload's step two ways: per pass a decode call on a second stream beside
    a prefill call, and bench's timed configuration, one attn_varlen_fwd_mixed launch per
    pass. One JSON line each: wall ms per step and, for the one-launch step, the per-pass
    launch spans. Then, per pass, the decode rows alone through the one-launch kernel (its 64
    decode workgroups) and through the split-KV call."""
    import torch
    import gen
    batch = gen.config(5, seed=seed)
    layers = [gen.make_tensors(batch, seed, dev, layer=li) for li in range(len(batch.passes))]
    for name, make in (("two-stream", mixed_step), ("one-launch", mixed_one_launch_step)):
        step, _, _ = make(batch, layers, dev)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in layers]
               for _ in range(steps)]
        t0 = time.perf_counter()
        for s_ in range(steps):
            step(evs[s_])
        torch.cuda.synchronize()
        ms = 1e3 * (time.perf_counter() - t0) / steps
        rec = {"report": "mixed-launch", "step": name, "ms_per_step": round(ms, 4)}
        if name == "one-launch":
            rec["pass_ms"] = [round(float(np.mean([e[li][0].elapsed_time(e[li][1])
                                                   for e in evs])), 4)
                              for li in range(len(layers))]
        print(json.dumps(rec), flush=True)
        del step
        torch.cuda.synchronize()
    # the decode rows alone, through the one-launch kernel (its decode workgroups only) and
    # through the split-KV call: what one CU streams when the decode side runs by itself
    import exact_softmax_attention_paged_amd as A
    b = gen.subset_meta(batch, list(range(batch.num_decodes)))
    q = layers[0][0][:b.num_tokens].contiguous()
    kv = layers[0][1]
    bt, qsl, sl = (torch.from_numpy(x).to(dev) for x in (b.block_table, b.query_start_loc,
                                                         b.seq_lens))
    desc = A.make_desc(num_seqs=b.num_seqs, num_tokens=b.num_tokens, num_decodes=b.num_decodes,
                       max_query_len=1, max_seq_len=b.max_seq_len, num_heads=b.num_heads,
                       num_kv_heads=b.num_kv_heads, head_size=b.head_size,
                       num_blocks=b.num_blocks, block_size=b.block_size,
                       max_blocks_per_seq=b.max_blocks_per_seq, dtype=A.ATTN_BF16)
    out = torch.empty_like(q)
    lse = torch.empty(b.num_tokens, b.num_heads, dtype=torch.float32, device=dev)
    ws = torch.empty(A.attn_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    for li, (causal, window) in enumerate(batch.passes):
        _, dbytes, _ = algorithmic_work(batch, causal, window)
        tm = _time_ms(lambda: A.attn_varlen_fwd_mixed(desc, q, kv, bt, qsl, sl, b.scale, causal,
                                                      window, out, lse, None), 10)
        tp = _time_ms(lambda: A.attn_varlen_fwd(desc, q, kv, bt, qsl, sl, b.scale, causal,
                                                window, out, lse, ws), 10)
        print(json.dumps({"report": "mixed-launch", "step": f"decode rows alone, pass {li}",
                          "one_launch_kernel_ms": round(tm, 4), "split_kv_call_ms": round(tp, 4),
                          "decode_gb_unique": round(dbytes / 1e9, 3),
                          "one_launch_kernel_tbps": round(dbytes / tm / 1e9, 2),
                          "split_kv_call_tbps": round(dbytes / tp / 1e9, 2)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="run the 1 GiB copy calibration before the timed steps")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/mixed_pass_traffic.json from two rocprofv3 --pmc runs")
    ap.add_argument("--record-command", default="", help="command line stored with the record")
    ap.add_argument("--report", choices=["configs", "cascade", "kv-write", "fp8-decode",
                                         "schedule", "ceilings", "mixed-launch"],
                    help="instead of the headline step, time one of the next-step paths "
                         "against the plain path and print one JSON line per batch")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.record_traffic[0], args.record_traffic[1], args.record_command)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the attention kernels run on one device and "
              "there is no multi-GPU launch (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_softmax_attention_paged_amd as A
    import gen

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.pmc_probe:
        pmc_probe(dev)
    if args.report == "configs":
        configs_report(dev, args.seed)
        return
    if args.report == "cascade":
        cascade_report(dev, args.seed)
        return
    if args.report == "kv-write":
        kv_write_report(dev, args.seed)
        return
    if args.report == "fp8-decode":
        fp8_decode_report(dev, args.seed)
        return
    if args.report == "schedule":
        schedule_report(dev, args.seed)
        return
    if args.report == "ceilings":
        ceilings_report(dev)
        return
    if args.report == "mixed-launch":
        mixed_launch_report(dev, args.seed)
        return
    batch = gen.config(5, seed=args.seed)
    layers = [gen.make_tensors(batch, args.seed, dev, layer=li) for li in range(len(batch.passes))]
    step, outs, lses = mixed_one_launch_step(batch, layers, dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in layers]
           for _ in range(args.steps)]
    t_start = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_step = 1e3 * wall / args.steps

    flops = dbytes_u = dbytes_l = 0.0
    per_pass = []
    for li, (causal, window) in enumerate(batch.passes):
        f, bu, bl = algorithmic_work(batch, causal, window)
        per_pass.append({"causal": causal, "window": window, "prefill_gflop": f / 1e9,
                         "decode_gb_unique": bu / 1e9, "decode_gb_logical": bl / 1e9,
                         "launch_ms": round(float(np.mean([e[li][0].elapsed_time(e[li][1])
                                                           for e in evs])), 4)})
        flops += f
        dbytes_u += bu
        dbytes_l += bl
    floor_s = flops / PEAK_BF16_FLOPS + dbytes_u / PEAK_HBM_BYTES
    value = 100.0 * floor_s / (ms_step / 1e3)
    # dominant kernel: the one launch of layer pass 0 (causal), which holds the pass's decode
    # rows and its causal prefill rows
    pass0_ms = per_pass[0]["launch_ms"]
    flops0 = per_pass[0]["prefill_gflop"] * 1e9
    bytes0 = per_pass[0]["decode_gb_unique"] * 1e9
    achieved = flops0 / (pass0_ms / 1e3) / 1e12
    traffic = recorded_traffic()

    # after the timed region, each row set alone with the two-call helpers: the prefill rows'
    # launch and the decode rows' calls of each pass (their kernels' own roofline fractions,
    # which the combined launch does not show), and the two-stream step for comparison
    ts_step, _, _ = mixed_step(batch, layers, dev)
    for _ in range(2):
        ts_step()
    torch.cuda.synchronize()

    def timed(fn, reps=5):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for e in ev:
            e[0].record()
            fn()
            e[1].record()
        torch.cuda.synchronize()
        return float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    pre_alone = [timed(lambda li=li: ts_step.prefill_call(li)) for li in range(len(layers))]
    dec_alone = [timed(lambda li=li: ts_step.decode_call(li)) for li in range(len(layers))]
    ts_ms = timed(ts_step, 5)
    alone_ms = pre_alone[0]
    achieved_alone = flops0 / (alone_ms / 1e3) / 1e12
    # the shader clock under a full MFMA load (own probe, right after the timed region): the
    # 2.5 PFLOP/s spec assumes 2.4 GHz, and the chip runs MFMA-bound kernels below that
    try:
        probe_tflops, sclk_mhz = mfma_probe(dev, 256, 20000)
    except Exception as exc:          # the probes library is optional for the headline line
        print(f"mfma probe unavailable: {exc}", file=sys.stderr)
        probe_tflops, sclk_mhz = None, None
    pre_frac = flops / (sum(pre_alone) / 1e3) / PEAK_BF16_FLOPS
    dec_frac = dbytes_u / (sum(dec_alone) / 1e3) / PEAK_HBM_BYTES
    rec = {
        "metric": METRIC, "value": round(value, 3), "unit": "% of roofline",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "mixed-long-context: 120 decode (ctx U[4096,32768]) + 8 prefill "
                               "(q 2048, ctx U[4096,32768]), 64 q / 8 kv heads, d 128, bf16, "
                               "block 64, 2048-token shared prefix, 2 layer passes "
                               "(causal; causal + window 4096)",
                   "global_batch": batch.num_seqs, "num_tokens": batch.num_tokens,
                   "seed": args.seed, "parallelism": "none (1 GPU)"},
        "launch": "per step the prefill work schedule of each distinct mask (2 small kernels), "
                  "then per layer pass ONE attn_varlen_fwd_mixed launch holding the decode rows "
                  "(one wave per request and kv head, no split-KV partitions) and the prefill "
                  "rows",
        "two_stream_ms_per_step": round(ts_ms, 4),
        "two_stream_note": "the same step as two calls per pass (decode rows split-KV on a "
                           "second stream beside the prefill call), timed after the timed "
                           "region",
        "per_pass": per_pass,
        "prefill_ms_alone": [round(x, 4) for x in pre_alone],
        "decode_ms_alone": [round(x, 4) for x in dec_alone],
        "prefill_tflops_alone": round(flops / (sum(pre_alone) / 1e3) / 1e12, 2),
        "decode_gbps_alone": round(dbytes_u / (sum(dec_alone) / 1e3) / 1e9, 1),
        "prefill_frac": round(pre_frac, 4), "prefill_frac_target": 0.50,
        "decode_frac": round(dec_frac, 4), "decode_frac_target": 0.70,
        "fractions_note": "each row set alone after the timed region: prefill_frac = both "
                          "passes' prefill flops / their prefill-rows launches / 2.5 PFLOP/s; "
                          "decode_frac = unique decode bytes / the decode-rows calls (split-KV "
                          "kernel + merge, prebuilt schedule) / 8 TB/s; value is the combined "
                          "floor over the timed one-launch step",
        "roofline": {"bound": "mfma", "kernel": DOMINANT_KERNEL +
                     " (one launch: layer pass 0, its decode rows and causal prefill rows)",
                     "launch_ms": pass0_ms, "flop_per_launch": flops0,
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_FLOPS / 1e12,
                     "unit": "TFLOP/s", "frac": round(achieved / (PEAK_BF16_FLOPS / 1e12), 4),
                     "traffic": None if traffic is None else round(traffic),
                     "decode_bytes_per_launch": bytes0,
                     "floor_frac": round((flops0 / PEAK_BF16_FLOPS + bytes0 / PEAK_HBM_BYTES) /
                                         (pass0_ms / 1e3), 4)},
        "roofline_alone": {"kernel": "prefill_bf16_kernel<128, true, false> (the causal "
                                     "prefill rows of layer pass 0 alone, 5 launches after the "
                                     "timed region)",
                           "launch_ms": round(alone_ms, 4), "achieved": round(achieved_alone, 2),
                           "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                           "frac": round(achieved_alone / (PEAK_BF16_FLOPS / 1e12), 4)},
        "clock": None if sclk_mhz is None else {
            "shader_clock_mhz_under_mfma_load": round(sclk_mhz, 1),
            "probe": "own back-to-back v_mfma_f32_32x32x16_bf16 loop on every CU right after "
                     "the timed region (s_memtime against the 100 MHz s_memrealtime)",
            "probe_tflops": round(probe_tflops, 1),
            "roofline_frac_at_that_clock": round(
                achieved / (PEAK_BF16_FLOPS / 1e12 * sclk_mhz / 2400.0), 4),
            "roofline_alone_frac_at_that_clock": round(
                achieved_alone / (PEAK_BF16_FLOPS / 1e12 * sclk_mhz / 2400.0), 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(batch, layers, args.seed)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
