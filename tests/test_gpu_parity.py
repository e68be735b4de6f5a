"""Parity of the HIP path with the CPU oracle, element by element, on seeded inputs.

Small batches (several tiles, ragged tails, every mask kind, GQA ratios 1..20, block sizes
16..512, decode and prefill rows, NaN in every slot no request may read) are compared in
full. The five workloads are run at full size in the bench's launch configuration: the tiny
fp32, BERT-large-shaped, GPT-2-shaped and paged GQA decode workloads are compared in full
(every row, every head), the mixed long-context workload on all of its decode rows and on the
rows of its 2048-token prefill requests where the kernels change behaviour (query-tile
edges, causal-diagonal and window-edge rows, plus seeded random rows)."""
import zlib

import numpy as np
import pytest
import torch

import exact_softmax_attention_paged_amd as A
import gen
from parity import compare, device_meta, oracle_on, run_library

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _batch(seed, *, ql, sl, hq, hkv, d, bs, dtype="bf16", pool_factor=2, shared=0):
    return gen.make_batch(f"case{seed}", num_heads=hq, num_kv_heads=hkv, head_size=d,
                          block_size=bs, dtype=dtype, query_lens=ql, seq_lens=sl,
                          passes=[(True, 0)], seed=seed, pool_factor=pool_factor,
                          shared_prefix_blocks=shared)


SMALL = [
    # name, kwargs
    ("prefill-d64-mha", dict(ql=[200, 1, 64, 129], sl=[200, 50, 300, 129], hq=4, hkv=4, d=64, bs=16)),
    ("prefill-d128-gqa4", dict(ql=[77, 130, 5], sl=[300, 130, 900], hq=8, hkv=2, d=128, bs=32)),
    ("decode-then-prefill-d128-gqa8", dict(ql=[1, 1, 1, 40, 300], sl=[1, 700, 1500, 1000, 300],
                                           hq=16, hkv=2, d=128, bs=16)),
    ("decode-d64-gqa20", dict(ql=[1, 1, 1], sl=[513, 2000, 64], hq=40, hkv=2, d=64, bs=64)),
    ("decode-d128-g1-bs512", dict(ql=[1, 1, 9], sl=[1025, 511, 520], hq=3, hkv=3, d=128, bs=512)),
    # block sizes that are multiples of 16 but not powers of two (block index by reciprocal)
    ("mixed-d128-gqa4-bs48", dict(ql=[1, 1, 200, 37], sl=[1000, 50, 700, 400], hq=8, hkv=2,
                                  d=128, bs=48)),
    ("mixed-d64-gqa4-bs80", dict(ql=[1, 150, 3], sl=[3000, 1500, 81], hq=4, hkv=1, d=64,
                                 bs=80)),
    # 8 decodes x 8 kv heads: the one-launch kernel's 8 decode workgroups each take one kv head
    ("decode8-kv8-then-prefill", dict(ql=[1] * 8 + [70], sl=[900, 33, 2500, 64, 1, 700, 1300,
                                                           129, 300], hq=16, hkv=8, d=128,
                                      bs=16)),
]
MASKS = [(False, 0), (True, 0), (True, 1), (True, 100), (True, 513)]


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("causal,window", MASKS, ids=[f"c{int(c)}w{w}" for c, w in MASKS])
def test_small_batches_match_oracle(name, kw, causal, window):
    seed = zlib.crc32(name.encode()) % 1000
    b = _batch(seed, **kw)
    print(f"[case] {name} causal={causal} window={window} decodes={b.num_decodes}", flush=True)
    q, kv = gen.make_tensors(b, seed, DEV, poison=True)
    out, lse = run_library(b, q, kv, causal, window)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_on(b, q, kv, causal, window)
    compare(out, lse, ref_out, ref_lse, label=name)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 300)])
def test_large_prefill_matches_oracle(d, causal, window):
    """Several 256-row query tiles per request, ragged ends, GQA 4."""
    b = _batch(11, ql=[1024, 1000, 777, 1024], sl=[1024, 1300, 2000, 1100], hq=32, hkv=8, d=d,
               bs=32)
    print(f"[case] large prefill d={d} causal={causal} window={window}", flush=True)
    q, kv = gen.make_tensors(b, 11, DEV, poison=True)
    out, lse = run_library(b, q, kv, causal, window)
    ref_out, ref_lse = oracle_on(b, q, kv, causal, window)
    compare(out, lse, ref_out, ref_lse, label="large prefill")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 37)])
def test_f32_matches_oracle(d, causal, window):
    b = _batch(5, ql=[100, 1, 33], sl=[100, 300, 200], hq=4, hkv=2, d=d, bs=16, dtype="f32")
    q, kv = gen.make_tensors(b, 5, DEV, poison=True)
    out, lse = run_library(b, q, kv, causal, window)
    ref_out, ref_lse = oracle_on(b, q, kv, causal, window)
    res = compare(out, lse, ref_out, ref_lse, label="f32")
    assert res["out_max"] < 1e-4 and res["lse_max"] < 1e-4, res


# ---------------------------------------------------------------- the five workloads
@pytest.mark.parametrize("k", [1, 2, 3])
def test_workload_full_parity(k):
    b = gen.config(k)
    causal, window = b.passes[0]
    print(f"[case] workload {k} ({b.name}) full", flush=True)
    q, kv = gen.make_tensors(b, k, DEV, poison=True)
    out, lse = run_library(b, q, kv, causal, window)
    ref_out, ref_lse = oracle_on(b, q, kv, causal, window)
    print(compare(out, lse, ref_out, ref_lse, label=b.name))


def _rows_all(b, r):
    return np.arange(int(b.query_lens[r]))


def _rows_tile_edges(b, r, window, seed=0):
    """Rows of a prefill request that sit where the kernels change behaviour: the first and
    last row of every 256-row query tile, the rows whose causal edge falls at the start or end
    of a 128-key tile (the diagonal tiles), the rows whose window start falls there, and a few
    seeded random rows."""
    ql = int(b.query_lens[r])
    cl = int(b.seq_lens[r]) - ql
    i = np.arange(ql)
    picks = [i[(i % 256 == 0) | (i % 256 == 255) | (i == ql - 1)]]
    diag = i[((cl + i) % 128 == 0) | ((cl + i) % 128 == 127)]
    picks.append(diag[:6])
    if window > 0:
        lo = cl + i - window + 1
        edge = i[(lo >= 0) & ((lo % 128 == 0) | (lo % 128 == 127))]
        picks.append(edge[:6])
    picks.append(np.random.default_rng(seed + r).choice(ql, min(ql, 8), replace=False))
    return np.unique(np.concatenate(picks))


def _compare_requests(b, q, kv, out, lse, causal, window, requests, rows_of, chunk):
    """Compare out / lse with the oracle on rows_of(b, r) of every request in ``requests``,
    handing the oracle ``chunk`` requests at a time (gen.subset copies just their blocks to
    the host). Every chunk must meet the tolerances; returns the worst figures and the
    number of rows compared."""
    worst = {"out_max": 0.0, "out_mean": 0.0, "lse_max": 0.0, "rows": 0}
    qsl = b.query_start_loc
    for c0 in range(0, len(requests), chunk):
        req = list(requests[c0:c0 + chunk])
        sub, qs, kvs = gen.subset(b, req, q, kv)
        qsl_sub = sub.query_start_loc
        rows_sub, rows_full = [], []
        for i, r in enumerate(req):
            pick = rows_of(b, r)
            rows_sub.extend(qsl_sub[i] + pick)
            rows_full.extend(qsl[r] + pick)
        ref_out, ref_lse = oracle_on(sub, qs, kvs, causal, window, rows=rows_sub)
        idx = torch.as_tensor(np.asarray(rows_full, dtype=np.int64), device=out.device)
        res = compare(out[idx], lse[idx], ref_out[rows_sub], ref_lse[rows_sub],
                      label=f"{b.name} requests {req[0]}..{req[-1]}")
        for k in ("out_max", "out_mean", "lse_max"):
            worst[k] = max(worst[k], res[k])
        worst["rows"] += len(rows_full)
        del sub, qs, kvs, ref_out, ref_lse
    return worst


@pytest.mark.parametrize("partition_tokens", [512, 0], ids=["part512", "default-part"])
def test_workload4_full_parity(partition_tokens):
    """The paged GQA decode workload at full size, every one of its 256 requests compared with
    the oracle: at its stated 512-token partitions (split-KV plus the LSE merge) and at the
    library default (what the per-workload report times)."""
    b = gen.config(4)
    print(f"[case] paged GQA decode full size, all requests, partition {partition_tokens}", flush=True)
    q, kv = gen.make_tensors(b, 4, DEV)
    out, lse = run_library(b, q, kv, True, 0, partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    print(_compare_requests(b, q, kv, out, lse, True, 0, list(range(b.num_seqs)), _rows_all,
                            chunk=32))


@pytest.mark.parametrize("layer", [0, 1])
def test_workload5_full_decode_parity(layer):
    """The mixed long-context workload at full size in one call (decode and prefill rows
    together): every third decode row (the bench launch test below compares all 120) and the
    tile-edge rows of every prefill request, every q head, compared with the oracle."""
    b = gen.config(5)
    causal, window = b.passes[layer]
    print(f"[case] mixed long-context layer {layer} full size, all decode rows", flush=True)
    q, kv = gen.make_tensors(b, 5, DEV, layer=layer)
    out, lse = run_library(b, q, kv, causal, window)
    torch.cuda.synchronize()
    print(_compare_requests(b, q, kv, out, lse, causal, window,
                            list(range(0, b.num_decodes, 3)), _rows_all, chunk=20))
    print(_compare_requests(b, q, kv, out, lse, causal, window,
                            list(range(b.num_decodes, b.num_seqs)),
                            lambda bb, r: _rows_tile_edges(bb, r, window), chunk=2))


@pytest.mark.parametrize("layer", [0, 1])
def test_workload5_bench_launch_parity(layer):
    """The timed step's own launch configuration (bench.mixed_step: the decode rows and the
    prefill rows as two calls with their own descriptors, the decode call on a second
    stream): all 120 decode rows and the tile-edge rows of every prefill request."""
    import dataclasses
    import bench
    b = gen.config(5)
    q, kv = gen.make_tensors(b, 5, DEV, layer=layer)
    bl = dataclasses.replace(b, passes=[b.passes[layer]])
    causal, window = bl.passes[0]
    print(f"[case] mixed long-context layer {layer} in the bench launch configuration", flush=True)
    step, outs, lses = bench.mixed_step(bl, [(q, kv)], torch.device(DEV))
    step()
    torch.cuda.synchronize()
    print(_compare_requests(b, q, kv, outs[0], lses[0], causal, window,
                            list(range(b.num_decodes)), _rows_all, chunk=20))
    print(_compare_requests(b, q, kv, outs[0], lses[0], causal, window,
                            list(range(b.num_decodes, b.num_seqs)),
                            lambda bb, r: _rows_tile_edges(bb, r, window), chunk=2))


@pytest.mark.parametrize("layer", [0, 1])
def test_workload5_one_launch_parity(layer):
    """One attn_varlen_fwd_mixed launch per layer pass (bench.mixed_one_launch_step): all
    120 decode rows and the tile-edge rows of every prefill request."""
    import dataclasses
    import bench
    b = gen.config(5)
    q, kv = gen.make_tensors(b, 5, DEV, layer=layer)
    bl = dataclasses.replace(b, passes=[b.passes[layer]])
    causal, window = bl.passes[0]
    print(f"[case] mixed long-context layer {layer} in one launch", flush=True)
    step, outs, lses = bench.mixed_one_launch_step(bl, [(q, kv)], torch.device(DEV))
    step()
    torch.cuda.synchronize()
    print(_compare_requests(b, q, kv, outs[0], lses[0], causal, window,
                            list(range(b.num_decodes)), _rows_all, chunk=20))
    print(_compare_requests(b, q, kv, outs[0], lses[0], causal, window,
                            list(range(b.num_decodes, b.num_seqs)),
                            lambda bb, r: _rows_tile_edges(bb, r, window), chunk=2))


ONE_LAUNCH = ["decode-then-prefill-d128-gqa8", "decode-d64-gqa20", "decode-d128-g1-bs512",
              "mixed-d128-gqa4-bs48", "mixed-d64-gqa4-bs80", "decode8-kv8-then-prefill"]


@pytest.mark.parametrize("name", ONE_LAUNCH)
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 37)],
                         ids=["noncausal", "causal", "w37"])
def test_one_launch_small_batches(name, causal, window):
    """attn_varlen_fwd_mixed on small mixed batches, every row against the oracle; its
    prefill rows run the prefill kernel's code and equal the plain call's bit for bit."""
    kw = dict(SMALL)[name]
    seed = 300 + ONE_LAUNCH.index(name)
    b = _batch(seed, **kw)
    print(f"[case] one launch {name} causal={causal} window={window}", flush=True)
    q, kv = gen.make_tensors(b, seed, DEV, poison=True)
    desc = A.make_desc(num_seqs=b.num_seqs, num_tokens=b.num_tokens, num_decodes=b.num_decodes,
                       max_query_len=b.max_query_len, max_seq_len=b.max_seq_len,
                       num_heads=b.num_heads, num_kv_heads=b.num_kv_heads,
                       head_size=b.head_size, num_blocks=b.num_blocks,
                       block_size=b.block_size, max_blocks_per_seq=b.max_blocks_per_seq,
                       dtype=A.ATTN_BF16)
    bt, qsl, sl = device_meta(b, DEV)
    sched = torch.empty(A.attn_schedule_bytes(desc) // 4, dtype=torch.int32, device=DEV)
    A.attn_build_schedule(desc, qsl, sl, causal, window, sched)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((b.num_tokens, b.num_heads), float("nan"), dtype=torch.float32, device=DEV)
    A.attn_varlen_fwd_mixed(desc, q, kv, bt, qsl, sl, b.scale, causal, window, out, lse, sched)
    out_p, lse_p = run_library(b, q, kv, causal, window)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_on(b, q, kv, causal, window)
    compare(out, lse, ref_out, ref_lse, label=f"one launch {name}")
    tok0 = int(b.query_start_loc[b.num_decodes])
    assert torch.equal(out[tok0:].view(torch.int16), out_p[tok0:].view(torch.int16))
    assert torch.equal(lse[tok0:], lse_p[tok0:])


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 8192)], ids=["causal", "w8192"])
def test_very_long_contexts(causal, window):
    """Contexts of 100K-131K keys, past the workloads' 32K: decode rows split into up to 64
    partitions, and a prefill request of 300 queries walking about 940 key tiles. Block size
    16, so a request spans up to 8192 blocks. Sampled rows of both kinds."""
    b = _batch(77, ql=[1, 1, 300], sl=[131072, 100003, 120300], hq=8, hkv=2, d=128, bs=16,
               pool_factor=1)
    print(f"[case] very long contexts causal={causal} window={window}", flush=True)
    q, kv = gen.make_tensors(b, 77, DEV, poison=True)
    out, lse = run_library(b, q, kv, causal, window)
    torch.cuda.synchronize()
    rows = [0, 1, 2, 3, 150, 300, 301]
    ref_out, ref_lse = oracle_on(b, q, kv, causal, window, rows=rows)
    print(compare(out, lse, ref_out, ref_lse, rows=rows, label="very long contexts"))


def test_many_tiny_decodes():
    """5000 decode requests with 1..64 keys (single-key contexts included), GQA 4: many small
    workgroups, partitions holding a handful of keys, and direct writes from the split
    kernel. Every row is compared."""
    rng = np.random.default_rng(123)
    sl = rng.integers(1, 64, size=5000, endpoint=True)
    sl[:3] = 1
    b = _batch(123, ql=[1] * 5000, sl=sl.tolist(), hq=8, hkv=2, d=64, bs=16)
    print("[case] 5000 tiny decodes", flush=True)
    q, kv = gen.make_tensors(b, 123, DEV, poison=True)
    out, lse = run_library(b, q, kv, True, 0)
    ref_out, ref_lse = oracle_on(b, q, kv, True, 0)
    print(compare(out, lse, ref_out, ref_lse, label="tiny decodes"))


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 37)],
                         ids=["noncausal", "causal", "w37"])
def test_requests_without_queries_write_nothing(causal, window):
    """Requests with query_len 0 (a context but no new token, or nothing at all) sit between
    decode and prefill requests: they own no output row, and every other row still matches
    the oracle. The rows of the whole output are checked, and a sentinel shows that nothing
    outside them is written."""
    b = _batch(88, ql=[1, 1, 0, 300, 0, 5, 0], sl=[100, 2000, 500, 300, 0, 900, 17], hq=8,
               hkv=2, d=128, bs=16)
    print(f"[case] zero-length queries causal={causal} window={window}", flush=True)
    q, kv = gen.make_tensors(b, 88, DEV, poison=True)
    bt, qsl, sl = device_meta(b, DEV)
    desc = A.make_desc(num_seqs=b.num_seqs, num_tokens=b.num_tokens, num_decodes=b.num_decodes,
                       max_query_len=b.max_query_len, max_seq_len=b.max_seq_len, num_heads=8,
                       num_kv_heads=2, head_size=128, num_blocks=b.num_blocks, block_size=16,
                       max_blocks_per_seq=b.max_blocks_per_seq, dtype=A.ATTN_BF16)
    ws = torch.empty(A.attn_workspace_bytes(desc), dtype=torch.uint8, device=DEV)
    # one sentinel row beyond the last token in both outputs
    out_full = torch.full((b.num_tokens + 1, 8, 128), 7.0, dtype=q.dtype, device=DEV)
    lse_full = torch.full((b.num_tokens + 1, 8), 7.0, dtype=torch.float32, device=DEV)
    A.attn_varlen_fwd(desc, q, kv, bt, qsl, sl, b.scale, causal, window,
                      out_full[:b.num_tokens], lse_full[:b.num_tokens], ws)
    torch.cuda.synchronize()
    assert bool((out_full[b.num_tokens] == 7.0).all()) and bool((lse_full[b.num_tokens] == 7.0).all())
    ref_out, ref_lse = oracle_on(b, q, kv, causal, window)
    compare(out_full[:b.num_tokens], lse_full[:b.num_tokens], ref_out, ref_lse,
            label="zero-length queries")
