"""The device-built prefill schedule and the scheduled forward call: the schedule holds every
work item once with non-increasing cost (checked against the oracle's items, which are
defined from the attention mask; equal-cost items may come in any order), and the scheduled
call's results are bit-identical to the plain call's and match the oracle."""
import numpy as np
import pytest
import torch

import exact_softmax_attention_paged_amd as A
import gen
import oracle
from parity import compare, device_meta, oracle_on

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _desc(b):
    return A.make_desc(num_seqs=b.num_seqs, num_tokens=b.num_tokens, num_decodes=b.num_decodes,
                       max_query_len=b.max_query_len, max_seq_len=b.max_seq_len,
                       num_heads=b.num_heads, num_kv_heads=b.num_kv_heads, head_size=b.head_size,
                       num_blocks=b.num_blocks, block_size=b.block_size,
                       max_blocks_per_seq=b.max_blocks_per_seq, dtype=A.ATTN_BF16)


def build(b, causal, window):
    desc = _desc(b)
    bt, qsl, sl = device_meta(b, DEV)
    sched = torch.empty(A.attn_schedule_bytes(desc) // 4, dtype=torch.int32, device=DEV)
    A.attn_build_schedule(desc, qsl, sl, causal, window, sched)
    return desc, sched


BATCHES = [
    ("varlen-causal-d64", dict(ql=[200, 1, 1000, 640, 33, 257], sl=[200, 300, 1000, 2000, 900, 257],
                               hq=12, hkv=12, d=64, bs=16)),
    ("mixed-d128-gqa4", dict(ql=[1, 1, 1, 700, 1500, 64], sl=[100, 3000, 5, 4000, 1500, 5000],
                             hq=16, hkv=4, d=128, bs=32)),
]


def _batch(name, kw):
    seed = 80 + [x[0] for x in BATCHES].index(name)
    ql = kw["ql"]
    order = np.argsort([q != 1 for q in ql], kind="stable")      # decode rows first
    return gen.make_batch(name, num_heads=kw["hq"], num_kv_heads=kw["hkv"], head_size=kw["d"],
                          block_size=kw["bs"], dtype="bf16", query_lens=np.array(ql)[order],
                          seq_lens=np.array(kw["sl"])[order], passes=[(True, 0)], seed=seed,
                          pool_factor=2), seed


MASKS = [(False, 0), (True, 0), (True, 300)]


@pytest.mark.parametrize("name,kw", BATCHES, ids=[x[0] for x in BATCHES])
@pytest.mark.parametrize("causal,window", MASKS, ids=["noncausal", "causal", "w300"])
def test_schedule_lists_every_item_longest_first(name, kw, causal, window):
    b, _ = _batch(name, kw)
    print(f"[case] schedule {name} causal={causal} window={window}", flush=True)
    desc, sched = build(b, causal, window)
    torch.cuda.synchronize()
    s = sched.cpu().numpy()
    items = oracle.prefill_items(b.query_lens, b.seq_lens, b.num_decodes, causal, window)
    maxq = -(-b.max_query_len // 256)
    cost = {(r, t): c for r, t, c in items}
    n = int(s[0])
    assert n == len(items)
    listed = [(b.num_decodes + e // maxq, e % maxq) for e in s[1:1 + n]]
    assert sorted(listed) == sorted(cost)                     # every item exactly once
    costs = [cost[x] for x in listed]
    assert all(a >= c for a, c in zip(costs, costs[1:])), costs   # longest first


@pytest.mark.parametrize("name,kw", BATCHES, ids=[x[0] for x in BATCHES])
@pytest.mark.parametrize("causal,window", MASKS, ids=["noncausal", "causal", "w300"])
def test_scheduled_call_matches_plain_call_and_oracle(name, kw, causal, window):
    b, seed = _batch(name, kw)
    print(f"[case] scheduled fwd {name} causal={causal} window={window}", flush=True)
    q, kv = gen.make_tensors(b, seed, DEV, poison=True)
    desc, sched = build(b, causal, window)
    bt, qsl, sl = device_meta(b, DEV)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=DEV)
    ws = torch.empty(max(A.attn_workspace_bytes(desc), 1), dtype=torch.uint8, device=DEV)
    A.attn_varlen_fwd_scheduled(desc, q, kv, bt, qsl, sl, b.scale, causal, window, out, lse, ws,
                                sched)
    out2 = torch.empty_like(q)
    lse2 = torch.empty_like(lse)
    A.attn_varlen_fwd(desc, q, kv, bt, qsl, sl, b.scale, causal, window, out2, lse2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    ref_out, ref_lse = oracle_on(b, q, kv, causal, window)
    compare(out, lse, ref_out, ref_lse, label=name)


def test_one_schedule_serves_several_layers():
    name, kw = BATCHES[1]
    b, seed = _batch(name, kw)
    desc, sched = build(b, True, 0)
    bt, qsl, sl = device_meta(b, DEV)
    ws = torch.empty(max(A.attn_workspace_bytes(desc), 1), dtype=torch.uint8, device=DEV)
    for layer in range(2):
        q = gen.make_q(b, seed, DEV, layer=layer)
        kv = gen.make_kv(b, seed, DEV, layer=layer, poison=True)
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=DEV)
        A.attn_varlen_fwd_scheduled(desc, q, kv, bt, qsl, sl, b.scale, True, 0, out, lse, ws,
                                    sched)
        torch.cuda.synchronize()
        ref_out, ref_lse = oracle_on(b, q, kv, True, 0)
        compare(out, lse, ref_out, ref_lse, label=f"layer {layer}")


# ---- decode work schedule (built by every split-KV decode call, in the call's workspace)
DECODE_LENS = [1, 15, 16, 17, 511, 512, 513, 2047, 2048, 2049, 4095, 4096, 4097, 6000, 9000,
               300, 7777, 12345]


def segment(P):
    """Keys of one decode work item for partition length P (include/attn.h): a partition of
    up to 1024 keys is streamed by one wave, as many whole partitions per item as fit in 1024
    keys; a longer partition is one item."""
    return 1024 // P * P if P <= 1024 else P


def capped(n_keys, P, window):
    n = -(-n_keys // P)
    return min(n, -(-window // P) + 1) if window > 0 else n


def default_partition(num_decodes, num_heads, num_kv_heads, max_seq_len):
    """The library's partition length for partition_tokens = 0 (include/attn.h): the longest
    of 16384, 8192, ..., 256 giving at least 2048 split workgroups, else 256."""
    per_part = num_decodes * num_kv_heads * -(-(num_heads // num_kv_heads) // 16)
    P = 16384
    while P > 256 and per_part * -(-max_seq_len // P) < 2048:
        P //= 2
    return P


@pytest.mark.parametrize("window,part", [(0, 0), (0, 512), (3000, 0), (100, 1024)],
                         ids=["default", "p512", "w3000", "w100-p1024"])
def test_decode_schedule_lists_every_segment_longest_first(window, part):
    nd = len(DECODE_LENS)
    print(f"[case] decode schedule window={window} partition={part}", flush=True)
    b = gen.make_batch("decode-schedule", num_heads=8, num_kv_heads=2, head_size=64,
                       block_size=16, dtype="bf16", query_lens=[1] * nd, seq_lens=DECODE_LENS,
                       passes=[(True, window)], seed=91)
    q, kv = gen.make_tensors(b, 91, DEV, poison=True)
    desc = A.make_desc(num_seqs=nd, num_tokens=nd, num_decodes=nd, max_query_len=1,
                       max_seq_len=b.max_seq_len, num_heads=8, num_kv_heads=2, head_size=64,
                       num_blocks=b.num_blocks, block_size=16,
                       max_blocks_per_seq=b.max_blocks_per_seq, dtype=A.ATTN_BF16,
                       partition_tokens=part)
    bt, qsl, sl = device_meta(b, DEV)
    ws = torch.zeros(A.attn_workspace_bytes(desc), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty(nd, 8, dtype=torch.float32, device=DEV)
    A.attn_varlen_fwd(desc, q, kv, bt, qsl, sl, b.scale, True, window, out, lse, ws)
    torch.cuda.synchronize()
    # workspace layout of the C layer: partition results ([nd][Hq][max_parts][d] bf16 and
    # [nd][Hq][max_parts] fp32, padded to 256 bytes), then the schedule of the work items:
    # (request, segment) pairs, a segment being segment(P) keys
    P = part or default_partition(nd, 8, 2, b.max_seq_len)
    max_parts = capped(b.max_seq_len, P, window)
    S = segment(P)
    max_segs = capped(b.max_seq_len, S, window)
    rows = nd * 8 * max_parts
    off = -(-(rows * 64 * 2 + rows * 4) // 256) * 256
    s = ws[off:off + 4 * (1 + nd * max_segs)].view(torch.int32).cpu().numpy()
    items = oracle.decode_items(b.seq_lens, nd, window, S)
    cost = {(r, p): c for r, p, c in items}
    n = int(s[0])
    assert n == len(items)
    listed = [(int(e) // max_segs, int(e) % max_segs) for e in s[1:1 + n]]
    assert sorted(listed) == sorted(cost)                     # every partition exactly once
    costs = [cost[x] for x in listed]
    assert all(a >= c for a, c in zip(costs, costs[1:])), costs   # longest first
    ref_out, ref_lse = oracle_on(b, q, kv, True, window)
    compare(out, lse, ref_out, ref_lse, label=f"decode schedule w{window} p{part}")


# ---- decode schedule built ahead of the call (attn_build_decode_schedule) and read by
# attn_varlen_fwd_prescheduled
@pytest.mark.parametrize("window,part", [(0, 0), (0, 512), (3000, 0), (100, 1024)],
                         ids=["default", "p512", "w3000", "w100-p1024"])
def test_built_decode_schedule_equals_the_in_call_one(window, part):
    nd = len(DECODE_LENS)
    print(f"[case] built decode schedule window={window} partition={part}", flush=True)
    b = gen.make_batch("decode-schedule", num_heads=8, num_kv_heads=2, head_size=64,
                       block_size=16, dtype="bf16", query_lens=[1] * nd, seq_lens=DECODE_LENS,
                       passes=[(True, window)], seed=92)
    q, kv = gen.make_tensors(b, 92, DEV, poison=True)
    desc = A.make_desc(num_seqs=nd, num_tokens=nd, num_decodes=nd, max_query_len=1,
                       max_seq_len=b.max_seq_len, num_heads=8, num_kv_heads=2, head_size=64,
                       num_blocks=b.num_blocks, block_size=16,
                       max_blocks_per_seq=b.max_blocks_per_seq, dtype=A.ATTN_BF16,
                       partition_tokens=part)
    bt, qsl, sl = device_meta(b, DEV)
    P = part or default_partition(nd, 8, 2, b.max_seq_len)
    max_parts = capped(b.max_seq_len, P, window)
    S = segment(P)
    max_segs = capped(b.max_seq_len, S, window)
    # sized for one item per partition (at least one per segment)
    assert A.attn_decode_schedule_bytes(desc, window) == -(-(4 * (1 + nd * max_parts)) // 256) * 256
    sched = torch.full((A.attn_decode_schedule_bytes(desc, window) // 4,), -7, dtype=torch.int32,
                       device=DEV)
    A.attn_build_decode_schedule(desc, sl, window, sched)
    ws = torch.zeros(A.attn_workspace_bytes(desc), dtype=torch.uint8, device=DEV)
    out, out2 = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty(nd, 8, dtype=torch.float32, device=DEV)
    lse2 = torch.empty_like(lse)
    A.attn_varlen_fwd(desc, q, kv, bt, qsl, sl, b.scale, True, window, out, lse, ws)
    torch.cuda.synchronize()
    rows = nd * 8 * max_parts
    off = -(-(rows * 64 * 2 + rows * 4) // 256) * 256
    s_call = ws[off:off + 4 * (1 + nd * max_segs)].view(torch.int32).cpu().numpy()
    s_built = sched.cpu().numpy()
    n = int(s_built[0])
    assert n == int(s_call[0]) == len(oracle.decode_items(b.seq_lens, nd, window, S))
    cost = {(r, p): c for r, p, c in oracle.decode_items(b.seq_lens, nd, window, S)}
    listed = [(int(e) // max_segs, int(e) % max_segs) for e in s_built[1:1 + n]]
    assert sorted(listed) == sorted(cost)
    assert [cost[x] for x in listed] == [cost[(int(e) // max_segs, int(e) % max_segs)]
                                         for e in s_call[1:1 + n]]       # same cost order
    # the prescheduled call reads the built schedule and writes what the plain call wrote;
    # a fresh workspace shows that it builds nothing there
    ws2 = torch.zeros_like(ws)
    A.attn_varlen_fwd_prescheduled(desc, q, kv, bt, qsl, sl, b.scale, True, window, out2, lse2,
                                   ws2, decode_schedule=sched)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    assert not ws2[off:].any()


def test_prescheduled_call_serves_several_layers_of_a_mixed_batch():
    """Both schedules built once, three layer passes of the mixed GQA batch (decode rows +
    prefill rows, window 300): each pass is bit-identical to the plain call and matches the
    oracle; with only one of the two schedules the results are the same again."""
    name, kw = BATCHES[1]
    b, seed = _batch(name, kw)
    window = 300
    desc = _desc(b)
    bt, qsl, sl = device_meta(b, DEV)
    psched = torch.empty(A.attn_schedule_bytes(desc) // 4, dtype=torch.int32, device=DEV)
    A.attn_build_schedule(desc, qsl, sl, True, window, psched)
    dsched = torch.empty(A.attn_decode_schedule_bytes(desc, window) // 4, dtype=torch.int32,
                         device=DEV)
    A.attn_build_decode_schedule(desc, sl, window, dsched)
    ws = torch.empty(A.attn_workspace_bytes(desc), dtype=torch.uint8, device=DEV)
    for layer in range(3):
        print(f"[case] prescheduled {name} layer {layer}", flush=True)
        q = gen.make_q(b, seed, DEV, layer=layer)
        kv = gen.make_kv(b, seed, DEV, layer=layer, poison=True)
        res = []
        for ps, ds in ((None, None), (psched, dsched), (psched, None), (None, dsched)):
            out = torch.empty_like(q)
            lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=DEV)
            if ps is None and ds is None:
                A.attn_varlen_fwd(desc, q, kv, bt, qsl, sl, b.scale, True, window, out, lse, ws)
            else:
                A.attn_varlen_fwd_prescheduled(desc, q, kv, bt, qsl, sl, b.scale, True, window,
                                               out, lse, ws, prefill_schedule=ps,
                                               decode_schedule=ds)
            res.append((out, lse))
        torch.cuda.synchronize()
        for out, lse in res[1:]:
            assert torch.equal(out, res[0][0]) and torch.equal(lse, res[0][1])
        ref_out, ref_lse = oracle_on(b, q, kv, True, window)
        compare(res[1][0], res[1][1], ref_out, ref_lse, label=f"layer {layer}")
