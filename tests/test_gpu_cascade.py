"""Parity of the cascade path (attn_cascade_fwd: prefix pass over all query tokens, suffix
pass, log-sum-exp merge) with the CPU oracle, element by element, on seeded inputs.

The reference is plain attention over all keys (the method is exact, and the cascade
oracle's decomposition is pinned to plain attention on the CPU). Cases cover decode and
prefill rows, causal and non-causal suffixes, GQA, several block sizes and partition sizes,
contexts that end exactly at the prefix, and NaN in every slot no request may read; the
mixed long-context workload (2048-token shared prefix) is checked at full size on sampled
rows."""
import numpy as np
import pytest
import torch

import exact_softmax_attention_paged_amd as A
import gen
import oracle
from parity import compare, device_meta, host_f32, oracle_on, run_library

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_cascade(b, q, kv, causal, prefix, partition_tokens=0):
    bt, qsl, sl = device_meta(b, q.device)
    desc = A.make_desc(num_seqs=b.num_seqs, num_tokens=q.shape[0], num_decodes=b.num_decodes,
                       max_query_len=b.max_query_len, max_seq_len=b.max_seq_len,
                       num_heads=b.num_heads, num_kv_heads=b.num_kv_heads,
                       head_size=b.head_size, num_blocks=b.num_blocks,
                       block_size=b.block_size, max_blocks_per_seq=b.max_blocks_per_seq,
                       dtype=A.ATTN_BF16, partition_tokens=partition_tokens)
    assert A.attn_check_cascade_host(desc, b.block_table, b.query_start_loc, b.seq_lens,
                                     prefix) == A.ATTN_OK
    out = torch.empty_like(q)
    lse = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device=q.device)
    n = A.attn_cascade_workspace_bytes(desc, prefix)
    ws = torch.empty(n, dtype=torch.uint8, device=q.device) if n else None
    A.attn_cascade_fwd(desc, q, kv, bt, qsl, sl, prefix, b.scale, causal, out, lse, ws)
    return out, lse


def _batch(seed, *, ql, cl, hq, hkv, d, bs, prefix_blocks):
    ql = np.asarray(ql)
    return gen.make_batch(f"cascade{seed}", num_heads=hq, num_kv_heads=hkv, head_size=d,
                          block_size=bs, dtype="bf16", query_lens=ql,
                          seq_lens=ql + np.asarray(cl), passes=[(True, 0)], seed=seed,
                          pool_factor=2, shared_prefix_blocks=prefix_blocks)


CASES = [
    # name, batch kwargs, partition_tokens
    ("mixed-d128-gqa8-bs16", dict(ql=[1, 1, 1, 40, 300], cl=[48, 700, 1499, 48, 1000], hq=16,
                                  hkv=2, d=128, bs=16, prefix_blocks=3), 0),
    ("prefill-d64-mha-bs32", dict(ql=[300, 77, 257], cl=[64, 200, 500], hq=4, hkv=4, d=64,
                                  bs=32, prefix_blocks=2), 0),
    ("decode-d128-gqa4-bs64-pt128", dict(ql=[1] * 6, cl=[256, 300, 700, 1024, 2000, 257],
                                         hq=8, hkv=2, d=128, bs=64, prefix_blocks=4), 128),
    ("mixed-d64-gqa20-bs64", dict(ql=[1, 1, 600, 129], cl=[1100, 1024, 1024, 3000], hq=40,
                                  hkv=2, d=64, bs=64, prefix_blocks=16), 0),
    # few query rows and a long prefix: the prefix pass splits its keys into 8 slices
    ("decode-d128-gqa8-bs64-8slices", dict(ql=[1] * 6 + [50],
                                           cl=[4096, 4200, 5000, 4097, 6000, 4500, 4096],
                                           hq=16, hkv=2, d=128, bs=64, prefix_blocks=64), 0),
]


@pytest.mark.parametrize("name,kw,pt", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
def test_cascade_matches_oracle(name, kw, pt, causal):
    seed = 40 + [c[0] for c in CASES].index(name)
    b = _batch(seed, **kw)
    prefix = kw["prefix_blocks"] * kw["bs"]
    print(f"[case] cascade {name} causal={causal} prefix={prefix}", flush=True)
    q, kv = gen.make_tensors(b, seed, DEV, poison=True)
    out, lse = run_cascade(b, q, kv, causal, prefix, pt)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_on(b, q, kv, causal, 0)
    print(compare(out, lse, ref_out, ref_lse, label=name))
    # the cascade oracle (the pages' three steps) agrees with the same reference
    c_out, c_lse = oracle.cascade_attention(host_f32(q), host_f32(kv), b.block_table,
                                            b.query_start_loc, b.seq_lens, b.scale, causal,
                                            prefix)
    np.testing.assert_allclose(c_out, ref_out, rtol=0, atol=1e-10)
    np.testing.assert_allclose(c_lse, ref_lse, rtol=0, atol=1e-10)


def test_cascade_without_prefix_is_the_plain_call():
    name, kw, pt = CASES[0]
    b = _batch(40, **kw)
    q, kv = gen.make_tensors(b, 40, DEV, poison=True)
    out, lse = run_cascade(b, q, kv, True, 0)
    out2, lse2 = run_library(b, q, kv, True, 0)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_workload5_cascade_sampled_parity():
    """Mixed long-context workload, layer pass 0 (causal), cascade over its 2048-token
    shared prefix, at full size; compared on sampled requests and rows."""
    b = gen.config(5)
    causal, window = b.passes[0]
    assert window == 0
    prefix = b.shared_prefix_blocks * b.block_size
    print(f"[case] mixed long-context cascade prefix={prefix}", flush=True)
    q, kv = gen.make_tensors(b, 5, DEV, layer=0)
    out, lse = run_cascade(b, q, kv, causal, prefix)
    torch.cuda.synchronize()
    dec = np.argsort(b.seq_lens[:120])
    req = sorted(set(dec[:4].tolist() + dec[-4:].tolist() + [17, 60, 99])) + list(range(120, 128))
    sub, qs, kvs = gen.subset(b, req, q, kv)
    rows_sub, rows_full = [], []
    for i, r in enumerate(req):
        ql = int(b.query_lens[r])
        pick = np.unique(np.concatenate([[0, ql - 1], np.linspace(0, ql - 1, 12).astype(int)]))
        rows_sub.extend(sub.query_start_loc[i] + pick)
        rows_full.extend(b.query_start_loc[r] + pick)
    ref_out, ref_lse = oracle_on(sub, qs, kvs, causal, 0, rows=rows_sub)
    idx = torch.as_tensor(rows_full, device=out.device)
    print(compare(out[idx], lse[idx], ref_out[rows_sub], ref_lse[rows_sub], label="mixed long-context cascade"))
