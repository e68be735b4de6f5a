"""Invariances of the HIP path that hold without any reference to the oracle.

The definition of the attention does not depend on where a request's blocks sit in the pool,
on the block size, on whether kv heads are shared by several q heads, on which run computes it,
or on how the keys of a decode row are cut into split-KV partitions. The first four leave the
arithmetic of every kernel unchanged (the same values reach the same instructions in the same
order), so the outputs must be bitwise equal; the partitioning changes the order in which fp32
partial results are combined, so those outputs must agree to within the rounding that
reordering can cause. Sources: the paged layout and the block table of the FlashAttentionBackend
and FlashAttentionMetadata sections and num_queries_per_kv of the FlashAttentionImpl section of
the vLLM FlashAttention page; the partition merge of the Overview of the RBLN "Attention 모드"
page.
"""
import numpy as np
import pytest
import torch

import exact_softmax_attention_paged_amd as A
import gen
from parity import compare, device_meta, oracle_on, run_library

pytestmark = pytest.mark.gpu
DEV = "cuda"
MASKS = [(False, 0), (True, 0), (True, 100)]
MASK_IDS = ["noncausal", "causal", "w100"]


def _mixed(seed, hq=16, hkv=4, d=128, bs=16):
    """Decode rows first, then prefill rows of several 256-row tiles with ragged ends."""
    return gen.make_batch(f"inv{seed}", num_heads=hq, num_kv_heads=hkv, head_size=d,
                          block_size=bs, dtype="bf16",
                          query_lens=[1, 1, 1, 300, 37, 600],
                          seq_lens=[2500, 130, 4100, 900, 37, 1700], passes=[(True, 0)],
                          seed=seed, pool_factor=2)


def _equal(a, b):
    """Bitwise equality of two output tensors (NaN never appears: the inputs are finite on
    every readable slot)."""
    return bool(torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                            b.view(torch.int16) if b.dtype == torch.bfloat16 else b))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,window", MASKS, ids=MASK_IDS)
def test_block_table_permutation_is_bitwise_invariant(d, causal, window):
    """Moving every block of the pool to another slot, with the block table rewritten to
    match, leaves every output and lse bit unchanged."""
    b = _mixed(31, d=d)
    print(f"[case] block permutation d={d} causal={causal} window={window}", flush=True)
    q, kv = gen.make_tensors(b, 31, DEV, poison=True)
    out0, lse0 = run_library(b, q, kv, causal, window, partition_tokens=512)
    perm = np.random.default_rng(7).permutation(b.num_blocks)        # new slot of block i
    kv2 = torch.empty_like(kv)
    kv2[:, torch.from_numpy(perm).to(DEV)] = kv
    b2 = gen.Batch(**{**b.__dict__, "block_table": perm[b.block_table].astype(np.int32),
                      "pad_block": int(perm[b.pad_block])})
    out1, lse1 = run_library(b2, q, kv2, causal, window, partition_tokens=512)
    torch.cuda.synchronize()
    assert _equal(out0, out1) and _equal(lse0, lse1)


@pytest.mark.parametrize("causal,window", MASKS, ids=MASK_IDS)
def test_paged_equals_one_block_per_request_bitwise(causal, window):
    """The paged batch (block size 16, shuffled pool) against its twin with one block per
    request (block size = the longest sequence rounded up to 16): bitwise equal."""
    b = _mixed(32)
    print(f"[case] paged vs contiguous causal={causal} window={window}", flush=True)
    q, kv = gen.make_tensors(b, 32, DEV, poison=True)
    twin, kvc = gen.contiguous_twin(b, kv)
    out0, lse0 = run_library(b, q, kv, causal, window, partition_tokens=512)
    out1, lse1 = run_library(twin, q, kvc, causal, window, partition_tokens=512)
    torch.cuda.synchronize()
    assert _equal(out0, out1) and _equal(lse0, lse1)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,window", MASKS, ids=MASK_IDS)
def test_gqa_equals_mha_with_repeated_kv_heads_bitwise(d, causal, window):
    """GQA with 4 q heads per kv head against MHA over the kv heads repeated 4 times (kv head
    k serves q heads 4k .. 4k+3): bitwise equal, decode and prefill rows alike. The partition
    length is fixed (the library default depends on the number of kv heads)."""
    b = _mixed(33, hq=16, hkv=4, d=d)
    print(f"[case] GQA vs MHA d={d} causal={causal} window={window}", flush=True)
    q, kv = gen.make_tensors(b, 33, DEV, poison=True)
    out0, lse0 = run_library(b, q, kv, causal, window, partition_tokens=1024)
    kv_rep = kv.repeat_interleave(4, dim=3).contiguous()
    b2 = gen.Batch(**{**b.__dict__, "num_kv_heads": 16})
    out1, lse1 = run_library(b2, q, kv_rep, causal, window, partition_tokens=1024)
    torch.cuda.synchronize()
    assert _equal(out0, out1) and _equal(lse0, lse1)


@pytest.mark.parametrize("causal,window", MASKS, ids=MASK_IDS)
def test_two_eager_calls_are_bitwise_equal(causal, window):
    """Run-to-run determinism: the decode schedule's order among equal-cost items may differ
    between calls, but every result is combined in a fixed order."""
    b = _mixed(34)
    q, kv = gen.make_tensors(b, 34, DEV, poison=True)
    out0, lse0 = run_library(b, q, kv, causal, window)
    out1, lse1 = run_library(b, q, kv, causal, window)
    torch.cuda.synchronize()
    assert _equal(out0, out1) and _equal(lse0, lse1)


# The tolerance of the partition comparisons. Each result rounds its probabilities to bf16
# against its own running maximum (that of a partition, of a wave's share of it, or of the whole
# row) before the P.V product, so a weight may carry a different rounding (up to 2^-9 relative)
# in the two results; a split row also stores each partition's normalised result in bf16
# before the merge (at most 2^-9 of that partition result's magnitude, and the merge weights
# sum to 1); and the final bf16 rounding of two nearby fp32 values may differ by one unit
# (2^-8 relative). On this batch that is at most one bf16 unit of an output below 0.25 (2^-10)
# and a mean of 3-7e-5 on every partition length (measured on gfx950); the bounds below leave
# 3-4x margin on each. The lse is formed in fp32 from the same scores on both sides (only
# the order of the partial sums and the reference maxima differ): measured 1-2e-6, bound 1e-5.
PART_OUT_MAX, PART_OUT_MEAN, PART_LSE_MAX = 4e-3, 2e-4, 1e-5


def _close(a, b, la, lb, label):
    err = (a.float() - b.float()).abs()
    both_inf = torch.isneginf(la) & torch.isneginf(lb)
    lerr = torch.where(both_inf, torch.zeros_like(la), (la - lb).abs())
    res = {"out_max": err.max().item(), "out_mean": err.mean().item(),
           "lse_max": lerr.max().item()}
    print(label, res, flush=True)
    assert res["out_max"] <= PART_OUT_MAX and res["out_mean"] <= PART_OUT_MEAN and \
        res["lse_max"] <= PART_LSE_MAX, (label, res)


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 3000)], ids=["causal", "w3000"])
def test_decode_partition_length_invariance(causal, window):
    """Decode rows split into 128-, 512-, 2048- and 16384-key partitions agree with each other
    (and with the prefill kernel's unsplit walk over the same rows, num_decodes = 0) to within
    the reordering tolerance above; each also meets the oracle tolerances."""
    rng = np.random.default_rng(35)
    sl = rng.integers(1, 20000, size=24).tolist()
    b = gen.make_batch("partitions", num_heads=32, num_kv_heads=8, head_size=128,
                       block_size=16, dtype="bf16", query_lens=[1] * 24, seq_lens=sl,
                       passes=[(causal, window)], seed=35, pool_factor=2)
    q, kv = gen.make_tensors(b, 35, DEV, poison=True)
    res = {}
    for pt in (128, 512, 2048, 16384):
        res[pt] = run_library(b, q, kv, causal, window, partition_tokens=pt)
    res["prefill-kernel"] = run_library(b, q, kv, causal, window, num_decodes=0)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_on(b, q, kv, causal, window)
    base_out, base_lse = res[512]
    for key, (o, l) in res.items():
        compare(o, l, ref_out, ref_lse, label=f"partition {key}")
        if key != 512:
            _close(o, base_out, l, base_lse, f"partition {key} vs 512")


def test_binding_rejects_wrong_metadata_shapes():
    """The kernels index block_table, query_start_loc, seq_lens and lse by the descriptor's
    sizes; the binding refuses arrays of other sizes before anything is queued."""
    b = _mixed(36)
    q, kv = gen.make_tensors(b, 36, DEV)
    bt, qsl, sl = device_meta(b, DEV)
    desc = A.make_desc(num_seqs=b.num_seqs, num_tokens=b.num_tokens, num_decodes=b.num_decodes,
                       max_query_len=b.max_query_len, max_seq_len=b.max_seq_len,
                       num_heads=b.num_heads, num_kv_heads=b.num_kv_heads,
                       head_size=b.head_size, num_blocks=b.num_blocks,
                       block_size=b.block_size, max_blocks_per_seq=b.max_blocks_per_seq,
                       dtype=A.ATTN_BF16)
    ws = torch.empty(A.attn_workspace_bytes(desc), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty(b.num_tokens, b.num_heads, dtype=torch.float32, device=DEV)
    bad = {
        "block_table rows": dict(block_table=bt[:-1].contiguous()),
        "block_table columns": dict(block_table=bt[:, :-1].contiguous()),
        "query_start_loc": dict(query_start_loc=qsl[:-1].contiguous()),
        "seq_lens": dict(seq_lens=sl[:-1].contiguous()),
        "lse rows": dict(lse=lse[:-1]),
        "lse heads": dict(lse=torch.empty(b.num_tokens, b.num_heads - 1, dtype=torch.float32,
                                          device=DEV)),
    }
    for what, kw in bad.items():
        args = dict(block_table=bt, query_start_loc=qsl, seq_lens=sl, lse=lse)
        args.update(kw)
        with pytest.raises(ValueError):
            A.attn_varlen_fwd(desc, q, kv, args["block_table"], args["query_start_loc"],
                              args["seq_lens"], b.scale, True, 0, out, args["lse"], ws)
        print("refused:", what, flush=True)
    A.attn_varlen_fwd(desc, q, kv, bt, qsl, sl, b.scale, True, 0, out, lse, ws)
    torch.cuda.synchronize()
