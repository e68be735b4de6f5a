"""attn_varlen_fwd_noalloc (the entry point for callers that cannot allocate) against
attn_varlen_fwd with a torch-allocated workspace: two calls in a row through the C ABI, the
second with a smaller batch, each bitwise equal to the workspace entry point's result on the
same inputs (both run the same kernels), and the first also within the oracle tolerances."""
import numpy as np
import pytest
import torch

import exact_softmax_attention_paged_amd as A
import gen
from parity import compare, device_meta, oracle_on

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _desc(b, partition_tokens):
    return A.make_desc(num_seqs=b.num_seqs, num_tokens=b.num_tokens, num_decodes=b.num_decodes,
                       max_query_len=b.max_query_len, max_seq_len=b.max_seq_len,
                       num_heads=b.num_heads, num_kv_heads=b.num_kv_heads,
                       head_size=b.head_size, num_blocks=b.num_blocks,
                       block_size=b.block_size, max_blocks_per_seq=b.max_blocks_per_seq,
                       dtype=A.ATTN_BF16, partition_tokens=partition_tokens)


def _both(b, seed, causal, window, partition_tokens):
    q, kv = gen.make_tensors(b, seed, DEV, poison=True)
    bt, qsl, sl = device_meta(b, DEV)
    desc = _desc(b, partition_tokens)
    out_ws, out_na = torch.empty_like(q), torch.empty_like(q)
    lse_ws = torch.empty(b.num_tokens, b.num_heads, dtype=torch.float32, device=DEV)
    lse_na = torch.empty_like(lse_ws)
    ws = torch.empty(max(A.attn_workspace_bytes(desc), 1), dtype=torch.uint8, device=DEV)
    A.attn_varlen_fwd(desc, q, kv, bt, qsl, sl, b.scale, causal, window, out_ws, lse_ws, ws)
    A.attn_varlen_fwd_noalloc(desc, q, kv, bt, qsl, sl, b.scale, causal, window, out_na, lse_na)
    torch.cuda.synchronize()
    return q, kv, out_ws, lse_ws, out_na, lse_na


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 700)], ids=["causal", "w700"])
def test_noalloc_matches_workspace_entry_point(causal, window):
    big = gen.make_batch("noalloc-big", num_heads=32, num_kv_heads=8, head_size=128,
                         block_size=16, dtype="bf16",
                         query_lens=[1] * 40 + [300, 77],
                         seq_lens=np.random.default_rng(41).integers(1, 9000, 40).tolist()
                         + [2000, 500], passes=[(causal, window)], seed=41, pool_factor=2)
    small = gen.make_batch("noalloc-small", num_heads=32, num_kv_heads=8, head_size=128,
                           block_size=16, dtype="bf16", query_lens=[1, 1, 1, 20],
                           seq_lens=[3000, 17, 600, 40], passes=[(causal, window)], seed=42,
                           pool_factor=2)
    print(f"[case] noalloc causal={causal} window={window}: big batch", flush=True)
    q, kv, o_ws, l_ws, o_na, l_na = _both(big, 41, causal, window, 512)
    assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16))
    assert torch.equal(l_ws, l_na)
    ref_out, ref_lse = oracle_on(big, q, kv, causal, window)
    compare(o_na, l_na, ref_out, ref_lse, label="noalloc big")
    print(f"[case] noalloc causal={causal} window={window}: smaller batch", flush=True)
    q, kv, o_ws, l_ws, o_na, l_na = _both(small, 42, causal, window, 0)
    assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16))
    assert torch.equal(l_ws, l_na)
    ref_out, ref_lse = oracle_on(small, q, kv, causal, window)
    compare(o_na, l_na, ref_out, ref_lse, label="noalloc small")


def test_noalloc_refuses_a_batch_beyond_its_array():
    """A decode batch whose partial results exceed the fixed array is refused before any
    launch (the binding raises AttnError with ATTN_ERR_WORKSPACE); its outputs stay untouched."""
    b = gen.make_batch("noalloc-too-big", num_heads=8, num_kv_heads=8, head_size=128,
                       block_size=16, dtype="bf16", query_lens=[1] * 512,
                       seq_lens=[16384] + [16] * 511, passes=[(True, 0)], seed=43)
    desc = _desc(b, 128)
    assert A.attn_workspace_bytes(desc) > A.NOALLOC_SCRATCH_BYTES
    bt, qsl, sl = device_meta(b, DEV)
    q = torch.zeros(b.num_tokens, 8, 128, dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros(2, b.num_blocks, 16, 8, 128, dtype=torch.bfloat16, device=DEV)
    out = torch.full_like(q, 3.0)
    with pytest.raises(A.AttnError) as e:
        A.attn_varlen_fwd_noalloc(desc, q, kv, bt, qsl, sl, b.scale, True, 0, out, None)
    assert e.value.status == A.ATTN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
