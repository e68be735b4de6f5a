"""Capture safety: a forward call recorded into a HIP graph (torch.cuda.CUDAGraph) replays to
the same results as the eager call. The call covers every kernel of a mixed batch: the decode
work schedule, the split-KV decode, the LSE merge and the prefill kernel; the library makes no
allocation, host synchronisation or memset inside the call. Each replay follows eager work of
its own on the same stream and is checked bit for bit against the eager result and, once,
against the oracle."""
import pytest
import torch

import exact_softmax_attention_paged_amd as A
import gen
from parity import compare, device_meta, oracle_on

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("window", [0, 700], ids=["causal", "w700"])
def test_graph_replays_match_the_eager_call(window):
    print(f"[case] graph capture window={window}", flush=True)
    b = gen.make_batch("graph", num_heads=16, num_kv_heads=4, head_size=128, block_size=16,
                       dtype="bf16", query_lens=[1, 1, 1, 300, 777],
                       seq_lens=[5000, 64, 9000, 1200, 777], passes=[(True, window)], seed=61,
                       pool_factor=2)
    q, kv = gen.make_tensors(b, 61, DEV, poison=True)
    bt, qsl, sl = device_meta(b, DEV)
    desc = A.make_desc(num_seqs=b.num_seqs, num_tokens=b.num_tokens, num_decodes=b.num_decodes,
                       max_query_len=b.max_query_len, max_seq_len=b.max_seq_len,
                       num_heads=16, num_kv_heads=4, head_size=128, num_blocks=b.num_blocks,
                       block_size=16, max_blocks_per_seq=b.max_blocks_per_seq,
                       dtype=A.ATTN_BF16, partition_tokens=1024)
    ws = torch.empty(A.attn_workspace_bytes(desc), dtype=torch.uint8, device=DEV)
    out_e = torch.empty_like(q)
    lse_e = torch.empty(b.num_tokens, 16, dtype=torch.float32, device=DEV)
    A.attn_varlen_fwd(desc, q, kv, bt, qsl, sl, b.scale, True, window, out_e, lse_e, ws)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_on(b, q, kv, True, window)
    compare(out_e, lse_e, ref_out, ref_lse, label="eager")

    out_g = torch.empty_like(q)
    lse_g = torch.empty_like(lse_e)
    side = torch.cuda.Stream()                  # warm up on a side stream, as torch advises
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        A.attn_varlen_fwd(desc, q, kv, bt, qsl, sl, b.scale, True, window, out_g, lse_g, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        A.attn_varlen_fwd(desc, q, kv, bt, qsl, sl, b.scale, True, window, out_g, lse_g, ws)
    x = torch.randn(512, 512, device=DEV)
    for rep in range(4):
        out_g.fill_(float("nan"))               # eager work between the replays
        lse_g.fill_(float("nan"))
        ws.fill_(0xAB)
        x = torch.tanh(x @ x.t() / 512)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {rep}: out differs from the eager call"
        assert torch.equal(lse_g, lse_e), f"replay {rep}: lse differs from the eager call"
