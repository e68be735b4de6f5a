"""Shared helpers of the GPU tests: run one batch through the library, run the oracle on the
very same inputs (copied back to the host), and compare to the stated tolerances."""
import numpy as np
import torch

import exact_softmax_attention_paged_amd as A
import gen
import oracle

# Tolerances against the fp64 oracle on bf16 inputs with fp32 accumulation.
OUT_MAX_ERR = 2e-2
OUT_MEAN_ERR = 2e-3
LSE_MAX_ERR = 1e-3


def device_meta(batch, device="cuda"):
    return (torch.from_numpy(batch.block_table).to(device),
            torch.from_numpy(batch.query_start_loc).to(device),
            torch.from_numpy(batch.seq_lens).to(device))


def run_library(batch, q, kv, causal, window, *, num_decodes=None, partition_tokens=0,
                meta=None, stream=None):
    bt, qsl, sl = meta if meta is not None else device_meta(batch, q.device)
    nd = batch.num_decodes if num_decodes is None else num_decodes
    if stream is None:
        return A.varlen_fwd(q, kv, bt, qsl, sl, scale=batch.scale, causal=causal, window=window,
                            num_decodes=nd, max_query_len=batch.max_query_len,
                            max_seq_len=batch.max_seq_len, partition_tokens=partition_tokens)
    with torch.cuda.stream(stream):
        return A.varlen_fwd(q, kv, bt, qsl, sl, scale=batch.scale, causal=causal, window=window,
                            num_decodes=nd, max_query_len=batch.max_query_len,
                            max_seq_len=batch.max_seq_len, partition_tokens=partition_tokens)


def host_f32(t) -> np.ndarray:
    """Exact host copy of a bf16/f32 tensor as float32 (the oracle upcasts to float64)."""
    return t.detach().to("cpu", torch.float32).numpy()


def oracle_on(batch, q, kv, causal, window, rows=None):
    """Oracle output for ``batch`` given host or device tensors (copied to the host)."""
    return oracle.attention(host_f32(q), host_f32(kv), batch.block_table,
                            batch.query_start_loc, batch.seq_lens, batch.scale, causal, window,
                            rows=rows)


def compare(out, lse, ref_out, ref_lse, rows=None, label=""):
    """Element-wise comparison on ``rows`` (all rows if None). Returns the error summary."""
    o = gen.to_numpy_f64(out)
    l = gen.to_numpy_f64(lse) if lse is not None else None
    if rows is not None:
        rows = np.asarray(rows)
        o, ref_out = o[rows], ref_out[rows]
        if l is not None:
            l, ref_lse = l[rows], ref_lse[rows]
    assert np.all(np.isfinite(ref_out)), "oracle left rows uncomputed"
    assert np.all(np.isfinite(o)), f"{label}: non-finite output"
    err = np.abs(o - ref_out)
    res = {"out_max": float(err.max()) if err.size else 0.0,
           "out_mean": float(err.mean()) if err.size else 0.0}
    if l is not None:
        both_inf = np.isneginf(l) & np.isneginf(ref_lse)
        lerr = np.where(both_inf, 0.0, np.abs(l - ref_lse))
        res["lse_max"] = float(lerr.max()) if lerr.size else 0.0
    assert res["out_max"] <= OUT_MAX_ERR, f"{label}: {res}"
    assert res["out_mean"] <= OUT_MEAN_ERR, f"{label}: {res}"
    if l is not None:
        assert res["lse_max"] <= LSE_MAX_ERR, f"{label}: {res}"
    return res
