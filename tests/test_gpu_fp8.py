"""Parity of the E4M3 (FP8) KV-cache paths with the CPU oracle: the quantising cache write is
bit-exact against the oracle's quantizer (same fp32 quotient, ties to even, saturation), and
decode over an E4M3 cache matches the oracle's attention over the dequantised cache to the
bf16 tolerances. Unreadable slots hold the NaN code, so a stray read would show."""
import numpy as np
import pytest
import torch

import exact_softmax_attention_paged_amd as A
import gen
import oracle
from parity import compare, device_meta, host_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"
# random codes span the whole E4M3 range (|code value| <= 448); these scales keep the
# dequantised K and V within +-3.6, the magnitude range the bf16 tolerances are stated for
K_SCALE, V_SCALE = 0.008, 0.008


def _desc(b, num_tokens=None):
    return A.make_desc(num_seqs=b.num_seqs, num_tokens=b.num_tokens if num_tokens is None
                       else num_tokens, num_decodes=b.num_decodes, max_query_len=b.max_query_len,
                       max_seq_len=b.max_seq_len, num_heads=b.num_heads,
                       num_kv_heads=b.num_kv_heads, head_size=b.head_size,
                       num_blocks=b.num_blocks, block_size=b.block_size,
                       max_blocks_per_seq=b.max_blocks_per_seq, dtype=A.ATTN_BF16)


def fp8_cache(b, seed):
    """A seeded E4M3 cache: uniformly random finite codes (every exponent, subnormals and
    both signs occur), the NaN code in every slot no request may read."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(2, b.num_blocks, b.block_size, b.num_kv_heads,
                                       b.head_size), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00
    codes[:, ~gen.readable_mask(b)] = 0x7F
    return codes


def run_fp8_decode(b, q, codes_dev, window, ks=K_SCALE, vs=V_SCALE, partition_tokens=0):
    bt, qsl, sl = device_meta(b, DEV)
    desc = _desc(b)
    desc.partition_tokens = partition_tokens
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=DEV)
    n = A.attn_fp8_decode_workspace_bytes(desc)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
    A.attn_fp8_decode_fwd(desc, q, codes_dev, bt, qsl, sl, b.scale, ks, vs, window, out, lse, ws)
    return out, lse


DECODE = [
    ("d128-gqa8-bs16", dict(sl=[1, 17, 700, 1500, 4097], hq=16, hkv=2, d=128, bs=16)),
    ("d64-gqa20-bs64", dict(sl=[513, 2000, 64], hq=40, hkv=2, d=64, bs=64)),
    ("d128-mha-bs32", dict(sl=[33, 1025, 300], hq=4, hkv=4, d=128, bs=32)),
    ("d128-gqa4-bs48", dict(sl=[47, 49, 1000, 3000], hq=8, hkv=2, d=128, bs=48)),
]


@pytest.mark.parametrize("name,kw", DECODE, ids=[c[0] for c in DECODE])
@pytest.mark.parametrize("window,pt", [(0, 0), (0, 128), (100, 0), (1000, 256)],
                         ids=["full", "pt128", "w100", "w1000-pt256"])
def test_fp8_decode_matches_oracle(name, kw, window, pt):
    seed = 60 + [c[0] for c in DECODE].index(name)
    b = gen.make_batch(f"fp8{seed}", num_heads=kw["hq"], num_kv_heads=kw["hkv"],
                       head_size=kw["d"], block_size=kw["bs"], dtype="bf16",
                       query_lens=[1] * len(kw["sl"]), seq_lens=kw["sl"], passes=[(True, 0)],
                       seed=seed, pool_factor=2)
    print(f"[case] fp8 decode {name} window={window} partition={pt}", flush=True)
    codes = fp8_cache(b, seed)
    q = gen.make_q(b, seed, DEV)
    out, lse = run_fp8_decode(b, q, torch.from_numpy(codes).to(DEV), window, partition_tokens=pt)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.attention_fp8_kv(host_f32(q), codes, K_SCALE, V_SCALE,
                                               b.block_table, b.query_start_loc, b.seq_lens,
                                               b.scale, True, window)
    print(compare(out, lse, ref_out, ref_lse, label=name))


@pytest.mark.parametrize("pt", [512, 0], ids=["pt512", "default"])
def test_fp8_decode_workload4_shape_sampled(pt):
    """The paged GQA decode workload's shape (256 requests, contexts U[512, 8192], 32 q / 8 kv
    heads, d 128, block 16) over an E4M3 cache, checked on sampled requests, at the workload's
    512-key partitions and at the E4M3 default (1024 keys here)."""
    b = gen.config(4)
    print(f"[case] fp8 decode, paged GQA decode shape, partition {pt}", flush=True)
    codes = fp8_cache(b, 4)
    q = gen.make_q(b, 4, DEV)
    out, lse = run_fp8_decode(b, q, torch.from_numpy(codes).to(DEV), 0, partition_tokens=pt)
    torch.cuda.synchronize()
    order = np.argsort(b.seq_lens)
    req = sorted(set(order[:6].tolist() + order[-6:].tolist() + [3, 100, 200]))
    sub, qs, cs = gen.subset(b, req, q, torch.from_numpy(codes))   # only the sampled requests
    ref_out, ref_lse = oracle.attention_fp8_kv(host_f32(qs), cs.numpy(), K_SCALE, V_SCALE,
                                               sub.block_table, sub.query_start_loc,
                                               sub.seq_lens, b.scale, True, 0)
    rows = torch.as_tensor(req, device=DEV)           # decode rows: token index = request
    print(compare(out[rows], lse[rows], ref_out, ref_lse, label="paged GQA decode fp8"))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("scales", [(1.0, 1.0), (0.0125, 0.02), (0.37, 3.0)],
                         ids=["s1", "s-small", "s-mixed"])
def test_fp8_write_is_bit_exact(d, scales):
    ks, vs = scales
    hq, hkv, bs, nb, T = 8, 4, 16, 50, 400
    print(f"[case] fp8 write d={d} scales={scales}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(d)
    # magnitudes from the subnormal range to beyond saturation
    mag = torch.pow(10.0, torch.empty(T, (hq + 2 * hkv) * d).uniform_(-4, 3, generator=g))
    sign = torch.where(torch.rand(T, (hq + 2 * hkv) * d, generator=g) < 0.5, -1.0, 1.0)
    qkv = (mag * sign).to(torch.bfloat16).to(DEV)
    key = qkv[:, hq * d:(hq + hkv) * d].view(T, hkv, d)
    val = qkv[:, (hq + hkv) * d:].view(T, hkv, d)
    slots = np.random.default_rng(d).permutation(nb * bs)[:T].astype(np.int64)
    slots[::9] = -1
    cache = torch.full((2, nb, bs, hkv, d), 0x7F, dtype=torch.uint8, device=DEV)
    desc = A.make_desc(num_seqs=1, num_tokens=T, num_decodes=0, max_query_len=1, max_seq_len=bs,
                       num_heads=hkv, num_kv_heads=hkv, head_size=d, num_blocks=nb,
                       block_size=bs, max_blocks_per_seq=1, dtype=A.ATTN_BF16)
    A.attn_kv_cache_write_fp8(desc, key, val, torch.from_numpy(slots).to(DEV), ks, vs, cache)
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    ref = np.full_like(got, 0x7F)
    kf, vf = host_f32(key), host_f32(val)
    for t, s in enumerate(slots):
        if s >= 0:
            ref[0, s // bs, s % bs] = oracle.e4m3_quantize(kf[t], ks)
            ref[1, s // bs, s % bs] = oracle.e4m3_quantize(vf[t], vs)
    assert np.array_equal(got, ref), f"{(got != ref).sum()} codes differ"


def test_fp8_write_then_decode():
    """Layer step over an E4M3 cache: the decode tokens' K/V are quantised into the cache
    through slot_mapping, then decode reads them; against the oracle's quantizer + attention."""
    b = gen.make_batch("fp8step", num_heads=32, num_kv_heads=8, head_size=128, block_size=16,
                       dtype="bf16", query_lens=[1] * 6, seq_lens=[1, 40, 300, 1023, 2048, 77],
                       passes=[(True, 0)], seed=71, pool_factor=2)
    print("[case] fp8 write then decode", flush=True)
    codes = fp8_cache(b, 71)
    q = gen.make_q(b, 71, DEV)
    g = torch.Generator(device="cpu").manual_seed(5)
    key = torch.randn(6, 8, 128, generator=g).to(torch.bfloat16)
    val = torch.randn(6, 8, 128, generator=g).to(torch.bfloat16)
    bs = b.block_size
    slots = np.array([int(b.block_table[r, (s - 1) // bs]) * bs + (s - 1) % bs
                      for r, s in enumerate(b.seq_lens)], np.int64)
    cache = torch.from_numpy(codes).to(DEV)
    A.attn_kv_cache_write_fp8(_desc(b), key.to(DEV), val.to(DEV), torch.from_numpy(slots).to(DEV),
                              K_SCALE, V_SCALE, cache)
    out, lse = run_fp8_decode(b, q, cache, 0)
    torch.cuda.synchronize()
    ref_codes = codes.copy()
    for t, s in enumerate(slots):
        ref_codes[0, s // bs, s % bs] = oracle.e4m3_quantize(key[t].float().numpy(), K_SCALE)
        ref_codes[1, s // bs, s % bs] = oracle.e4m3_quantize(val[t].float().numpy(), V_SCALE)
    assert np.array_equal(cache.cpu().numpy(), ref_codes)
    ref_out, ref_lse = oracle.attention_fp8_kv(host_f32(q), ref_codes, K_SCALE, V_SCALE,
                                               b.block_table, b.query_start_loc, b.seq_lens,
                                               b.scale, True)
    print(compare(out, lse, ref_out, ref_lse, label="fp8 write+decode"))
