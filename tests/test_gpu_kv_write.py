"""Parity of the KV-cache write (attn_kv_cache_write) with the CPU oracle: bit-exact, since
the step only moves bytes. Covers bf16 and f32, both head sizes, padding slots, slots past
the cache (skipped), keys and values read as strided column slices of a packed QKV tensor,
NaN in every slot the call must not touch, a full-size write of the mixed workload's shape,
and the layer step: write the new tokens, then attention over the cache."""
import numpy as np
import pytest
import torch

import exact_softmax_attention_paged_amd as A
import gen
import oracle
from parity import compare, device_meta, host_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _desc(num_tokens, hkv, d, num_blocks, bs, dtype):
    return A.make_desc(num_seqs=1, num_tokens=num_tokens, num_decodes=0, max_query_len=1,
                       max_seq_len=bs, num_heads=hkv, num_kv_heads=hkv, head_size=d,
                       num_blocks=num_blocks, block_size=bs, max_blocks_per_seq=1,
                       dtype=A.ATTN_BF16 if dtype == torch.bfloat16 else A.ATTN_F32)


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("packed", [False, True], ids=["separate", "packed-qkv"])
def test_write_is_bit_exact(dtype, d, packed):
    hq, hkv, bs, nb, T = 12, 4, 32, 40, 300
    print(f"[case] kv write dtype={dtype} d={d} packed={packed}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(d + (7 if packed else 0))
    cache = torch.full((2, nb, bs, hkv, d), float("nan"), dtype=dtype, device=DEV)
    rng = np.random.default_rng(d)
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    slots[::17] = -1                                      # padding tokens
    slots[5] = nb * bs + 3                                # past the cache: skipped
    if packed:
        qkv = torch.randn(T, (hq + 2 * hkv) * d, generator=g).to(dtype).to(DEV)
        key = qkv[:, hq * d:(hq + hkv) * d].view(T, hkv, d)
        val = qkv[:, (hq + hkv) * d:].view(T, hkv, d)
    else:
        key = torch.randn(T, hkv, d, generator=g).to(dtype).to(DEV)
        val = torch.randn(T, hkv, d, generator=g).to(dtype).to(DEV)
    ref = oracle.kv_cache_write(host_f32(cache), host_f32(key), host_f32(val),
                                np.where(slots < nb * bs, slots, -1))
    A.attn_kv_cache_write(_desc(T, hkv, d, nb, bs, dtype), key, val,
                          torch.from_numpy(slots).to(DEV), cache)
    torch.cuda.synchronize()
    got = host_f32(cache)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), f"{(~same).sum()} elements differ"
    # untouched slots keep their exact bytes (NaN payload included)
    before = torch.full_like(cache, float("nan"))
    untouched = np.ones((nb * bs,), bool)
    untouched[slots[(slots >= 0) & (slots < nb * bs)]] = False
    b_bits = _bits(before).reshape(2, nb * bs, -1)[:, untouched]
    c_bits = _bits(cache).reshape(2, nb * bs, -1)[:, untouched]
    assert np.array_equal(b_bits, c_bits)


def test_full_size_write_of_the_mixed_workload_shape():
    """16504 new tokens (the mixed workload's query rows), 8 kv heads, d 128, bf16, into a
    cache of its size (32.9K blocks of 64 slots), random distinct slots."""
    b = gen.config(5)
    T, hkv, d, bs, nb = b.num_tokens, b.num_kv_heads, b.head_size, b.block_size, b.num_blocks
    print(f"[case] full-size kv write T={T} blocks={nb}", flush=True)
    cache = torch.zeros((2, nb, bs, hkv, d), dtype=torch.bfloat16, device=DEV)
    slots = np.random.default_rng(1).permutation(nb * bs)[:T].astype(np.int64)
    g = torch.Generator(device="cpu").manual_seed(2)
    key = torch.randn(T, hkv, d, generator=g).to(torch.bfloat16).to(DEV)
    val = torch.randn(T, hkv, d, generator=g).to(torch.bfloat16).to(DEV)
    A.attn_kv_cache_write(_desc(T, hkv, d, nb, bs, torch.bfloat16), key, val,
                          torch.from_numpy(slots).to(DEV), cache)
    torch.cuda.synchronize()
    blk, off = slots // bs, slots % bs
    idx_b = torch.from_numpy(blk).to(DEV)
    idx_o = torch.from_numpy(off).to(DEV)
    assert torch.equal(cache[0, idx_b, idx_o], key)
    assert torch.equal(cache[1, idx_b, idx_o], val)
    written = torch.zeros(nb * bs, dtype=torch.bool, device=DEV)
    written[torch.from_numpy(slots).to(DEV)] = True
    rest = cache.view(2, nb * bs, hkv * d)[:, ~written]
    assert int(rest.ne(0).sum()) == 0


@pytest.mark.parametrize("causal", [False, True])
def test_layer_step_write_then_attend(causal):
    """The new tokens' K/V go into the cache through slot_mapping, then attention reads them
    through the block table; the result matches the oracle's write followed by its attention."""
    b = gen.make_batch("step", num_heads=8, num_kv_heads=2, head_size=128, block_size=16,
                       dtype="bf16", query_lens=[1, 1, 37, 200], seq_lens=[70, 300, 37, 650],
                       passes=[(causal, 0)], seed=9, pool_factor=2)
    print(f"[case] write then attend causal={causal}", flush=True)
    q, kv = gen.make_tensors(b, 9, DEV, poison=True)
    g = torch.Generator(device="cpu").manual_seed(3)
    key = torch.randn(b.num_tokens, 2, 128, generator=g).to(torch.bfloat16).to(DEV)
    val = torch.randn(b.num_tokens, 2, 128, generator=g).to(torch.bfloat16).to(DEV)
    qsl, bs = b.query_start_loc, b.block_size
    slots = np.empty(b.num_tokens, np.int64)
    for r in range(b.num_seqs):
        cl = int(b.seq_lens[r] - b.query_lens[r])
        for i in range(int(b.query_lens[r])):
            p = cl + i
            slots[qsl[r] + i] = int(b.block_table[r, p // bs]) * bs + p % bs
    kv_host = host_f32(kv)
    desc_w = A.make_desc(num_seqs=b.num_seqs, num_tokens=b.num_tokens, num_decodes=b.num_decodes,
                         max_query_len=b.max_query_len, max_seq_len=b.max_seq_len,
                         num_heads=b.num_heads, num_kv_heads=2, head_size=128,
                         num_blocks=b.num_blocks, block_size=bs,
                         max_blocks_per_seq=b.max_blocks_per_seq, dtype=A.ATTN_BF16)
    assert A.attn_check_slot_mapping_host(desc_w, slots) == A.ATTN_OK
    A.attn_kv_cache_write(desc_w, key, val, torch.from_numpy(slots).to(DEV), kv)
    bt, qsl_d, sl_d = device_meta(b, DEV)
    out, lse = A.varlen_fwd(q, kv, bt, qsl_d, sl_d, scale=b.scale, causal=causal,
                            num_decodes=b.num_decodes, max_query_len=b.max_query_len,
                            max_seq_len=b.max_seq_len)
    torch.cuda.synchronize()
    kv_ref = oracle.kv_cache_write(kv_host, host_f32(key), host_f32(val), slots)
    ref_out, ref_lse = oracle.attention(host_f32(q), kv_ref, b.block_table, b.query_start_loc,
                                        b.seq_lens, b.scale, causal)
    print(compare(out, lse, ref_out, ref_lse, label="write+attend"))
