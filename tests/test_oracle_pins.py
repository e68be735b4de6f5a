"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test fixes one part of the definition (scores, mask, softmax, xV, paging, GQA, lse)
with a closed form, an invariant, a hand-worked fixture, a library routine computing the
same special case, or high-precision brute force on tiny inputs. A plausible slip in the
oracle (dropped scale, wrong sign, off-by-one mask, wrong kv-head mapping, transposed
operand, lse without the max) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import gen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(seed, num_seqs=3, ql_range=(1, 40), ctx_range=(0, 30), hq=4, hkv=2, d=8, bs=16):
    rng = np.random.default_rng(seed)
    ql = rng.integers(ql_range[0], ql_range[1] + 1, size=num_seqs)
    cl = rng.integers(ctx_range[0], ctx_range[1] + 1, size=num_seqs)
    b = gen.make_batch("pin", num_heads=hq, num_kv_heads=hkv, head_size=d, block_size=bs,
                       dtype="f32", query_lens=ql, seq_lens=ql + cl, passes=[(True, 0)],
                       seed=seed, pool_factor=2)
    q, kv = gen.make_tensors(b, seed)
    return b, gen.to_numpy_f64(q), gen.to_numpy_f64(kv)


def _run(b, q, kv, causal, window=0, scale=None):
    return oracle.attention(q, kv, b.block_table, b.query_start_loc, b.seq_lens,
                            b.scale if scale is None else scale, causal, window)


MASKS = [(False, 0), (True, 0), (True, 1), (True, 5)]


# ---------------------------------------------------------------- hand-worked fixture
@pytest.mark.parametrize("case", range(3))
def test_hand_worked_example(case):
    fx = json.load(open(os.path.join(GOLDEN, "hand_worked.json")))
    c = fx["cases"][case]
    kv = np.zeros((2, 2, 16, 1, 2))
    kv[0, 1, :3, 0] = fx["k"]
    kv[1, 1, :3, 0] = fx["v"]
    q = np.asarray(fx["q"], dtype=np.float64)[:, None, :]
    out, lse = oracle.attention(q, kv, np.array([[1]]), np.array([0, 3]), np.array([3]), 1.0,
                                c["causal"], c["window"])
    ns = {"e": math.e, "log": math.log}
    exp_out = np.array([[eval(x, {"__builtins__": {}}, ns) for x in row] for row in c["out"]])
    exp_lse = np.array([eval(x, {"__builtins__": {}}, ns) for x in c["lse"]])
    np.testing.assert_allclose(out[:, 0], exp_out, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[:, 0], exp_lse, rtol=0, atol=1e-14)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("causal,window", MASKS)
def test_constant_v_gives_that_constant(causal, window):
    b, q, kv = _rand_case(11)
    c = np.random.default_rng(5).standard_normal((b.num_kv_heads, b.head_size))
    kv[1] = c                          # every value row of kv head h equals c[h]
    out, _ = _run(b, q, kv, causal, window)
    g = b.num_heads // b.num_kv_heads
    for h in range(b.num_heads):
        np.testing.assert_allclose(out[:, h], np.broadcast_to(c[h // g], out[:, h].shape),
                                   rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal,window", MASKS)
def test_zero_query_gives_mean_of_visible_values(causal, window):
    """q = 0 makes every visible score 0: out is the plain mean of the visible v rows and
    lse = ln(#visible). The count is (context_len + i + 1) for causal, clipped to W by the
    window, and seq_len without the mask: this pins the mask bounds exactly."""
    b, q, kv = _rand_case(12)
    q[:] = 0.0
    out, lse = _run(b, q, kv, causal, window)
    qsl = b.query_start_loc
    g = b.num_heads // b.num_kv_heads
    for r in range(b.num_seqs):
        ql, sl = int(b.query_lens[r]), int(b.seq_lens[r])
        cl = sl - ql
        vals = np.stack([kv[1, b.block_table[r, t // b.block_size], t % b.block_size]
                         for t in range(sl)])            # [sl, Hkv, d], read slot by slot
        for i in range(ql):
            p = cl + i
            hi = p + 1 if causal else sl
            lo = max(0, p - window + 1) if window > 0 else 0
            n = hi - lo
            for h in range(b.num_heads):
                np.testing.assert_allclose(out[qsl[r] + i, h], vals[lo:hi, h // g].mean(0),
                                           rtol=0, atol=1e-13)
                assert abs(lse[qsl[r] + i, h] - math.log(n)) < 1e-13


def test_single_visible_key_returns_its_value():
    """Causal row 0 with no context, and any row with W = 1, see exactly one key:
    out = v of that key and lse = scale * q.k of that key."""
    b = gen.make_batch("one", num_heads=2, num_kv_heads=1, head_size=8, block_size=16,
                       dtype="f32", query_lens=[7], seq_lens=[7], passes=[(True, 0)], seed=3)
    q, kv = gen.make_tensors(b, 3)
    q, kv = gen.to_numpy_f64(q), gen.to_numpy_f64(kv)
    blk = b.block_table[0, 0]
    out, lse = _run(b, q, kv, True, 0)
    for h in range(2):
        np.testing.assert_allclose(out[0, h], kv[1, blk, 0, 0], atol=1e-15)
        assert abs(lse[0, h] - b.scale * float(q[0, h] @ kv[0, blk, 0, 0])) < 1e-14
    out, lse = _run(b, q, kv, True, 1)
    for i in range(7):
        for h in range(2):
            np.testing.assert_allclose(out[i, h], kv[1, blk, i, 0], atol=1e-15)
            assert abs(lse[i, h] - b.scale * float(q[i, h] @ kv[0, blk, i, 0])) < 1e-14


def test_two_keys_logistic_closed_form():
    rng = np.random.default_rng(4)
    d = 16
    qv, k0, k1, v0, v1 = (rng.standard_normal(d) for _ in range(5))
    kv = np.zeros((2, 1, 16, 1, d))
    kv[0, 0, 0, 0], kv[0, 0, 1, 0], kv[1, 0, 0, 0], kv[1, 0, 1, 0] = k0, k1, v0, v1
    scale = 0.37
    out, lse = oracle.attention(qv[None, None, :], kv, np.array([[0]]), np.array([0, 1]),
                                np.array([2]), scale, False, 0)
    s0, s1 = scale * qv @ k0, scale * qv @ k1
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    np.testing.assert_allclose(out[0, 0], sig(s0 - s1) * v0 + sig(s1 - s0) * v1, atol=1e-14)
    assert abs(lse[0, 0] - np.logaddexp(s0, s1)) < 1e-14


def test_softmax_weights_rows_sum_to_one():
    rng = np.random.default_rng(6)
    s = rng.standard_normal((50, 40)) * 30
    vis = rng.random((50, 40)) < 0.6
    vis[3] = False                     # an empty row
    w, lse = oracle.softmax_weights(s, vis)
    assert np.all(w >= 0) and np.all(w[~vis] == 0)
    full = vis.any(1)
    np.testing.assert_allclose(w[full].sum(1), 1.0, atol=1e-14)
    assert np.all(w[3] == 0) and lse[3] == -np.inf


def test_empty_row_is_zero_with_minus_inf_lse():
    out, lse = oracle.attend_rows(np.ones((2, 4)), np.ones((3, 4)), np.ones((3, 4)), 1.0,
                                  np.zeros((2, 3), dtype=bool))
    assert np.all(out == 0) and np.all(lse == -np.inf)


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("causal,window", MASKS)
def test_key_shift_moves_lse_only(causal, window):
    """Adding one vector u to every key shifts each row's scores by scale*q.u: out is
    unchanged and lse moves by exactly that amount (pins lse = max + ln sum)."""
    b, q, kv = _rand_case(13)
    out0, lse0 = _run(b, q, kv, causal, window)
    u = np.random.default_rng(1).standard_normal((b.num_kv_heads, b.head_size)) * 3
    kv2 = kv.copy()
    kv2[0] = kv[0] + u
    out1, lse1 = _run(b, q, kv2, causal, window)
    g = b.num_heads // b.num_kv_heads
    shift = np.stack([b.scale * q[:, h] @ u[h // g] for h in range(b.num_heads)], 1)
    np.testing.assert_allclose(out1, out0, atol=1e-12)
    np.testing.assert_allclose(lse1, lse0 + shift, atol=1e-12)


def test_scale_is_applied_to_scores():
    b, q, kv = _rand_case(14)
    o1, l1 = _run(b, q, kv, True, 0, scale=0.5)
    o2, l2 = _run(b, q * 0.5, kv, True, 0, scale=1.0)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


@pytest.mark.parametrize("causal,window", MASKS)
def test_block_permutation_is_bitwise_invariant(causal, window):
    b, q, kv = _rand_case(15)
    out0, lse0 = _run(b, q, kv, causal, window)
    perm = np.random.default_rng(2).permutation(b.num_blocks)     # new slot of block i
    kv2 = np.empty_like(kv)
    kv2[:, perm] = kv
    b2 = gen.Batch(**{**b.__dict__, "block_table": perm[b.block_table].astype(np.int32)})
    out1, lse1 = _run(b2, q, kv2, causal, window)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


@pytest.mark.parametrize("causal,window", MASKS)
def test_paged_equals_contiguous_bitwise(causal, window):
    b, q, kv = _rand_case(16)
    qt, kvt = gen.make_tensors(b, 16)
    twin, kvc = gen.contiguous_twin(b, kvt)
    out0, lse0 = _run(b, q, kv, causal, window)
    out1, lse1 = _run(twin, q, gen.to_numpy_f64(kvc), causal, window)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


@pytest.mark.parametrize("causal,window", MASKS)
def test_gqa_equals_mha_with_repeated_kv_heads(causal, window):
    b, q, kv = _rand_case(17, hq=6, hkv=2)
    out0, lse0 = _run(b, q, kv, causal, window)
    kv_rep = np.repeat(kv, 3, axis=3)      # kv head k serves q heads 3k, 3k+1, 3k+2
    b2 = gen.Batch(**{**b.__dict__, "num_kv_heads": 6})
    out1, lse1 = _run(b2, q, kv_rep, causal, window)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


def test_decode_row_equals_last_row_of_prefill():
    """A query_len-1 request with context c gives the same row as the last query row of a
    causal prefill of length c+1 over the same keys (the decode/prefill split of the
    Linear-attention page's split rule changes nothing in the definition)."""
    b, q, kv = _rand_case(18, num_seqs=1, ql_range=(9, 9), ctx_range=(20, 20))
    out0, lse0 = _run(b, q, kv, True, 0)
    out1, lse1 = oracle.attention(q[-1:], kv, b.block_table, np.array([0, 1]), b.seq_lens,
                                  b.scale, True, 0)
    np.testing.assert_allclose(out1[0], out0[-1], atol=1e-15)
    np.testing.assert_allclose(lse1[0], lse0[-1], atol=1e-15)


# ---------------------------------------------------------------- library special case
@pytest.mark.parametrize("causal,window", MASKS)
def test_matches_torch_sdpa_fp64(causal, window):
    """One unpaged request: torch's scaled_dot_product_attention (fp64, CPU) with an explicit
    boolean mask built for bottom-right alignment, and torch.logsumexp for the lse."""
    b, q, kv = _rand_case(19, num_seqs=1, ql_range=(33, 33), ctx_range=(21, 21), hq=6, hkv=3)
    out, lse = _run(b, q, kv, causal, window)
    sl, ql = int(b.seq_lens[0]), int(b.query_lens[0])
    k, v = oracle.gather_kv(kv, b.block_table[0], sl)      # only the gather is shared
    g = b.num_heads // b.num_kv_heads
    K = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, 0)     # [Hq, sl, d]
    V = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, 0)
    Q = torch.from_numpy(q).permute(1, 0, 2)                             # [Hq, ql, d]
    i = torch.arange(ql)[:, None] + (sl - ql)
    j = torch.arange(sl)[None, :]
    mask = torch.ones(ql, sl, dtype=torch.bool)
    if causal:
        mask &= j <= i
    if window > 0:
        mask &= j >= i - window + 1
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask,
                                                           scale=b.scale)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), atol=1e-12)
    s = torch.matmul(Q, K.transpose(1, 2)) * b.scale
    ref_lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)
    np.testing.assert_allclose(lse, ref_lse.T.numpy(), atol=1e-12)


def test_gather_reads_block_table_slots():
    """The paged read of the FlashAttentionBackend layout: token t of a request is slot
    t % block_size of block table[t // block_size], K at index 0 and V at index 1."""
    kv = np.zeros((2, 5, 16, 2, 3))
    for blk in range(5):
        for s in range(16):
            kv[0, blk, s] = 1000 * blk + s
            kv[1, blk, s] = -(1000 * blk + s)
    table = np.array([3, 0, 4])
    k, v = oracle.gather_kv(kv, table, 40)
    for t in range(40):
        want = 1000 * table[t // 16] + t % 16
        assert np.all(k[t] == want) and np.all(v[t] == -want)


# ---------------------------------------------------------------- brute force
def test_mpmath_brute_force_tiny():
    """Three requests, all mask kinds, GQA 4/2, d = 8: an mpmath evaluation at 50 digits,
    reading K/V slot by slot, agrees to 1e-12."""
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 50
    b, q, kv = _rand_case(20, num_seqs=3, ql_range=(1, 12), ctx_range=(0, 20))
    qsl = b.query_start_loc
    g = b.num_heads // b.num_kv_heads
    for causal, window in MASKS:
        out, lse = _run(b, q, kv, causal, window)
        for r in range(b.num_seqs):
            ql, sl = int(b.query_lens[r]), int(b.seq_lens[r])
            for i in range(ql):
                p = sl - ql + i
                for h in range(b.num_heads):
                    terms = []
                    for t in range(sl):
                        if causal and t > p:
                            continue
                        if window > 0 and t < p - window + 1:
                            continue
                        blk, slot = b.block_table[r, t // b.block_size], t % b.block_size
                        s = mpmath.mpf(b.scale) * mpmath.fsum(
                            mpmath.mpf(q[qsl[r] + i, h, x]) * mpmath.mpf(kv[0, blk, slot, h // g, x])
                            for x in range(b.head_size))
                        terms.append((s, kv[1, blk, slot, h // g]))
                    z = mpmath.fsum(mpmath.exp(s) for s, _ in terms)
                    assert abs(float(mpmath.log(z)) - lse[qsl[r] + i, h]) < 1e-12
                    for x in range(b.head_size):
                        o = mpmath.fsum(mpmath.exp(s) * mpmath.mpf(vv[x]) for s, vv in terms) / z
                        assert abs(float(o) - out[qsl[r] + i, h, x]) < 1e-12


def test_visible_pair_count_matches_mask():
    rng = np.random.default_rng(7)
    for _ in range(20):
        ql = rng.integers(1, 50, size=4)
        sl = ql + rng.integers(0, 60, size=4)
        for causal, window in MASKS:
            n = sum(int(oracle.visible_keys(int(a), int(c), causal, window).sum())
                    for a, c in zip(ql, sl))
            assert oracle.flops_visible_pairs(ql, sl, causal, window) == n
