"""Pins of the cascade oracle (prefix pass + suffix pass + log-sum-exp merge).

The method is exact, so the decomposition must reproduce plain attention over all keys
(``oracle.attention``, itself pinned elsewhere); the merge is also pinned on its own: a
split of one key set into parts, merged, gives the softmax over the whole set, and closed
forms fix the weights. Planted mistakes in the cascade code must fail one of these pins.
"""
import inspect
import math
import types

import numpy as np
import pytest

import gen
import oracle
import oracle.cascade as oc


def _prefix_case(seed, causal, num_decodes=2, num_prefill=3, prefix_blocks=2, bs=16, hq=4,
                 hkv=2, d=8):
    rng = np.random.default_rng(seed)
    P = prefix_blocks * bs
    ql = np.concatenate([np.ones(num_decodes, np.int64),
                         rng.integers(2, 40, size=num_prefill, endpoint=True)])
    cl = P + rng.integers(0, 30, size=ql.size, endpoint=True)     # context covers the prefix
    b = gen.make_batch("cascade-pin", num_heads=hq, num_kv_heads=hkv, head_size=d,
                       block_size=bs, dtype="f32", query_lens=ql, seq_lens=ql + cl,
                       passes=[(causal, 0)], seed=seed, pool_factor=2,
                       shared_prefix_blocks=prefix_blocks)
    q, kv = gen.make_tensors(b, seed)
    return b, gen.to_numpy_f64(q), gen.to_numpy_f64(kv), P


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_cascade_equals_plain_attention(seed, causal):
    b, q, kv, P = _prefix_case(seed, causal)
    o1, l1 = oracle.attention(q, kv, b.block_table, b.query_start_loc, b.seq_lens, b.scale,
                              causal)
    o2, l2 = oracle.cascade_attention(q, kv, b.block_table, b.query_start_loc, b.seq_lens,
                                      b.scale, causal, P)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)


def test_cascade_with_zero_prefix_is_plain_attention():
    b, q, kv, _ = _prefix_case(4, True)
    o1, l1 = oracle.attention(q, kv, b.block_table, b.query_start_loc, b.seq_lens, b.scale, True)
    o2, l2 = oracle.cascade_attention(q, kv, b.block_table, b.query_start_loc, b.seq_lens,
                                      b.scale, True, 0)
    np.testing.assert_array_equal(o2, o1)
    np.testing.assert_array_equal(l2, l1)


def test_cascade_prefix_is_one_block_per_request_closed_form():
    # q = 0: every visible key gets the same weight. Prefix of P keys with values a_j, one
    # suffix key (the decode query's own) with value b: out = (sum a_j + b) / (P + 1),
    # lse = ln(P + 1).
    bs, P = 16, 16
    kv = np.zeros((2, 3, bs, 1, 2))
    a = np.arange(P, dtype=np.float64)
    kv[1, 2, :P, 0, 0] = a                       # prefix block (physical block 2)
    kv[1, 0, 0, 0, 0] = 100.0                    # suffix key of request 0 (block 0)
    kv[1, 1, 0, 0, 0] = -50.0                    # suffix key of request 1 (block 1)
    q = np.zeros((2, 1, 2))
    bt = np.array([[2, 0], [2, 1]])
    out, lse = oracle.cascade_attention(q, kv, bt, np.array([0, 1, 2]), np.array([P + 1, P + 1]),
                                        0.5, True, P)
    np.testing.assert_allclose(out[:, 0, 0], [(a.sum() + 100) / (P + 1), (a.sum() - 50) / (P + 1)],
                               rtol=0, atol=1e-12)
    np.testing.assert_allclose(out[:, 0, 1], 0.0, atol=0)
    np.testing.assert_allclose(lse[:, 0], math.log(P + 1), rtol=0, atol=1e-14)


@pytest.mark.parametrize("split", [1, 5, 17])
def test_merge_of_a_key_split_is_the_softmax_over_all_keys(split):
    rng = np.random.default_rng(split)
    s = rng.normal(size=(6, 23)) * 3                    # scaled scores of 6 rows over 23 keys
    v = rng.normal(size=(23, 4))
    def part(cols):
        m = s[:, cols].max(axis=1, keepdims=True)
        e = np.exp(s[:, cols] - m)
        return (e @ v[cols]) / e.sum(axis=1, keepdims=True), (m[:, 0] + np.log(e.sum(axis=1)))
    o_all, l_all = part(np.arange(23))
    o1, l1 = part(np.arange(split))
    o2, l2 = part(np.arange(split, 23))
    o, l = oracle.merge_partials([o1, o2], [l1, l2])
    np.testing.assert_allclose(o, o_all, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, l_all, rtol=0, atol=1e-13)
    o_r, l_r = oracle.merge_partials([o2, o1], [l2, l1])  # order does not matter
    np.testing.assert_allclose(o_r, o, rtol=0, atol=1e-15)
    np.testing.assert_allclose(l_r, l, rtol=0, atol=1e-15)


def test_merge_weights_closed_form_and_empty_parts():
    # lse values ln 1 and ln 3: weights 1/4 and 3/4, merged lse ln 4
    o, l = oracle.merge_partials([np.array([[1.0, 0.0]]), np.array([[0.0, 2.0]])],
                                 [np.array([0.0]), np.array([math.log(3.0)])])
    np.testing.assert_allclose(o, [[0.25, 1.5]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(l, [math.log(4.0)], rtol=0, atol=1e-15)
    # an empty part (lse = -inf) changes nothing; two empty parts give out 0, lse -inf
    o1, l1 = oracle.merge_partials([np.array([[3.0, -1.0]]), np.zeros((1, 2))],
                                   [np.array([0.7]), np.array([-np.inf])])
    np.testing.assert_array_equal(o1, [[3.0, -1.0]])
    np.testing.assert_allclose(l1, [0.7], rtol=0, atol=1e-15)
    o0, l0 = oracle.merge_partials([np.zeros((1, 2)), np.zeros((1, 2))],
                                   [np.array([-np.inf]), np.array([-np.inf])])
    np.testing.assert_array_equal(o0, [[0.0, 0.0]])
    assert np.isneginf(l0[0])


MUTATIONS = {
    "merge_weight_sign": ("e = np.exp(lse - m_safe)", "e = np.exp(m_safe - lse)"),
    "merge_unnormalised": ("w = e / np.where(empty, 1.0, s)", "w = e"),
    "merge_lse_without_log": ("m_safe + np.log(np.where(empty, 1.0, s))", "m_safe + np.where(empty, 1.0, s)"),
    "prefix_pass_causal": ("scale, causal=False)", "scale, causal=True)"),
    "suffix_lengths_unshifted": ("sl - P, scale, causal)", "sl, scale, causal)"),
    "suffix_blocks_unshifted": ("block_table[:, nb:]", "block_table[:, :]"),
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_a_planted_cascade_mistake_fails_some_pin(mutation, monkeypatch):
    before, after = MUTATIONS[mutation]
    src = inspect.getsource(oc)
    assert before in src
    mod = types.ModuleType("oracle_cascade_mutant")
    mod.__dict__["__package__"] = "oracle"
    src = src.replace("from .naive_attention import attention", "from oracle import attention")
    exec(compile(src.replace(before, after, 1), "oracle_cascade_mutant", "exec"), mod.__dict__)
    monkeypatch.setattr(oracle, "cascade_attention", mod.cascade_attention)
    monkeypatch.setattr(oracle, "merge_partials", mod.merge_partials)
    pins = [lambda: test_cascade_equals_plain_attention(1, True),
            lambda: test_cascade_equals_plain_attention(2, False),
            test_cascade_prefix_is_one_block_per_request_closed_form,
            lambda: test_merge_of_a_key_split_is_the_softmax_over_all_keys(5),
            test_merge_weights_closed_form_and_empty_parts]
    failed = 0
    for pin in pins:
        try:
            pin()
        except Exception:
            failed += 1
    assert failed, f"no pin caught mutation {mutation}"
