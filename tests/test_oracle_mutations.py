"""The pins catch planted mistakes: each mutation below is applied to a copy of the
oracle's source on the CPU, the copy replaces the oracle's functions, and at least one pin
must then fail."""
import inspect
import types

import pytest

import oracle
import oracle.naive_attention as na
import test_oracle_pins as pins

MUTATIONS = {
    "drop_scale": ("scores = scale * (", "scores = ("),
    "causal_off_by_one": ("vis &= j <= p", "vis &= j < p"),
    "window_off_by_one": ("vis &= j >= p - window + 1", "vis &= j >= p - window"),
    "top_left_causal": ("p = context_len + np.arange(query_len)[:, None]",
                        "p = np.arange(query_len)[:, None]"),
    "lse_without_max": ("m_safe + np.log", "np.log"),
    "kv_head_modulo": ("heads = np.arange(kvh * group, (kvh + 1) * group)",
                       "heads = np.arange(kvh, num_heads, num_kv_heads)"),
    "v_read_from_k": ("v = np.asarray(kv_cache[1]", "v = np.asarray(kv_cache[0]"),
    "slot_shifted": ("slots = t % block_size", "slots = (t + 1) % block_size"),
    "exp_sign": ("np.exp(s - m_safe)", "np.exp(m_safe - s)"),
    "unnormalised": ("e / np.where(empty, 1.0, l)", "e"),
    "values_key_order_reversed": ("return w @ np.asarray(v, np.float64), lse",
                                  "return w @ np.asarray(v, np.float64)[::-1], lse"),
    "query_rows_misaligned": ("q_rows = q[q0 + ii][:, heads]", "q_rows = q[ii][:, heads]"),
}


def _pin_calls():
    calls = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_") or name == "test_mpmath_brute_force_tiny":
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if not params:
            calls.append((fn, {}))
            continue
        argnames, values = params[0].args
        argnames = [a.strip() for a in argnames.split(",")] if isinstance(argnames, str) else argnames
        for v in values:
            v = v if isinstance(v, tuple) else (v,)
            calls.append((fn, dict(zip(argnames, v))))
    return calls


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_a_planted_mistake_fails_some_pin(mutation, monkeypatch):
    before, after = MUTATIONS[mutation]
    src = inspect.getsource(na)
    assert before in src
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(before, after, 1), "oracle_mutant", "exec"), mod.__dict__)
    for name in oracle.__all__:
        if hasattr(mod, name):          # the names that come from naive_attention
            monkeypatch.setattr(oracle, name, getattr(mod, name))
    failed = []
    for fn, kw in _pin_calls():
        try:
            fn(**kw)
        except Exception:           # an assertion, or a shape error the mistake causes
            failed.append(fn.__name__)
    assert failed, f"no pin caught mutation {mutation}"
