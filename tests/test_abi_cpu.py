"""The C ABI on the host: the library loads, exports what include/attn.h declares, and turns
every argument error into its status code before anything touches a GPU."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import exact_softmax_attention_paged_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "attn.h")).read()
    return sorted(set(re.findall(r"^\S[^\n(]*?\b(attn_[a-z0-9_]+)\s*\(", src, re.M)))


def test_header_declares_the_python_names():
    assert _declared() == sorted(A.EXPORTED)


def test_probe_library_exports_its_header():
    src = open(os.path.join(ROOT, "include", "attn_probes.h")).read()
    declared = sorted(set(re.findall(r"^\S[^\n(]*?\b(attn_probe_[a-z0-9_]+)\s*\(", src, re.M)))
    assert declared == ["attn_probe_lds_read", "attn_probe_mfma_loop", "attn_probe_read_stream"]
    lib = os.path.join(os.path.dirname(A.LIB_PATH), "libattn_probes.so")
    out = subprocess.run(["nm", "-D", "--defined-only", lib], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r" T (attn_probe_\w+)", out))
    assert set(declared) <= exported


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", A.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (attn_\w+)", out))
    for name in _declared():
        assert name in exported, name
        assert hasattr(A.lib(), name)


def test_status_strings():
    names = ["ATTN_OK", "ATTN_ERR_NULL", "ATTN_ERR_SHAPE", "ATTN_ERR_BLOCK_SIZE", "ATTN_ERR_GQA",
             "ATTN_ERR_UNSUPPORTED", "ATTN_ERR_WORKSPACE", "ATTN_ERR_METADATA", "ATTN_ERR_HIP"]
    assert [A.attn_status_str(i) for i in range(9)] == names
    assert A.attn_status_str(99) == "ATTN_ERR_UNKNOWN"


def _desc(**kw):
    base = dict(num_seqs=2, num_tokens=5, num_decodes=1, max_query_len=4, max_seq_len=40,
                num_heads=8, num_kv_heads=2, head_size=128, num_blocks=8, block_size=16,
                max_blocks_per_seq=3, dtype=A.ATTN_BF16, partition_tokens=0)
    base.update(kw)
    return A.make_desc(**base)


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


def _fwd(desc, causal=1, window=0, scale=0.125, ws=None, ws_bytes=0, q=FAKE, out=FAKE):
    return A.lib().attn_varlen_fwd(ctypes.byref(desc), q, FAKE, FAKE, FAKE, FAKE, scale,
                                   causal, window, out, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(block_size=24), A.ATTN_ERR_BLOCK_SIZE),
    (dict(block_size=0), A.ATTN_ERR_BLOCK_SIZE),
    (dict(num_heads=6, num_kv_heads=4), A.ATTN_ERR_GQA),
    (dict(head_size=96), A.ATTN_ERR_UNSUPPORTED),
    (dict(dtype=7), A.ATTN_ERR_UNSUPPORTED),
    (dict(partition_tokens=100), A.ATTN_ERR_UNSUPPORTED),
    (dict(partition_tokens=16384 + 128), A.ATTN_ERR_UNSUPPORTED),
    (dict(num_decodes=3), A.ATTN_ERR_SHAPE),
    (dict(num_tokens=-1), A.ATTN_ERR_SHAPE),
    (dict(max_seq_len=49), A.ATTN_ERR_SHAPE),       # exceeds max_blocks_per_seq * block_size
    (dict(max_query_len=41), A.ATTN_ERR_SHAPE),
    # more than 65535 256-row query tiles (a grid dimension of the prefill kernel)
    (dict(max_query_len=256 * 65535 + 1, max_seq_len=256 * 65535 + 1,
          max_blocks_per_seq=(256 * 65535) // 16 + 1), A.ATTN_ERR_SHAPE),
    # more than 65535 decode partitions of max_seq_len (a grid dimension of the split kernel)
    (dict(partition_tokens=128, max_seq_len=128 * 65535 + 1,
          max_blocks_per_seq=(128 * 65535) // 16 + 1), A.ATTN_ERR_SHAPE),
])
def test_descriptor_errors(kw, status):
    d = _desc(**kw)
    assert _fwd(d) == status
    n = ctypes.c_size_t(0)
    assert A.lib().attn_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == status


def test_window_needs_causal_and_scale_must_be_positive():
    assert _fwd(_desc(), causal=0, window=8) == A.ATTN_ERR_UNSUPPORTED
    assert _fwd(_desc(), scale=0.0) == A.ATTN_ERR_UNSUPPORTED
    assert _fwd(_desc(), scale=float("nan")) == A.ATTN_ERR_UNSUPPORTED


def test_null_pointers():
    assert A.lib().attn_varlen_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, 1, 0, FAKE, None,
                                   None, 0, None) == A.ATTN_ERR_NULL
    assert _fwd(_desc(), q=None) == A.ATTN_ERR_NULL
    assert _fwd(_desc(), out=None) == A.ATTN_ERR_NULL
    assert A.lib().attn_workspace_bytes(ctypes.byref(_desc()), None) == A.ATTN_ERR_NULL


def test_workspace_size_and_check():
    d = _desc(num_decodes=1, max_seq_len=40)
    need = A.attn_workspace_bytes(d)
    parts = -(-40 // 2048)                     # the default partition length

    def expected(decodes, parts):              # partition results, then the work schedule
        return (-(-(decodes * 8 * parts * (128 * 2 + 4)) // 256) * 256 +
                -(-((1 + decodes * parts) * 4) // 256) * 256)
    assert need == expected(1, parts)
    assert _fwd(d, ws=None, ws_bytes=0) == A.ATTN_ERR_WORKSPACE
    assert _fwd(d, ws=FAKE, ws_bytes=need - 1) == A.ATTN_ERR_WORKSPACE
    big = _desc(num_decodes=1, max_seq_len=40000, max_blocks_per_seq=2500)
    parts = -(-40000 // 256)
    assert A.attn_workspace_bytes(_desc(num_decodes=1, max_seq_len=40000, max_blocks_per_seq=2500,
                                        partition_tokens=256)) == expected(1, parts)
    assert A.attn_workspace_bytes(_desc(num_decodes=0)) == 0
    assert A.attn_workspace_bytes(_desc(dtype=A.ATTN_F32)) == 0
    assert big is not None


def test_fp8_decode_workspace_uses_its_own_default_partition():
    """The E4M3 decode's default partition is the bf16 default capped at 1024 keys; its
    workspace query sizes for that, and for a stated partition equals attn_workspace_bytes."""
    kw = dict(num_seqs=256, num_tokens=256, num_decodes=256, max_query_len=1, max_seq_len=8192,
              num_heads=32, num_kv_heads=8, num_blocks=40000, max_blocks_per_seq=512)
    d = _desc(**kw)
    assert A.attn_decode_partition_tokens(d) == 16384     # bf16: one partition per request

    def expected(decodes, heads, parts, segs):   # partition results, then the work schedule
        return (-(-(decodes * heads * parts * (128 * 2 + 4)) // 256) * 256 +
                -(-((1 + decodes * segs) * 4) // 256) * 256)
    assert A.attn_workspace_bytes(d) == expected(256, 32, 1, 1)
    # 1024-key partitions, one per 1024-key segment
    assert A.attn_fp8_decode_workspace_bytes(d) == expected(256, 32, 8, 8)
    for pt in (512, 4096):
        dp = _desc(partition_tokens=pt, **kw)
        assert A.attn_fp8_decode_workspace_bytes(dp) == A.attn_workspace_bytes(dp)
    small = _desc()                                 # a default below 1024 keys is kept
    assert A.attn_fp8_decode_workspace_bytes(small) >= A.attn_workspace_bytes(small)
    n = ctypes.c_size_t(0)
    assert A.lib().attn_fp8_decode_workspace_bytes(ctypes.byref(d), None) == A.ATTN_ERR_NULL
    assert A.lib().attn_fp8_decode_workspace_bytes(ctypes.byref(_desc(block_size=24)),
                                                   ctypes.byref(n)) == A.ATTN_ERR_BLOCK_SIZE


def test_empty_batch_is_a_no_op():
    d = _desc(num_seqs=0, num_tokens=0, num_decodes=0, max_query_len=0, max_seq_len=0)
    assert _fwd(d, q=None, out=None) == A.ATTN_OK


def _meta():
    qsl = np.array([0, 1, 5], np.int32)
    sl = np.array([17, 40], np.int32)
    bt = np.array([[3, 4, 7], [0, 1, 2]], np.int32)
    return bt, qsl, sl


def test_metadata_checker_accepts_good_and_rejects_bad():
    d = _desc()
    bt, qsl, sl = _meta()
    assert A.attn_check_metadata_host(d, bt, qsl, sl) == A.ATTN_OK
    bad = []
    b = bt.copy(); b[1, 2] = 8; bad.append((b, qsl, sl))              # block id out of range
    b = bt.copy(); b[0, 1] = -1; bad.append((b, qsl, sl))
    bad.append((bt, np.array([0, 2, 5], np.int32), sl))                 # decode row with ql 2
    bad.append((bt, np.array([0, 1, 4], np.int32), sl))                 # ends before num_tokens
    bad.append((bt, np.array([1, 1, 5], np.int32), sl))                 # does not start at 0
    bad.append((bt, qsl, np.array([17, 3], np.int32)))                  # seq_len < query_len
    bad.append((bt, qsl, np.array([17, 41], np.int32)))                 # > max_seq_len
    for b, q, s in bad:
        assert A.attn_check_metadata_host(d, b, q, s) == A.ATTN_ERR_METADATA
    # an unused table entry may hold anything
    b = bt.copy(); b[0, 2] = -5
    assert A.attn_check_metadata_host(d, b, qsl, sl) == A.ATTN_OK


def test_generated_workloads_pass_the_metadata_checker():
    import gen
    for k in (1, 2, 3, 4, 5):
        b = gen.config(k)
        d = A.make_desc(num_seqs=b.num_seqs, num_tokens=b.num_tokens, num_decodes=b.num_decodes,
                        max_query_len=b.max_query_len, max_seq_len=b.max_seq_len,
                        num_heads=b.num_heads, num_kv_heads=b.num_kv_heads,
                        head_size=b.head_size, num_blocks=b.num_blocks,
                        block_size=b.block_size, max_blocks_per_seq=b.max_blocks_per_seq,
                        dtype=A.ATTN_BF16 if b.dtype == "bf16" else A.ATTN_F32)
        assert A.attn_check_metadata_host(d, b.block_table, b.query_start_loc,
                                          b.seq_lens) == A.ATTN_OK


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(5, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        A.attn_varlen_fwd(_desc(), q, q, q, q, q, 0.1, True, 0, q, None, None)


# ---------------------------------------------------------------- cascade entry points
def _cascade(desc, prefix, causal=1, scale=0.125, ws=None, ws_bytes=0, q=FAKE, out=FAKE):
    return A.lib().attn_cascade_fwd(ctypes.byref(desc), q, FAKE, FAKE, FAKE, FAKE, prefix,
                                    scale, causal, out, None, ws, ws_bytes, None)


def test_cascade_argument_errors():
    d = _desc()
    assert _cascade(d, -16) == A.ATTN_ERR_SHAPE
    assert _cascade(d, 8) == A.ATTN_ERR_SHAPE                    # not a whole block
    assert _cascade(d, 48) == A.ATTN_ERR_SHAPE                   # beyond max_seq_len
    assert _cascade(_desc(dtype=A.ATTN_F32), 16) == A.ATTN_ERR_UNSUPPORTED
    assert _cascade(_desc(block_size=24), 16) == A.ATTN_ERR_BLOCK_SIZE
    assert _cascade(d, 16, scale=0.0) == A.ATTN_ERR_UNSUPPORTED
    assert _cascade(d, 16, q=None) == A.ATTN_ERR_NULL
    need = A.attn_cascade_workspace_bytes(d, 16)
    assert _cascade(d, 16, ws=None) == A.ATTN_ERR_WORKSPACE
    assert _cascade(d, 16, ws=FAKE, ws_bytes=need - 1) == A.ATTN_ERR_WORKSPACE
    n = ctypes.c_size_t(0)
    assert A.lib().attn_cascade_workspace_bytes(ctypes.byref(d), 16, None) == A.ATTN_ERR_NULL
    assert A.lib().attn_cascade_workspace_bytes(ctypes.byref(d), 8, ctypes.byref(n)) == \
        A.ATTN_ERR_SHAPE


def test_cascade_workspace_size():
    d = _desc(num_decodes=1, max_seq_len=40)
    plain = A.attn_workspace_bytes(d)
    assert A.attn_cascade_workspace_bytes(d, 0) == plain
    rows = 5 * 8                                              # num_tokens x num_heads
    pre = -(-(rows * 128 * 4) // 256) * 256 + -(-(rows * 4) // 256) * 256
    assert A.attn_cascade_workspace_bytes(d, 16) == pre + plain
    assert A.attn_cascade_workspace_bytes(_desc(num_decodes=0), 32) == pre
    # few rows and a long prefix: the prefix keys are split into slices of >= 512 keys, each
    # with its own copy of the partial result (here 4 slices of 512 keys, plus the merged copy)
    big = _desc(num_decodes=0, max_seq_len=4096, max_blocks_per_seq=256)
    assert A.attn_cascade_workspace_bytes(big, 2048) == 5 * pre
    assert A.attn_cascade_workspace_bytes(big, 512) == pre


def test_cascade_checker():
    d = _desc()
    qsl = np.array([0, 1, 5], np.int32)
    sl = np.array([17, 40], np.int32)                          # contexts 16 and 36
    bt = np.array([[3, 4, 7], [3, 1, 2]], np.int32)            # block 3 shared
    assert A.attn_check_cascade_host(d, bt, qsl, sl, 16) == A.ATTN_OK
    assert A.attn_check_cascade_host(d, bt, qsl, sl, 0) == A.ATTN_OK
    assert A.attn_check_cascade_host(d, bt, qsl, sl, 32) == A.ATTN_ERR_METADATA   # 2nd block differs
    b = bt.copy(); b[1, 0] = 5
    assert A.attn_check_cascade_host(d, b, qsl, sl, 16) == A.ATTN_ERR_METADATA    # prefix not shared
    assert A.attn_check_cascade_host(d, bt, qsl, np.array([15, 40], np.int32), 16) == \
        A.ATTN_ERR_METADATA                                    # context 14 < prefix 16
    assert A.attn_check_cascade_host(d, bt, qsl, sl, 8) == A.ATTN_ERR_SHAPE


def test_cascade_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(5, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        A.attn_cascade_fwd(_desc(), q, q, q, q, q, 16, 0.1, True, q, None, None)


# ---------------------------------------------------------------- KV-cache write
def _kvw(desc, ks=256, vs=256, key=FAKE, value=FAKE, slots=FAKE, cache=FAKE):
    return A.lib().attn_kv_cache_write(ctypes.byref(desc) if desc is not None else None, key,
                                       ks, value, vs, slots, cache, None)


def test_kv_write_argument_errors():
    d = _desc()                                       # Hkv 2, d 128: rows of 256 elements
    assert _kvw(None) == A.ATTN_ERR_NULL
    assert _kvw(d, key=None) == A.ATTN_ERR_NULL
    assert _kvw(d, slots=None) == A.ATTN_ERR_NULL
    assert _kvw(d, ks=255) == A.ATTN_ERR_SHAPE        # smaller than a row
    assert _kvw(d, vs=260) == A.ATTN_ERR_SHAPE        # 520 bytes: not a 16-byte multiple
    assert _kvw(d, key=ctypes.c_void_p(0x1008)) == A.ATTN_ERR_SHAPE   # misaligned
    assert _kvw(_desc(block_size=24)) == A.ATTN_ERR_BLOCK_SIZE
    assert _kvw(_desc(head_size=80)) == A.ATTN_ERR_UNSUPPORTED
    assert _kvw(_desc(dtype=5)) == A.ATTN_ERR_UNSUPPORTED
    assert _kvw(_desc(num_tokens=-1)) == A.ATTN_ERR_SHAPE
    assert _kvw(_desc(num_tokens=0), key=None, value=None, slots=None, cache=None) == A.ATTN_OK


def test_slot_mapping_checker():
    d = _desc(num_tokens=4)                           # 8 blocks x 16 slots
    ok = np.array([5, -1, 127, 16], np.int64)
    assert A.attn_check_slot_mapping_host(d, ok) == A.ATTN_OK
    assert A.attn_check_slot_mapping_host(d, np.array([5, -1, 128, 16], np.int64)) == \
        A.ATTN_ERR_METADATA                           # past the cache
    assert A.attn_check_slot_mapping_host(d, np.array([5, 9, 5, -1], np.int64)) == \
        A.ATTN_ERR_METADATA                           # duplicate
    assert A.attn_check_slot_mapping_host(d, np.array([-1, -1, -3, -1], np.int64)) == A.ATTN_OK


def test_kv_write_binding_refuses_cpu_tensors():
    import torch
    k = torch.zeros(5, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        A.attn_kv_cache_write(_desc(), k, k, torch.zeros(5, dtype=torch.int64),
                              torch.zeros(2, 8, 16, 2, 128, dtype=torch.bfloat16))


# ---------------------------------------------------------------- FP8 (E4M3) cache
def _fp8_decode(desc, scale=0.1, ks=0.02, vs=0.03, window=0, ws=None, ws_bytes=0, q=FAKE):
    return A.lib().attn_fp8_decode_fwd(ctypes.byref(desc), q, FAKE, FAKE, FAKE, FAKE, scale, ks,
                                       vs, window, FAKE, None, ws, ws_bytes, None)


def test_fp8_decode_argument_errors():
    dec = dict(num_seqs=2, num_tokens=2, num_decodes=2, max_query_len=1)
    d = _desc(**dec)
    assert _fp8_decode(_desc()) == A.ATTN_ERR_UNSUPPORTED          # prefill rows present
    assert _fp8_decode(_desc(dtype=A.ATTN_F32, **dec)) == A.ATTN_ERR_UNSUPPORTED
    assert _fp8_decode(d, ks=0.0) == A.ATTN_ERR_UNSUPPORTED
    assert _fp8_decode(d, vs=float("inf")) == A.ATTN_ERR_UNSUPPORTED
    assert _fp8_decode(d, scale=-1.0) == A.ATTN_ERR_UNSUPPORTED
    assert _fp8_decode(d, q=None) == A.ATTN_ERR_NULL
    need = A.attn_workspace_bytes(d)
    assert _fp8_decode(d, ws=FAKE, ws_bytes=need - 1) == A.ATTN_ERR_WORKSPACE
    assert _fp8_decode(_desc(block_size=24, **dec)) == A.ATTN_ERR_BLOCK_SIZE


def test_fp8_write_argument_errors():
    def w(desc, ks=0.02, vs=0.03, stride=256):
        return A.lib().attn_kv_cache_write_fp8(ctypes.byref(desc), FAKE, stride, FAKE, stride,
                                               FAKE, ks, vs, FAKE, None)
    assert w(_desc(dtype=A.ATTN_F32)) == A.ATTN_ERR_UNSUPPORTED
    assert w(_desc(), ks=-1.0) == A.ATTN_ERR_UNSUPPORTED
    assert w(_desc(), vs=float("nan")) == A.ATTN_ERR_UNSUPPORTED
    assert w(_desc(), stride=100) == A.ATTN_ERR_SHAPE
    assert w(_desc(), stride=260) == A.ATTN_ERR_SHAPE                # 520 bytes
    assert w(_desc(head_size=96)) == A.ATTN_ERR_UNSUPPORTED
    assert w(_desc(num_tokens=0)) == A.ATTN_OK


# ---------------------------------------------------------------- prefill work schedule
def test_schedule_sizes_and_errors():
    d = _desc(max_query_len=600, max_seq_len=40)
    with pytest.raises(A.AttnError):
        A.attn_schedule_bytes(d)                       # max_query_len > max_seq_len
    d = _desc(max_query_len=30, max_seq_len=40)      # 1 prefill request, 1 q tile
    assert A.attn_schedule_bytes(d) == 256
    big = _desc(num_seqs=300, num_tokens=5, num_decodes=0, max_query_len=1000,
                max_seq_len=1000, max_blocks_per_seq=63)
    assert A.attn_schedule_bytes(big) == -(-(4 * (1 + 300 * 4)) // 256) * 256
    lib = A.lib()
    assert lib.attn_build_schedule(ctypes.byref(d), FAKE, FAKE, 1, 0, None, 0, None) == \
        A.ATTN_ERR_WORKSPACE
    assert lib.attn_build_schedule(ctypes.byref(d), FAKE, FAKE, 1, 0, FAKE, 255, None) == \
        A.ATTN_ERR_WORKSPACE
    assert lib.attn_build_schedule(ctypes.byref(d), FAKE, FAKE, 0, 8, FAKE, 256, None) == \
        A.ATTN_ERR_UNSUPPORTED
    assert lib.attn_varlen_fwd_scheduled(ctypes.byref(_desc(dtype=A.ATTN_F32)), FAKE, FAKE, FAKE,
                                         FAKE, FAKE, 0.1, 1, 0, FAKE, None, None, 0, FAKE, 256,
                                         None) == A.ATTN_ERR_UNSUPPORTED
    assert lib.attn_varlen_fwd_scheduled(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, 1,
                                         0, FAKE, None, FAKE, 1 << 20, None, 0, None) == \
        A.ATTN_ERR_WORKSPACE


def test_decode_schedule_sizes_and_errors():
    """One count plus one slot per (decode, partition), the partitions capped for a window;
    nothing to build without split-KV decode rows."""
    d = _desc()                                        # 1 decode of <= 40 keys: 1 partition
    assert A.attn_decode_schedule_bytes(d) == 256
    assert A.attn_decode_schedule_bytes(_desc(dtype=A.ATTN_F32)) == 0
    assert A.attn_decode_schedule_bytes(_desc(num_decodes=0)) == 0
    long = _desc(num_seqs=64, num_tokens=64, num_decodes=64, max_query_len=1,
                 max_seq_len=40000, num_blocks=4000, max_blocks_per_seq=2500,
                 partition_tokens=256)
    assert A.attn_decode_schedule_bytes(long) == -(-(4 * (1 + 64 * 157)) // 256) * 256
    # a 1000-key window reaches at most ceil(1000 / 256) + 1 = 5 partitions
    assert A.attn_decode_schedule_bytes(long, 1000) == -(-(4 * (1 + 64 * 5)) // 256) * 256
    with pytest.raises(A.AttnError):
        A.attn_decode_schedule_bytes(_desc(block_size=24))
    lib = A.lib()
    assert lib.attn_build_decode_schedule(ctypes.byref(d), FAKE, 0, None, 0, None) == \
        A.ATTN_ERR_WORKSPACE
    assert lib.attn_build_decode_schedule(ctypes.byref(d), FAKE, 0, FAKE, 255, None) == \
        A.ATTN_ERR_WORKSPACE
    assert lib.attn_build_decode_schedule(ctypes.byref(d), None, 0, FAKE, 256, None) == \
        A.ATTN_ERR_NULL
    # no split-KV decode rows: nothing to build, nothing touched
    assert lib.attn_build_decode_schedule(ctypes.byref(_desc(num_decodes=0)), None, 0, None, 0,
                                          None) == A.ATTN_OK

    def pre(desc, ps, ps_bytes, ds, ds_bytes, causal=1, window=0):
        return lib.attn_varlen_fwd_prescheduled(
            ctypes.byref(desc), FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, causal, window, FAKE, None,
            FAKE, 1 << 20, ps, ps_bytes, ds, ds_bytes, None)
    assert pre(d, None, 0, FAKE, 255) == A.ATTN_ERR_WORKSPACE      # decode schedule too small
    assert pre(d, FAKE, 255, None, 0) == A.ATTN_ERR_WORKSPACE      # prefill schedule too small
    assert pre(_desc(dtype=A.ATTN_F32), FAKE, 256, None, 0) == A.ATTN_ERR_UNSUPPORTED
    assert pre(d, None, 0, None, 0, causal=0, window=8) == A.ATTN_ERR_UNSUPPORTED
    assert lib.attn_varlen_fwd_prescheduled(
        ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, 0.1, 1, 0, FAKE, None, FAKE, 1 << 20,
        None, 0, FAKE, 256, None) == A.ATTN_ERR_NULL
    assert lib.attn_varlen_fwd_prescheduled(
        ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, 1, 0, FAKE, None, None, 0,
        None, 0, FAKE, 256, None) == A.ATTN_ERR_WORKSPACE           # decode partials need it


def test_mixed_argument_errors():
    """The one-launch mixed call: bf16 only, window needs causal, a prefill schedule of the
    right size whenever prefill rows exist; no workspace."""
    lib = A.lib()

    def mixed(desc, sched, sched_bytes, causal=1, window=0, q=FAKE):
        return lib.attn_varlen_fwd_mixed(ctypes.byref(desc), q, FAKE, FAKE, FAKE, FAKE, 0.1,
                                         causal, window, FAKE, None, sched, sched_bytes, None)
    d = _desc()                                   # 1 decode + 1 prefill request
    need = A.attn_schedule_bytes(d)
    assert mixed(_desc(dtype=A.ATTN_F32), FAKE, need) == A.ATTN_ERR_UNSUPPORTED
    assert mixed(d, FAKE, need, causal=0, window=8) == A.ATTN_ERR_UNSUPPORTED
    assert mixed(d, None, 0) == A.ATTN_ERR_WORKSPACE
    assert mixed(d, FAKE, need - 1) == A.ATTN_ERR_WORKSPACE
    assert mixed(d, FAKE, need, q=None) == A.ATTN_ERR_NULL
    assert mixed(_desc(block_size=24), FAKE, need) == A.ATTN_ERR_BLOCK_SIZE
    # decode rows only: no schedule needed
    only_dec = _desc(num_seqs=2, num_tokens=2, num_decodes=2, max_query_len=1)
    assert mixed(only_dec, None, 0, q=None) == A.ATTN_ERR_NULL
    # an empty batch is a no-op (nothing is read)
    assert mixed(_desc(num_tokens=0), FAKE, need, q=None) == A.ATTN_OK


def test_default_partition_follows_the_batch_size():
    """partition_tokens 0: the longest of 16384 ... 256 keys that still gives at least 2048
    split workgroups (decodes x kv heads x head groups x partitions of max_seq_len), else 256
    (include/attn.h); observed through the workspace size, which holds one partial result and
    one schedule slot per (decode, partition)."""
    def need(num_decodes, max_seq_len, heads=32, kv=8):
        d = _desc(num_seqs=num_decodes, num_tokens=num_decodes, num_decodes=num_decodes,
                  max_query_len=1, max_seq_len=max_seq_len, num_heads=heads, num_kv_heads=kv,
                  num_blocks=num_decodes * 3000, max_blocks_per_seq=-(-max_seq_len // 16))
        return A.attn_workspace_bytes(d)

    def expected(decodes, parts, heads=32, d=128):
        return (-(-(decodes * heads * parts * (d * 2 + 4)) // 256) * 256 +
                -(-((1 + decodes * parts) * 4) // 256) * 256)
    # 256 requests x 8 kv heads = 2048 workgroups with one 16384-key partition each
    assert need(256, 8192) == expected(256, 1)
    # 120 x 8 = 960 per partition: 16384 keys give 1920 (< 2048), 8192 keys give 3840
    assert need(120, 32768) == expected(120, 4)
    # a single request of 40000 keys: 8 per partition, so the 256-key floor (157 partitions)
    assert need(1, 40000) == expected(1, -(-40000 // 256))
    # 64 q heads on one kv head form 4 workgroups of 16 heads: 64 x 4 = 256 per partition,
    # so 1024-key partitions (8 of them) are the longest reaching 2048
    assert need(64, 8192, heads=64, kv=1) == expected(64, 8, heads=64)


def test_partition_query_reports_the_length_in_use():
    def part(num_decodes, max_seq_len, pt=0, heads=32, kv=8):
        return A.attn_decode_partition_tokens(_desc(
            num_seqs=num_decodes, num_tokens=num_decodes, num_decodes=num_decodes,
            max_query_len=1, max_seq_len=max_seq_len, num_heads=heads, num_kv_heads=kv,
            num_blocks=num_decodes * 3000, max_blocks_per_seq=-(-max_seq_len // 16),
            partition_tokens=pt))
    assert part(256, 8192) == 16384
    assert part(120, 32768) == 8192
    assert part(1, 40000) == 256
    assert part(64, 8192, heads=64, kv=1) == 1024
    assert part(256, 8192, pt=512) == 512
    n = ctypes.c_int32(0)
    assert A.lib().attn_decode_partition_tokens(ctypes.byref(_desc(block_size=24)),
                                                ctypes.byref(n)) == A.ATTN_ERR_BLOCK_SIZE
    assert A.lib().attn_decode_partition_tokens(ctypes.byref(_desc()), None) == A.ATTN_ERR_NULL


# ---------------------------------------------------------------- no-allocation entry point
def _noalloc(desc, causal=1, window=0, scale=0.125, q=FAKE, out=FAKE):
    return A.lib().attn_varlen_fwd_noalloc(ctypes.byref(desc), q, FAKE, FAKE, FAKE, FAKE, scale,
                                           causal, window, out, None, None)


def test_noalloc_limit_matches_the_header():
    src = open(os.path.join(ROOT, "include", "attn.h")).read()
    m = re.search(r"#define ATTN_NOALLOC_SCRATCH_BYTES \((\d+)u \* (\d+)u \* (\d+)u\)", src)
    assert m and int(m[1]) * int(m[2]) * int(m[3]) == A.NOALLOC_SCRATCH_BYTES


def test_noalloc_argument_errors_and_size_limit():
    """Argument errors as for attn_varlen_fwd; a call whose split-KV partial results would not
    fit the fixed array is refused with ATTN_ERR_WORKSPACE before anything touches a GPU."""
    assert _noalloc(_desc(block_size=24)) == A.ATTN_ERR_BLOCK_SIZE
    assert _noalloc(_desc(), causal=0, window=8) == A.ATTN_ERR_UNSUPPORTED
    assert _noalloc(_desc(), scale=0.0) == A.ATTN_ERR_UNSUPPORTED
    assert A.lib().attn_varlen_fwd_noalloc(None, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, 1, 0, FAKE,
                                           None, None) == A.ATTN_ERR_NULL
    # 1024 decode requests of 32768 keys in 128-key partitions, 8 q heads: 1024 * 8 * 256
    # partials of 129 floats = 270 MB > 128 MiB
    big = _desc(num_seqs=1024, num_tokens=1024, num_decodes=1024, max_query_len=1,
                max_seq_len=32768, max_blocks_per_seq=2048, partition_tokens=128)
    assert A.attn_workspace_bytes(big) > A.NOALLOC_SCRATCH_BYTES
    assert _noalloc(big) == A.ATTN_ERR_WORKSPACE
    # with a 256-key window the same batch needs only 3 partitions per request: it fits, and
    # the call then fails on the NULL q instead
    assert _noalloc(big, window=256, q=None) == A.ATTN_ERR_NULL
    empty = _desc(num_seqs=0, num_tokens=0, num_decodes=0, max_query_len=0, max_seq_len=0)
    assert _noalloc(empty, q=None, out=None) == A.ATTN_OK
