"""Host-side checks of libkvq that need no GPU: exports, constant tables, config validation."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import codebooks as cbk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "kvq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    from rope_aware_bit_amd import kvq
    names = _declared_functions()
    assert len(names) >= 15
    lib = ctypes.CDLL(kvq._LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(kvq.EXPORTED)


def test_library_tables_equal_oracle_tables():
    # two independent implementations of the same definitions agree bit for bit
    from rope_aware_bit_amd import kvq
    for b in range(1, 9):
        cb, bd = kvq.codebook(b)
        assert np.array_equal(cb.view(np.uint16), cbk.codebook(b).view(np.uint16)), b
        assert np.array_equal(bd.view(np.uint32), cbk.boundaries(b).view(np.uint32)), b
    assert np.array_equal(kvq.delta().view(np.uint32), cbk.delta_table().view(np.uint32))
    lv, bd = kvq.nf16_codebook()
    assert np.array_equal(lv.view(np.uint16), cbk.nf16_levels().view(np.uint16))
    assert np.array_equal(bd.view(np.uint32), cbk.nf16_boundaries().view(np.uint32))


def test_boundaries_are_fp32_midpoints_of_fp16_centroids():
    # the decode step's in-kernel quantizer forms boundary k as 0.5 * (CB[k] + CB[k+1]) in fp32
    # from the fp16 centroids; that is the library's boundary table bit for bit, because the sum
    # of two neighbouring fp16 centroids is exact in fp32
    from rope_aware_bit_amd import kvq
    for b in range(1, 9):
        cb, bd = kvq.codebook(b)
        c = cb.astype(np.float32)
        mid = np.float32(0.5) * (c[:-1] + c[1:])
        assert np.array_equal(mid.view(np.uint32), bd[:len(mid)].view(np.uint32)), b
        exact = (cb[:-1].astype(np.float64) + cb[1:].astype(np.float64)) / 2
        assert np.array_equal(mid.astype(np.float64), exact), b


def test_codebook_bad_bits():
    from rope_aware_bit_amd import kvq
    for b in (0, 9, -1):
        assert kvq.lib.kvq_codebook(b, None, None) == kvq.KVQ_EINVAL
    assert kvq.lib.kvq_delta(None) == kvq.KVQ_EINVAL


BAD = [
    dict(head_dim=64),
    dict(n_q_heads=12),                 # group 3
    dict(n_q_heads=7),                  # not a multiple
    dict(n_q_heads=64, n_kv_heads=4),   # group 16
    dict(k_bits=0),
    dict(k_bits=9),
    dict(v_bits=0),
    dict(v_bits=9),
    dict(b_min=3, k_bits=2),
    dict(b_max=2, k_bits=3),
    dict(b_min=-1),
    dict(b_max=9),
    dict(batch=0),
    dict(n_layers=0),
    dict(max_tokens=0),
    dict(codec=7),
    dict(pairing=2),
    dict(codec=2, k_bits=3),            # NF16 needs K4V4
    dict(codec=2, n_kv_heads=1, n_q_heads=1),  # NF16 needs n_kv*128 % 256 == 0
    dict(recent_window=-1),
    dict(recent_window=4097),
    dict(recent_window=100),            # not a multiple of 128
    dict(per_sequence_plans=2),
    dict(codec=4, k_bits=5, b_max=8),   # KIVI codes are at most 4 bits
    dict(codec=4, v_bits=6),
    dict(codec=6),
]


@pytest.mark.parametrize("bad", BAD)
def test_create_rejects_bad_config_without_touching_gpu(bad):
    from rope_aware_bit_amd import kvq
    base = dict(n_layers=1, n_kv_heads=2, n_q_heads=16, batch=1, max_tokens=1024, k_bits=3, v_bits=3)
    base.update(bad)
    assert kvq.create_status(kvq.Config(**base)) == kvq.KVQ_EINVAL


def test_null_handles_and_status_strings():
    from rope_aware_bit_amd import kvq
    L = kvq.lib
    assert L.kvq_cache_create(None, None) == kvq.KVQ_EINVAL
    assert L.kvq_alloc_bits(None, 0, None, 0, 1, None, None) == kvq.KVQ_EINVAL
    assert L.kvq_quantize_append(None, 0, None, None, 0, 1, None) == kvq.KVQ_EINVAL
    assert L.kvq_decode_attn(None, 0, None, 0, 0.0, None, None) == kvq.KVQ_EINVAL
    assert L.kvq_get_plan(None, 0, None, None) == kvq.KVQ_EINVAL
    n = ctypes.c_int64()
    assert L.kvq_seq_len(None, 0, ctypes.byref(n)) == kvq.KVQ_EINVAL
    assert L.kvq_read_cache(None, 0, 0, 0, 0, None) == kvq.KVQ_EINVAL
    assert L.kvq_cache_status(None) == kvq.KVQ_EINVAL
    v = kvq.kvq_view()
    assert L.kvq_cache_view(None, 0, ctypes.byref(v)) == kvq.KVQ_EINVAL
    L.kvq_cache_destroy(None)
    for s, name in enumerate(["KVQ_OK", "KVQ_EINVAL", "KVQ_ENOMEM", "KVQ_ECAPACITY", "KVQ_ESTATE", "KVQ_EHIP"]):
        assert L.kvq_status_str(s).decode() == name
    assert L.kvq_status_str(99).decode() == "KVQ_UNKNOWN"


def test_oracle_and_product_share_no_code():
    # the product package never imports the oracle, and the oracle never imports the product
    # or the input generator
    imp = re.compile(r"^\s*(from|import)\s+([\w.]+)", re.M)
    inc = re.compile(r'^\s*#\s*include\s*[<"]([^>"]+)[>"]', re.M)
    pkg = os.path.join(ROOT, "rope_aware_bit_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            txt = open(os.path.join(dirpath, f), errors="ignore").read() if f.endswith(
                (".py", ".hip", ".cpp", ".h")) else ""
            mods = [m[1] for m in imp.findall(txt)] + inc.findall(txt)
            assert not any("oracle" in m for m in mods), (f, mods)
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            mods = [m[1] for m in imp.findall(open(os.path.join(ROOT, "oracle", f)).read())]
            assert not any(m.startswith(("rope_aware_bit_amd", "synth", "torch")) for m in mods), (f, mods)
