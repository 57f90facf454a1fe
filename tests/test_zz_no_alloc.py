"""kvq_decode_attn_noalloc (split scratch in the library's fixed device array) against
kvq_decode_attn on the same caches, through the C ABI: two calls in a row, the second on a
smaller input, then the separate-merge path and the scratch limit."""
import numpy as np
import pytest

from synth import WORKLOADS, gen_layer, gen_query
from tests.parity import assert_attention_close

pytestmark = pytest.mark.gpu


def _setup(wname, T, batch, k_bits, v_bits, recent=0):
    import torch
    from rope_aware_bit_amd import kvq
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    w = WORKLOADS[wname]
    dev = torch.device("cuda:0")
    k, v = gen_layer(w, 0, 0, T)
    K = torch.from_numpy(np.repeat(k[None], batch, axis=0)).to(dev)
    V = torch.from_numpy(np.repeat(v[None], batch, axis=0)).to(dev)
    q = torch.from_numpy(np.stack([gen_query(w, 0, T, seq=b) for b in range(batch)])).to(dev)
    cache = kvq.Cache(kvq.Config(1, w.n_kv, w.n_q, batch, T, k_bits, v_bits, recent_window=recent))
    cache.alloc_bits(0, K[0, :min(T, 2048)].contiguous())
    cache.quantize_append(0, K, V)
    return cache, q


def _compare(cache, q):
    import torch
    want = cache.decode_attn(0, q)
    got = torch.full_like(want, float("nan"))
    cache.decode_attn_noalloc(0, q, got)
    torch.cuda.synchronize()
    g, r = got.cpu().numpy(), want.cpu().numpy()
    assert np.isfinite(g).all()
    # same kernels, same split count and merge order: the very same numbers
    assert np.array_equal(g.view(np.uint32), r.view(np.uint32))
    assert_attention_close(g, r, "noalloc vs decode_attn")
    cache.status()


def test_noalloc_matches_decode_attn_twice_then_smaller():
    # first call: a 20000-position Qwen-shaped layer (several splits merged in the kernel)
    c1, q1 = _setup("qwen3b_128k", 20000, 1, 3, 3)
    _compare(c1, q1)
    _compare(c1, q1)
    c1.close()
    # second call on a smaller input (fewer positions, two sequences, K3V2): the array still
    # holds the first call's words
    c2, q2 = _setup("qwen3b_128k", 3000, 2, 3, 2)
    _compare(c2, q2)
    c2.close()


def test_noalloc_separate_merge_and_limit():
    from rope_aware_bit_amd import kvq
    # 32 sequences x 8 KV heads with a window: merged by the separate kernel
    c3, q3 = _setup("llama8b_b64", 700, 32, 4, 4, recent=128)
    _compare(c3, q3)
    c3.close()
    # a 4096-position window at 256 units needs more than the 8 MiB of scratch: refused
    c4, q4 = _setup("llama8b_b64", 4200, 32, 4, 4, recent=4096)
    import torch
    out = torch.empty(q4.shape, dtype=torch.float32, device=q4.device)
    with pytest.raises(kvq.KvqError) as e:
        c4.decode_attn_noalloc(0, q4, out)
    assert e.value.status == kvq.KVQ_EINVAL and "8388608" in str(e.value)
    c4.close()
