"""Plain, slow CPU oracle for the packed-KV hot path — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The product path
(``rope_aware_bit_amd``) never imports it and shares no code, table or
constant generator with it; the only thing both sides consume is the seeded
input generator in ``synth/``.

The oracle follows the method of "RoPE-Aware Bit Allocation for
KV-Cache Quantization" (Liang, Zhang, Jia; arXiv 2606.24033, abstract) and the
comparison codec of "NQKV: A KV Cache Quantization Scheme Based on Normal
Distribution Characteristics" (Pith review of arXiv 2505.16210: "What carries
the argument", referee major comment 1, Figures 4-5).  Floating point is fp64
unless a step is defined in IEEE fp32/fp16 (the quantizer's scale chain),
in which case numpy's correctly rounded fp32/fp16 operations are used in the
stated order.

Modules
-------
codebooks   Gaussian Lloyd-Max codebooks, their exact MSE, the greedy's
            per-bit gains delta(b), and the 16-level Gaussian-quantile codebook.
allocation  per-RoPE-block energy score, per-block gains, greedy allocation,
            field (plan) order.
quantize    per-row scale, codebook lookup; the per-256-value absmax codec.
layout      bit packing of K rows and dim-major V tiles, and unpacking.
attention   dequantization, fp64 GQA decode attention, RoPE block identity,
            compression arithmetic.
fidelity    logit MAE and softmax KL of stored keys against the given ones.
window      which positions pass through the fp16 recent window; packed length
            (also in whole 128-position groups).
rotation    randomized Hadamard rotations: of the whole row, and inside the
            plan's equal-width groups.
kivi        the KIVI-style asymmetric integer codec (keys per channel over
            128-position tiles, values per position) and its parameter layout.
codecs      each codec of the cache as one chain of the steps above, per KV head
            (Block-GTQ keys and values, rotated uniform, group-rotated Block-GTQ,
            the 256-value absmax codec's per-head slices).

Every function is pinned by a ``-m "not gpu"`` test against something other
than itself (closed forms, textbook values, library routines, brute force or
invariants); see tests/test_oracle_*.py.
"""
from . import codebooks, allocation, quantize, layout, attention  # noqa: F401
from . import fidelity, window, rotation, kivi, codecs  # noqa: F401
