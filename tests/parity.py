"""Helpers for GPU-vs-oracle parity tests (imported by the -m gpu tests and smoke()).

The oracle side quantizes the same seeded inputs on its own; nothing it
compares against comes from the GPU path except the GPU results under test.
"""
from __future__ import annotations

import numpy as np

from oracle import allocation as al
from oracle import codecs as cd
from oracle import kivi as kv
from oracle import layout as lay

PAIRING = {"half": 0, "interleaved": 1}
CODEC = {"bgtq": 0, "uniform": 1, "nf16": 2, "rot": 3, "kivi": 4, "bgtq_rot": 5}

ABS_TOL = 2e-3
REL_L2_TOL = 1e-3


def errors(gpu: np.ndarray, ref: np.ndarray):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    max_abs = float(np.max(np.abs(g - r))) if g.size else 0.0
    rel_l2 = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
    return max_abs, rel_l2


def assert_attention_close(gpu, ref, what=""):
    max_abs, rel_l2 = errors(gpu, ref)
    assert max_abs <= ABS_TOL and rel_l2 <= REL_L2_TOL, f"{what}: max_abs={max_abs:.3e} rel_l2={rel_l2:.3e}"
    return max_abs, rel_l2


class OracleLayer:
    """Oracle plan, codes, packed words and dequantized cache for one layer."""

    def __init__(self, calib, k_bits, v_bits, codec="bgtq", pairing="half", b_min=0, b_max=8,
                 block_weight=None, signs=None):
        self.k_bits, self.v_bits, self.codec, self.pairing = k_bits, v_bits, codec, pairing
        self.signs = signs   # key-rotation signs [H, 128] of the rotated codec
        H = calib.shape[1] if calib is not None else None
        if codec in ("bgtq", "bgtq_rot"):
            self.widths, self.g, self.ig, self.m = al.allocate(calib, k_bits, b_min, b_max, pairing,
                                                               block_weight=block_weight)
        else:
            kb = 4 if codec == "nf16" else k_bits
            self.widths = np.full((H, 64), kb, dtype=np.int64)
            self.g = np.ones((H, 64), np.float32)
            self.ig = np.ones((H, 64), np.float32)
        self.H = self.widths.shape[0]

    def fields(self, h):
        return al.field_order(self.widths[h], 128, self.pairing)

    def quantize_head(self, k_rows, v_rows, h, k_tok_all=None, v_tok_all=None):
        """Quantize rows of head h: k_rows, v_rows [N, 128].  For nf16, *_tok_all are the
        tokens' full [N, H*128] vectors.  Returns dict of codes, scales, words."""
        out = {}
        wid, pr = self.widths[h], self.pairing
        if self.codec == "nf16":
            ck, sk = cd.quantize_nf16_tokens(k_tok_all)
            cv, sv = cd.quantize_nf16_tokens(v_tok_all)
            out["k_codes"], out["k_s16"] = cd.nf16_head_slice(ck, sk, h)
            out["v_codes"], out["v_s16"] = cd.nf16_head_slice(cv, sv, h)
            out["k_scale_blocks"], out["v_scale_blocks"] = sk, sv
        elif self.codec == "kivi":
            # keys per channel over whole 128-position tiles, values per position
            ck, sk, lk = kv.quantize_k(k_rows, self.k_bits)
            cv, sv, lv = kv.quantize_v(v_rows, self.v_bits)
            out.update(k_codes=ck, k_s16=sk, k_lo16=lk, v_codes=cv, v_s16=sv, v_lo16=lv)
            out["k_params"] = kv.k_params_layout(sk, lk, self.pairing)
            out["v_params"] = kv.v_params_layout(sv, lv)
        else:
            if self.codec == "rot":
                ck, sk = cd.quantize_rotated_uniform(k_rows, self.k_bits, self.signs[h])
            elif self.codec == "bgtq_rot":
                ck, sk = cd.quantize_bgtq_group_rotated(k_rows, wid, self.ig[h], self.signs[h], pr)
            else:
                ck, sk = cd.quantize_bgtq_keys(k_rows, wid, self.ig[h], pr)
            cv, sv = cd.quantize_values(v_rows, self.v_bits)
            out.update(k_codes=ck, k_s16=sk, v_codes=cv, v_s16=sv)
        dims, ws = self.fields(h)
        kb = 4 if self.codec == "nf16" else self.k_bits
        out["k_words"] = lay.pack_k_rows(out["k_codes"], dims, ws, 4 * kb)
        return out

    def dequant(self, q_out, h):
        wid, pr = self.widths[h], self.pairing
        if self.codec == "kivi":
            return (kv.dequant_k(q_out["k_codes"], q_out["k_s16"], q_out["k_lo16"]),
                    kv.dequant_v(q_out["v_codes"], q_out["v_s16"], q_out["v_lo16"]))
        if self.codec == "nf16":
            return (cd.dequant_nf16_head(q_out["k_codes"], q_out["k_s16"]),
                    cd.dequant_nf16_head(q_out["v_codes"], q_out["v_s16"]))
        if self.codec == "bgtq_rot":
            kh = cd.dequant_bgtq_group_rotated(q_out["k_codes"], q_out["k_s16"], wid, self.g[h],
                                               self.signs[h], pr)
        elif self.codec == "rot":
            kh = cd.dequant_rotated_uniform(q_out["k_codes"], q_out["k_s16"], self.k_bits, self.signs[h])
        else:
            kh = cd.dequant_bgtq_keys(q_out["k_codes"], q_out["k_s16"], wid, self.g[h], pr)
        vh = cd.dequant_values(q_out["v_codes"], q_out["v_s16"], self.v_bits)
        return kh, vh
