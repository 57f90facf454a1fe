"""Helpers for GPU-vs-oracle parity tests (imported by the -m gpu tests and smoke()).

The oracle side quantizes the same seeded inputs on its own; nothing it
compares against comes from the GPU path except the GPU results under test.
"""
from __future__ import annotations

import numpy as np

from oracle import allocation as al
from oracle import attention as at
from oracle import kivi as kv
from oracle import layout as lay
from oracle import quantize as qz
from oracle import rotation as rt

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
        if self.codec == "nf16":
            ck, sk, _ = qz.quantize_nf16(k_tok_all)
            cv, sv, _ = qz.quantize_nf16(v_tok_all)
            out["k_codes"] = ck[:, h * 128:(h + 1) * 128]
            out["v_codes"] = cv[:, h * 128:(h + 1) * 128]
            out["k_scale_blocks"], out["v_scale_blocks"] = sk, sv
            out["k_s16"] = sk[:, h // 2]
            out["v_s16"] = sv[:, h // 2]
        elif self.codec == "kivi":
            # keys per channel over whole 128-position tiles, values per position
            ck, sk, lk = kv.quantize_k(k_rows, self.k_bits)
            cv, sv, lv = kv.quantize_v(v_rows, self.v_bits)
            out.update(k_codes=ck, k_s16=sk, k_lo16=lk, v_codes=cv, v_s16=sv, v_lo16=lv)
            out["k_params"] = kv.k_params_layout(sk, lk, self.pairing)
            out["v_params"] = kv.v_params_layout(sv, lv)
        else:
            wd = al.dim_widths(self.widths[h], 128, self.pairing)
            igd = al.dim_values(self.ig[h], 128, self.pairing)
            if self.codec == "rot":
                ck, sk, _ = qz.quantize_rows(rt.rotate_rows_fp32(k_rows, self.signs[h]), wd)
            elif self.codec == "bgtq_rot":
                # gain-normalised rows, rotated inside the equal-width groups, then quantized
                # with unit gains
                y32 = (np.asarray(k_rows).astype(np.float32) * igd.astype(np.float32)[None, :]).astype(np.float32)
                dims, ws = self.fields(h)
                yr = rt.rotate_in_groups(y32.astype(np.float64), self.signs[h], dims, ws).astype(np.float32)
                ck, sk, _ = qz.quantize_rows(yr, wd)
            else:
                ck, sk, _ = qz.quantize_rows(k_rows, wd, igd)
            cv, sv, _ = qz.quantize_rows(v_rows, np.full(128, self.v_bits))
            out.update(k_codes=ck, k_s16=sk, v_codes=cv, v_s16=sv)
        dims, ws = self.fields(h)
        kb = 4 if self.codec == "nf16" else self.k_bits
        out["k_words"] = lay.pack_k_rows(out["k_codes"], dims, ws, 4 * kb)
        return out

    def dequant(self, q_out, h):
        if self.codec == "kivi":
            return (kv.dequant_k(q_out["k_codes"], q_out["k_s16"], q_out["k_lo16"]),
                    kv.dequant_v(q_out["v_codes"], q_out["v_s16"], q_out["v_lo16"]))
        if self.codec == "nf16":
            lv = at.dequant_nf16(q_out["k_codes"], q_out["k_s16"][:, None], block=128)
            vv = at.dequant_nf16(q_out["v_codes"], q_out["v_s16"][:, None], block=128)
            return lv, vv
        wd = al.dim_widths(self.widths[h], 128, self.pairing)
        gd = al.dim_values(self.g[h], 128, self.pairing)
        if self.codec == "bgtq_rot":
            dims, ws = self.fields(h)
            kh = at.dequant_k(q_out["k_codes"], q_out["k_s16"], wd, np.ones(128, np.float32))
            kh = rt.unrotate_in_groups(kh, self.signs[h], dims, ws) * gd.astype(np.float64)[None, :]
        else:
            kh = at.dequant_k(q_out["k_codes"], q_out["k_s16"], wd, gd)
        if self.codec == "rot":
            kh = rt.unrotate(kh, self.signs[h])
        vh = at.dequant_v(q_out["v_codes"], q_out["v_s16"], self.v_bits)
        return kh, vh


def flips_excused(gpu_codes, ref_codes, u, width_dim, bounds_of):
    """Count code mismatches and check each lies within 1 ulp of a boundary of the oracle's u."""
    bad = np.argwhere(gpu_codes != ref_codes)
    excused = 0
    for r, i in bad:
        w = int(width_dim[i])
        bd = bounds_of(w)
        uu = np.float32(u[r, i])
        ulp = np.spacing(np.abs(uu))
        if np.min(np.abs(bd.astype(np.float64) - float(uu))) <= float(ulp):
            excused += 1
    return len(bad), excused
