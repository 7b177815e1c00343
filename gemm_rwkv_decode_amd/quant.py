"""Offline CPU quantizer: real-valued weights -> the packed layouts of include/rq.h.

The step before the hot path.  Every layout the library reads can be produced:

* symmetric 4-bit (groups of 32/64/128) and 8-bit (groups of 16/32/64) codes
  with one binary16 scale per group (w ~ s*q);
* asymmetric superblocks of 256 weights with 4-, 5- or 6-bit unsigned codes,
  a scale and a shift per 32-wide group stored as 6-bit sub-codes of a
  binary16 superblock scale and min (w ~ (d*sc_j)*q - (m*mn_j));
* FP8 E4M3 codes with one binary32 scale for the matrix.

Two ways to choose the per-group scale (and shift):

* ``"rtn"``: round to nearest on the full range of the group (symmetric:
  s = max|w| / qmax; asymmetric: the range [min(0, min w), max w]);
* ``"search"``: the rwkv-quant presets' rule (news article "rwkv-quant:
  keeping one matrix in bf16 ...", section "Two presets and six sizes"): the
  scale and shift of each group are chosen by a search weighted by the mean
  square of each input channel's activation, E[x^2].  Candidates shrink the
  group's range (symmetric: s = f * max|w| / qmax; asymmetric: the low and
  the high end independently), each is quantized by round to nearest, and the
  candidate with the least sum_k E[x_k^2] (w_k - w^_k)^2 wins.  With E[x^2]
  = 1 this is a plain mean-square search.  The full range is always a
  candidate, so the search never does worse than RTN on its own measure
  (asymmetric: before the superblock records round the chosen scale and
  shift to 6-bit sub-codes, which both methods then share).

FP8 follows the FP8 package page (section "Quantization Principle"):
scale = max|W| / 448, codes = float8_e4m3fn(clamp(W / scale, -448, 448)).

All arithmetic is float64 numpy on the host except the stored rounding steps
(binary16 scales, binary32 FP8 scale), which are applied where the format
stores them, so the weights the library dequantizes are the ones the search
scored.  The result is a ``synth.Packed`` on the CPU (``.to`` it as needed).
"""
from typing import Optional

import numpy as np
import torch

from . import synth as S

SYM_QMAX = {4: 7, 8: 127}
SUPERBLOCK = 256
SB_GROUP = 32
SUB_MAX = 63  # 6-bit sub-codes of the superblock records

# range factors tried by the search (1.0, the RTN choice, comes first)
SYM_FACTORS = np.linspace(1.0, 0.70, 16)
ASYM_FACTORS = np.array([1.0, 0.97, 0.94, 0.90, 0.86, 0.80])


def _f16(a):
    return np.asarray(a, dtype=np.float64).astype(np.float16).astype(np.float64)


def _weights(xsq, K):
    if xsq is None:
        return np.ones(K)
    w = np.asarray(xsq, dtype=np.float64).reshape(-1)
    if w.shape != (K,) or not np.all(np.isfinite(w)) or np.any(w < 0):
        raise ValueError("xsq must hold K finite non-negative values (E[x^2] per input channel)")
    return w


def quantize(W, fmt: "S.Fmt", xsq: Optional[np.ndarray] = None, method: str = "search"):
    """Quantize ``W`` (float [N][K], rows = outputs) to ``fmt``.

    ``xsq``: E[x^2] per input channel (length K), weighting the search;
    ``None`` weights every channel equally.  ``method``: ``"rtn"`` or
    ``"search"``.  Returns ``synth.Packed`` on the CPU."""
    W = np.asarray(W.detach().cpu().numpy() if torch.is_tensor(W) else W, dtype=np.float64)
    if W.ndim != 2 or not np.all(np.isfinite(W)):
        raise ValueError("W must be a finite 2-D array")
    if method not in ("rtn", "search"):
        raise ValueError(f"unknown method {method!r}")
    N, K = W.shape
    if fmt.layout == S.LAYOUT_FP8_TENSOR:
        return _fp8(W, fmt)
    xw = _weights(xsq, K)
    if fmt.layout == S.LAYOUT_SYM:
        return _sym(W, fmt, xw, method)
    return _asym(W, fmt, xw, method)


# ------------------------------------------------------------------ symmetric
def _sym(W, fmt, xw, method):
    N, K = W.shape
    g = fmt.group
    if fmt.bits not in SYM_QMAX or K % g:
        raise ValueError("symmetric layout: 4- or 8-bit codes and K a multiple of the group")
    qmax = SYM_QMAX[fmt.bits]
    Wg = W.reshape(N, K // g, g)
    xg = xw.reshape(1, K // g, g)
    amax = np.abs(Wg).max(axis=2)
    factors = SYM_FACTORS if method == "search" else SYM_FACTORS[:1]
    best_s = best_q = best_e = None
    for f in factors:
        s = _f16(amax * f / qmax)  # stored as binary16
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.where(s[..., None] > 0, np.rint(Wg / s[..., None]), 0.0)
        q = np.clip(q, -qmax, qmax)
        e = (xg * (Wg - s[..., None] * q) ** 2).sum(axis=2)
        if best_e is None:
            best_s, best_q, best_e = s, q, e
        else:
            take = e < best_e
            best_s = np.where(take, s, best_s)
            best_q = np.where(take[..., None], q, best_q)
            best_e = np.where(take, e, best_e)
    codes = torch.from_numpy(best_q.reshape(N, K).astype(np.int8))
    scales = torch.from_numpy(best_s.astype(np.float16))
    return S.encode(codes, fmt, scales=scales)


# ----------------------------------------------------------------- asymmetric
def _asym_group_fit(Wg, xg, qmax, method):
    """Per 32-wide group: (s, t) >= 0 before the records are quantized."""
    lo = np.minimum(Wg.min(axis=-1), 0.0)
    hi = np.maximum(Wg.max(axis=-1), 0.0)
    fa = ASYM_FACTORS if method == "search" else ASYM_FACTORS[:1]
    best = None
    for a in fa:
        for b in fa:
            l, h = lo * a, hi * b
            s = (h - l) / qmax
            t = -l
            with np.errstate(divide="ignore", invalid="ignore"):
                q = np.where(s[..., None] > 0, np.rint((Wg + t[..., None]) / s[..., None]), 0.0)
            q = np.clip(q, 0, qmax)
            e = (xg * (Wg - (s[..., None] * q - t[..., None])) ** 2).sum(axis=-1)
            if best is None:
                best = [s, t, e]
            else:
                take = e < best[2]
                best = [np.where(take, s, best[0]), np.where(take, t, best[1]),
                        np.where(take, e, best[2])]
    return best[0], best[1]


def _records(v):
    """Per superblock: v [..., 8] >= 0 -> (binary16 base, 6-bit sub-codes) with
    base * sub ~ v."""
    base = _f16(v.max(axis=-1) / SUB_MAX)
    with np.errstate(divide="ignore", invalid="ignore"):
        sub = np.where(base[..., None] > 0, np.rint(v / base[..., None]), 0.0)
    return base, np.clip(sub, 0, SUB_MAX)


def _asym(W, fmt, xw, method):
    N, K = W.shape
    if fmt.bits not in (4, 5, 6) or fmt.group != SB_GROUP or K % SUPERBLOCK:
        raise ValueError("asymmetric layout: 4-, 5- or 6-bit codes, group 32, K a multiple of 256")
    qmax = (1 << fmt.bits) - 1
    B = K // SUPERBLOCK
    Wg = W.reshape(N, B, 8, SB_GROUP)
    xg = xw.reshape(1, B, 8, SB_GROUP)
    s, t = _asym_group_fit(Wg, xg, qmax, method)
    d, sc = _records(s)
    m, mn = _records(t)
    s_hat = d[..., None] * sc  # the values the library decodes, exactly
    t_hat = m[..., None] * mn
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s_hat[..., None] > 0,
                     np.rint((Wg + t_hat[..., None]) / s_hat[..., None]), 0.0)
    q = np.clip(q, 0, qmax)
    codes = torch.from_numpy(q.reshape(N, K).astype(np.int8))
    return S.encode(codes, fmt,
                    d=torch.from_numpy(d.astype(np.float16)),
                    sc=torch.from_numpy(sc.astype(np.uint8)),
                    m=torch.from_numpy(m.astype(np.float16)),
                    mn=torch.from_numpy(mn.astype(np.uint8)))


# ------------------------------------------------------------------------ FP8
def _fp8(W, fmt):
    N, K = W.shape
    Wt = torch.from_numpy(W.astype(np.float32))
    scale = (Wt.abs().max() / 448.0).reshape(1).to(torch.float32)
    if scale.item() == 0.0:
        codes = torch.zeros((N, K), dtype=torch.uint8)
    else:
        codes = (Wt / scale).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    return S.Packed(codes.contiguous(), scale, None, N, K, fmt)

