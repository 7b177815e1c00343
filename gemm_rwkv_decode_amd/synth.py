"""Seeded synthetic inputs shaped like RWKV-7 decode projections.

This module holds only input generation and the byte encoding of the packed
formats (code packing and superblock records).  It decodes nothing and holds
none of the dequantize-or-multiply arithmetic; both the GPU path and the CPU
oracle consume what it produces.

Shapes and statistics follow the pages:

* model sizes (layers x width): 0.1B 12x768, 1.5B 24x2048, 2.9B 32x2560,
  13.3B 61x4096 (news article "rwkv-quant: keeping one matrix in bf16 ...",
  section "Two presets and six sizes");
* six quantized matrices per layer -- receptance, key, value, output and the
  FFN key/value (package page "RWKV-7 FP8 Quantized Inference", section
  "Core Approach: Full FP8, No Residuals"); weights are stored [out][in], the
  FFN key is 4D x D and the FFN value D x 4D (same page, section "Operator
  Optimization Details");
* massive activation channels: on the 2.9B model eight channels carry 98% of
  the energy, including channel 517; on 1.5B the channel is 1202; 7.2B
  reaches 99% (news article, section "Where 2.9B breaks");
* the vocabulary head is 65536 x 4096 (package page, section "Why is
  head.weight not quantized?").

Every random tensor comes from its own ``torch.Generator`` whose seed is the
first 8 bytes (little endian, masked to 63 bits) of
``sha256("rq/{workload}/l{layer}/m{matrix}/{role}/{format}/M{M}")``.  The same
seed on a CPU generator and on a GPU generator gives different (but equally
seeded) streams; a test compares a GPU result with the oracle on the very
tensors the GPU consumed.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass
from typing import Dict, List, Optional, Tuple

import torch

LAYOUT_SYM = 0
LAYOUT_ASYM_SB = 1
LAYOUT_FP8_TENSOR = 2
SUPERBLOCK = 256


@dataclass(frozen=True)
class Fmt:
    tag: str
    bits: int
    group: int
    layout: int

    def code_range(self) -> Tuple[int, int]:
        """Inclusive range of the codes the generators emit."""
        if self.layout == LAYOUT_ASYM_SB:
            return 0, (1 << self.bits) - 1
        return (-7, 7) if self.bits == 4 else (-127, 127)

    def weight_bytes(self, N: int, K: int) -> int:
        """Packed code bytes plus scale (and zero) bytes of an N x K matrix."""
        codes = N * K * self.bits // 8
        if self.layout == LAYOUT_FP8_TENSOR:
            return codes + 4  # one binary32 scale
        if self.layout == LAYOUT_ASYM_SB:
            return codes + 2 * 8 * N * (K // SUPERBLOCK)
        return codes + 2 * N * (K // self.group)


INT4_G64 = Fmt("int4g64", 4, 64, LAYOUT_SYM)
INT8_G16 = Fmt("int8g16", 8, 16, LAYOUT_SYM)
ASYM4_G32 = Fmt("asym4g32", 4, 32, LAYOUT_ASYM_SB)
# FP8 E4M3 weights with one binary32 scale per matrix (package page "RWKV-7
# FP8 Quantized Inference", section "Quantization Principle")
FP8_E4M3 = Fmt("fp8e4m3", 8, 0, LAYOUT_FP8_TENSOR)
# 5- and 6-bit codes in the asymmetric superblock layout (news article
# "rwkv-quant: ...", section "Two presets and six sizes": FFN key and head in
# 5 bits, FFN in 6 bits)
ASYM5_G32 = Fmt("asym5g32", 5, 32, LAYOUT_ASYM_SB)
ASYM6_G32 = Fmt("asym6g32", 6, 32, LAYOUT_ASYM_SB)
FORMATS = {f.tag: f for f in (INT4_G64, INT8_G16, ASYM4_G32, FP8_E4M3, ASYM5_G32, ASYM6_G32)}

MAT_NAMES = ("att.receptance", "att.key", "att.value", "att.output",
             "ffn.key", "ffn.value", "head")


@dataclass(frozen=True)
class XSpec:
    """Activation recipe: N(0,1) plus optional massive channels."""
    kind: str                 # "plain" | "fixed" | "energy"
    channel: int = -1         # "fixed": the channel index
    factor: float = 1.0       # "fixed": literal multiplier
    forced: Tuple[int, ...] = ()  # "energy": channels always in the set
    count: int = 0            # "energy": number of massive channels
    share: float = 0.0        # "energy": expected energy share they carry


@dataclass(frozen=True)
class Config:
    key: str                  # short workload name, also part of every seed
    name: str
    width: int
    layers: int
    formats: Tuple[Fmt, ...]
    ms: Tuple[int, ...]
    x: XSpec
    single: bool = False      # one matrix only (N = K = width)
    head: bool = False        # the step includes the 65536 x width head

    def matrices(self, with_head: Optional[bool] = None) -> List[Tuple[int, int, int, int]]:
        """(layer, mat, N, K) for one decode step, in execution order; the head
        (mat 6) is listed as layer `layers` when included (default: the
        workload's own choice)."""
        if with_head is None:
            with_head = self.head
        D = self.width
        if self.single:
            return [(0, 0, D, D)]
        shapes = [(D, D), (D, D), (D, D), (D, D), (4 * D, D), (D, 4 * D)]
        out = [(l, m, n, k) for l in range(self.layers)
               for m, (n, k) in enumerate(shapes)]
        if with_head:
            out.append((self.layers, 6, 65536, D))
        return out

    def step_weight_bytes(self, fmt: Fmt, with_head: Optional[bool] = None) -> int:
        return sum(fmt.weight_bytes(n, k) for _, _, n, k in self.matrices(with_head))


_WORKLOADS = (
    Config("gemv768", "single int4-g64 GEMV, 768x768", 768, 1, (INT4_G64,), (1,),
           XSpec("plain"), single=True),
    Config("rwkv7-0.1b", "RWKV-7 0.1B-shaped decode sweep", 768, 12, (INT4_G64,), (1,),
           XSpec("fixed", channel=300, factor=50.0)),
    Config("rwkv7-1.5b", "RWKV-7 1.5B-shaped projections", 2048, 24, (INT8_G16, INT4_G64),
           (1, 4, 16, 32), XSpec("fixed", channel=1202, factor=50.0)),
    Config("rwkv7-2.9b", "RWKV-7 2.9B-shaped projections, asymmetric", 2560, 32,
           (ASYM4_G32,), (1, 8, 32), XSpec("energy", forced=(517,), count=8, share=0.98)),
    Config("rwkv7-13.3b", "RWKV-7 13.3B-shaped projections and head", 4096, 61,
           (INT4_G64,), (1, 16, 32, 64), XSpec("energy", count=8, share=0.99), head=True),
)
# the workloads by name, smallest first
CONFIGS: Dict[str, Config] = {c.key: c for c in _WORKLOADS}


# --------------------------------------------------------------------------
# seeds
# --------------------------------------------------------------------------
def seed_for(wkey: str, layer: int, mat: int, role: str, fmt_tag: str, M: int) -> int:
    key = f"rq/{wkey}/l{layer}/m{mat}/{role}/{fmt_tag}/M{M}".encode()
    return int.from_bytes(hashlib.sha256(key).digest()[:8], "little") & ((1 << 63) - 1)


def generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(seed)
    return g


# --------------------------------------------------------------------------
# byte encodings of the formats
# --------------------------------------------------------------------------
def pack_nibbles(codes: torch.Tensor) -> torch.Tensor:
    """int codes [N][K] (each within -8..15) -> uint8 [N][K/2].

    The even k goes to bits 0-3 and the odd k to bits 4-7; a negative code is
    stored as its 4-bit two's complement."""
    c = codes.to(torch.int16)
    lo = c[:, 0::2] & 0xF
    hi = c[:, 1::2] & 0xF
    return (lo | (hi << 4)).to(torch.uint8).contiguous()


# high-bit placement of 5-/6-bit codes: shift of a (nibble dword i, g) group
_HI5 = lambda i, g: i - 4 if g == 0 else i + 4  # noqa: E731
_HI6 = ((-4, -2), (4, 6))


def pack_hi_planes(codes: torch.Tensor, bits: int) -> torch.Tensor:
    """Unsigned codes [N][K] (0..2^bits-1, bits 5 or 6) -> flat uint8: the low
    nibbles as the 4-bit layout stores them ([N][K/2]), then the high-bit
    plane: per row, per 32-code chunk, 1 (5-bit) or 2 (6-bit) little-endian
    dwords; code 8i+j of a chunk with base = (j >= 4 ? 16 : 0) + (j even ? 4 :
    8) and g = (j mod 4) / 2 has bit 4 at bit base + (g == 0 ? i-4 : i+4) of
    the chunk's dword (5-bit), or bits 4 and 5 at base + s and base + 1 + s of
    dword i/2, s = -4, -2, 4, 6 for (i mod 2, g) = (0,0), (0,1), (1,0), (1,1)
    (6-bit)."""
    N, K = codes.shape
    hb = bits - 4
    c = codes.to(torch.int64)
    nib = pack_nibbles(c & 0xF)
    hi = (c >> 4).reshape(N, K // 32, 4, 8)
    words = torch.zeros((N, K // 32, hb), dtype=torch.int64, device=codes.device)
    for i in range(4):
        for j in range(8):
            g = (j % 4) // 2
            base = (16 if j >= 4 else 0) + (4 if j % 2 == 0 else 8)
            for b in range(hb):
                if hb == 1:
                    w, pos = 0, base + _HI5(i, g)
                else:
                    w, pos = i // 2, base + b + _HI6[i % 2][g]
                words[:, :, w] |= ((hi[:, :, i, j] >> b) & 1) << pos
    plane = torch.stack([(words >> (8 * t)) & 0xFF for t in range(4)], dim=-1)
    return torch.cat([nib.reshape(-1), plane.to(torch.uint8).reshape(-1)]).contiguous()


def pack_records(base: torch.Tensor, sub: torch.Tensor) -> torch.Tensor:
    """base float16 [N][B], sub uint8 [N][B][8] (0..63) -> uint8 [N][B][8].

    Bytes 0-1 hold the binary16 base (little endian); bytes 2-7 hold a 48-bit
    little-endian field with sub-code j at bits 6j..6j+5."""
    N, B = base.shape
    bits = base.contiguous().view(torch.int16).to(torch.int64) & 0xFFFF
    field = torch.zeros((N, B), dtype=torch.int64, device=base.device)
    for j in range(8):
        field |= sub[:, :, j].to(torch.int64) << (6 * j)
    out = torch.empty((N, B, 8), dtype=torch.uint8, device=base.device)
    out[:, :, 0] = (bits & 0xFF).to(torch.uint8)
    out[:, :, 1] = ((bits >> 8) & 0xFF).to(torch.uint8)
    for i in range(6):
        out[:, :, 2 + i] = ((field >> (8 * i)) & 0xFF).to(torch.uint8)
    return out.contiguous()


# --------------------------------------------------------------------------
# value distributions
# --------------------------------------------------------------------------
def log_uniform_half(shape, lo: float, hi: float, g: torch.Generator, device):
    """exp(U(ln lo, ln hi)) computed in fp32, rounded once to binary16."""
    u = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    return torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))).half()


def gen_codes(N: int, K: int, fmt: Fmt, g: torch.Generator, device) -> torch.Tensor:
    lo, hi = fmt.code_range()
    return torch.randint(lo, hi + 1, (N, K), generator=g, device=device,
                         dtype=torch.int16).to(torch.int8)


@dataclass
class Packed:
    qweight: torch.Tensor            # uint8 [N][K/2] or int8 [N][K]
    scales: torch.Tensor             # float16 [N][K/g] or uint8 [N][K/256][8]
    zeros: Optional[torch.Tensor]    # None or uint8 [N][K/256][8]
    N: int
    K: int
    fmt: Fmt


def encode(codes: torch.Tensor, fmt: Fmt, scales=None, d=None, sc=None, m=None,
           mn=None) -> Packed:
    """Pack explicit codes and scale material into the stored format."""
    N, K = codes.shape
    if fmt.bits == 8:
        qw = codes.to(torch.int8).contiguous()
    elif fmt.bits in (5, 6):
        qw = pack_hi_planes(codes, fmt.bits)
    else:
        qw = pack_nibbles(codes)
    if fmt.layout == LAYOUT_SYM:
        return Packed(qw, scales.half().contiguous(), None, N, K, fmt)
    return Packed(qw, pack_records(d, sc), pack_records(m, mn), N, K, fmt)


def gen_matrix(wkey: str, layer: int, mat: int, N: int, K: int, fmt: Fmt,
               device="cpu", keep_codes: bool = False):
    """Seeded packed weights for one matrix.  Returns ``Packed`` (and the
    unpacked int8 codes when ``keep_codes``)."""
    dev = torch.device(device)
    if fmt.layout == LAYOUT_FP8_TENSOR:
        return gen_fp8_matrix(wkey, layer, mat, N, K, fmt, dev, keep_codes)
    gc = generator(seed_for(wkey, layer, mat, "codes", fmt.tag, 0), dev)
    codes = gen_codes(N, K, fmt, gc, dev)
    gs = generator(seed_for(wkey, layer, mat, "scales", fmt.tag, 0), dev)
    if fmt.layout == LAYOUT_SYM:
        scales = log_uniform_half((N, K // fmt.group), 1e-3, 1e-1, gs, dev)
        p = encode(codes, fmt, scales=scales)
    else:
        B = K // SUPERBLOCK
        d = log_uniform_half((N, B), 1e-4, 2e-3, gs, dev)
        sc = torch.randint(0, 64, (N, B, 8), generator=gs, device=dev,
                           dtype=torch.int16).to(torch.uint8)
        gz = generator(seed_for(wkey, layer, mat, "zeros", fmt.tag, 0), dev)
        m = log_uniform_half((N, B), 1e-4, 2e-3, gz, dev)
        mn = torch.randint(0, 64, (N, B, 8), generator=gz, device=dev,
                           dtype=torch.int16).to(torch.uint8)
        p = encode(codes, fmt, d=d, sc=sc, m=m, mn=mn)
    if keep_codes:
        return p, codes
    del codes
    return p


def gen_fp8_matrix(wkey: str, layer: int, mat: int, N: int, K: int, fmt: Fmt, dev,
                   keep_codes: bool = False):
    """FP8 weights by the page's per-tensor recipe: real-valued weights (normal,
    with a log-normal magnitude per row), scale = max|W| / 448, codes =
    float8_e4m3fn(clamp(W / scale, -448, 448)).  The weights are drawn on the
    CPU in row blocks (seeded per block), so the bytes do not depend on the
    device; the cast is torch's."""
    codes = torch.empty((N, K), dtype=torch.uint8)
    mags = []
    rows_per = max(1, (1 << 24) // K)
    blocks = []
    for b, r0 in enumerate(range(0, N, rows_per)):
        g = torch.Generator().manual_seed(seed_for(wkey, layer, mat, f"weights{b}", fmt.tag, 0))
        r1 = min(N, r0 + rows_per)
        W = torch.randn((r1 - r0, K), generator=g)
        W *= torch.exp(0.5 * torch.randn((r1 - r0, 1), generator=g))
        blocks.append((r0, r1, W))
        mags.append(W.abs().max())
    scale = (torch.stack(mags).max() / 448.0).reshape(1).to(torch.float32)
    for r0, r1, W in blocks:
        codes[r0:r1] = (W / scale).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    del blocks
    p = Packed(codes.to(dev), scale.to(dev), None, N, K, fmt)
    return (p, codes) if keep_codes else p


def massive_channels(cfg: Config, layer: int, mat: int, K: int) -> Tuple[List[int], float]:
    """(channel indices, multiplier) of the massive channels of one matrix input."""
    xs = cfg.x
    if xs.kind == "plain":
        return [], 1.0
    # the recipe's fixed channels must exist in a K-channel input (checked on
    # the host: an index past K would reach the device unchecked)
    fixed = [xs.channel] if xs.kind == "fixed" else list(xs.forced)
    if any(not 0 <= c < K for c in fixed):
        raise ValueError(f"{cfg.key}: massive channel {fixed} outside a {K}-wide input")
    if xs.kind == "fixed":
        return [xs.channel], xs.factor
    g = generator(seed_for(cfg.key, layer, mat, "channels", "x", 0), "cpu")
    chosen = [c for c in xs.forced]
    for c in torch.randperm(K, generator=g).tolist():
        if len(chosen) == xs.count:
            break
        if c not in chosen:
            chosen.append(c)
    # expected share f of the energy on `count` channels of a K-channel N(0,1)
    # vector: count*a^2 / (count*a^2 + K - count) = f
    alpha = math.sqrt(xs.share * (K - xs.count) / (xs.count * (1.0 - xs.share)))
    return chosen, alpha


def gen_x(cfg: Config, layer: int, mat: int, M: int, K: int, device="cpu",
          fmt_tag: str = "x") -> torch.Tensor:
    """fp16 activations [M][K]: N(0,1) in fp32, massive channels multiplied in
    fp32, then one rounding to binary16.  All M rows share the channel set."""
    dev = torch.device(device)
    g = generator(seed_for(cfg.key, layer, mat, "x", fmt_tag, M), dev)
    x = torch.randn((M, K), generator=g, device=dev, dtype=torch.float32)
    chans, mult = massive_channels(cfg, layer, mat, K)
    if chans:
        idx = torch.tensor(chans, dtype=torch.long, device=dev)
        x[:, idx] *= mult
    return x.half().contiguous()


def rows_of(p: Packed, rows) -> Packed:
    """A Packed holding only the listed rows (used to hand row samples to a
    checker); rows are independent, so the sub-matrix is a valid problem."""
    idx = torch.as_tensor(rows, dtype=torch.long, device=p.qweight.device)
    scales = p.scales if p.fmt.layout == LAYOUT_FP8_TENSOR else \
        p.scales.index_select(0, idx).contiguous()  # FP8: one scale for the matrix
    if p.fmt.bits in (5, 6):  # two planes: nibbles [N][K/2], high bits [N][K*(bits-4)/8]
        half = p.N * p.K // 2
        nib = p.qweight[:half].reshape(p.N, p.K // 2).index_select(0, idx)
        hi = p.qweight[half:].reshape(p.N, -1).index_select(0, idx)
        qw = torch.cat([nib.reshape(-1), hi.reshape(-1)]).contiguous()
    else:
        qw = p.qweight.index_select(0, idx).contiguous()
    return Packed(qw,
                  scales,
                  None if p.zeros is None else p.zeros.index_select(0, idx).contiguous(),
                  len(rows), p.K, p.fmt)
