"""The launch sequence of one decode step over a model's quantized matrices.

A step multiplies every quantized matrix of every layer by its activation rows,
in dependency order.  Within an RWKV-7 layer the receptance, key and value
projections read three independent (token-shift mixed) inputs and can run
together; the output projection needs the time-mix result, the FFN key needs
the output projection and the FFN value needs the FFN key (package page "RWKV-7
FP8 Quantized Inference", sections "Core Approach: Full FP8, No Residuals" and
"Operator Optimization Details", where receptance/key/value are fused into one
kernel).  The vocabulary head, when present, comes last.

This module only orders calls of the C interface; each call is a prepared
``rq.prepare`` callable, so a step loop (or a graph capture) pays no per-call
argument conversion.
"""
from typing import Callable, Dict, List, Sequence, Tuple

import gemm_rwkv_decode_amd as rq

# matrix indices within a layer (the head is 6)
RECEPTANCE, KEY, VALUE, OUTPUT, FFN_KEY, FFN_VALUE, HEAD = range(7)

# Smallest M a step sends to rq_gemm_smallm, which may split K over
# workgroups (through its workspace).  Below it the step calls rq_gemv and
# rq_gemv_batched, which pick the kernel for M (vector units at M <= 2, the
# same matrix-core kernel from M = 3 on, with K kept whole).
MFMA_MIN_M = 5

KINDS = ("layer", "matrix", "batched")


def product_entry(M: int) -> str:
    """The entry point a step uses for M activation rows."""
    return "rq_gemv" if M < MFMA_MIN_M else "rq_gemm_smallm"


def _args(p, x, y) -> Tuple:
    f = p.fmt
    return (p.qweight, p.scales, p.zeros, x, y, x.shape[0], p.N, p.K, f.bits, f.group,
            f.layout)


def step_calls(mats: Sequence[Tuple[int, int, int, int]], W: Sequence, X: Sequence,
               Y: Sequence, kind: str = "layer", stream=None) -> List[Callable[[], None]]:
    """Prepared calls of one step, in execution order.

    ``mats[i]`` is (layer, matrix, N, K); ``W[i]`` its packed weights
    (``synth.Packed``-like: qweight, scales, zeros, N, K, fmt); ``X[i]`` its
    float16 [M][K] input and ``Y[i]`` its float32 [M][N] output.  All share M
    and the format.

    kinds:
      "layer"   -- per layer: receptance, key and value in one grouped launch
                   (rq_gemv_batched), then output, FFN key, FFN value; the
                   head last.
      "matrix"  -- one launch per matrix, in order (rq_gemv below M = 5,
                   rq_gemm_smallm from M = 5 on).
      "batched" -- every product through rq_gemv_batched, up to RQ_MAX_BATCH
                   per call, ignoring the order between layers (a bound on
                   what grouping could reach, not a valid decode order).
    """
    if kind not in KINDS:
        raise ValueError(f"unknown step kind {kind!r}")
    if not mats:
        return []
    M = X[0].shape[0]
    f = W[0].fmt
    entry = product_entry(M)
    prep = lambda *a: rq.prepare(*a, stream=stream)  # noqa: E731
    single = lambda i: prep(entry, *_args(W[i], X[i], Y[i]))  # noqa: E731

    def grouped(ix: List[int]):
        probs = [(W[i].qweight, W[i].scales, W[i].zeros, X[i], Y[i], W[i].N, W[i].K)
                 for i in ix]
        return prep("rq_gemv_batched", probs, M, f.bits, f.group, f.layout)

    calls = []
    if kind == "batched":
        ix = list(range(len(mats)))
        for k in range(0, len(ix), rq.RQ_MAX_BATCH):
            calls.append(grouped(ix[k:k + rq.RQ_MAX_BATCH]))
        return calls
    if kind == "matrix":
        return [single(i) for i in range(len(mats))]
    by_layer: Dict[int, Dict[int, int]] = {}
    for i, (l, mi, _, _) in enumerate(mats):
        by_layer.setdefault(l, {})[mi] = i
    for l in sorted(by_layer):
        ix = by_layer[l]
        rkv = [ix[m] for m in (RECEPTANCE, KEY, VALUE) if m in ix]
        if len(rkv) > 1:
            calls.append(grouped(rkv))
        else:
            calls.extend(single(i) for i in rkv)
        for m in (OUTPUT, FFN_KEY, FFN_VALUE, HEAD):
            if m in ix:
                calls.append(single(ix[m]))
    return calls
