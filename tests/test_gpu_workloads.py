"""Full-size parity of every synthetic workload against the oracle.

Each case builds one decode step of a workload (all layers, every quantized
matrix, at its real shape and format) on the GPU from its seeds and runs it in
the launch sequence the benchmark times (gemm_rwkv_decode_amd.step, kind
"layer": grouped receptance/key/value launches, then rq_gemv below M = 5 and
rq_gemm_smallm from M = 5 on).  The oracle then recomputes the outputs from the
very bytes the GPU consumed:

* every output of every matrix for the 768-, 2048- and 2560-wide workloads;
* for the 13.3B-shaped workload (1.4 T multiply-adds in full at its four M),
  every output of layers 0, 30 and 60 and of the 65536x4096 head, and a
  seeded 1/16 of the rows (plus the first and last row) of every other
  matrix.

Layer 0 is also run through the other product entry point (rq_gemm_smallm
below M = 5, rq_gemv from M = 5), so both are checked at full size at every M.
Outputs start as NaN, so an output a kernel never wrote fails.
"""
import pytest
import torch

import oracle as O
from gemm_rwkv_decode_amd import step as ST
from gemm_rwkv_decode_amd import synth as S
from tests.rqtest import THREADS, assert_close, say, to_np

pytestmark = pytest.mark.gpu

CASES = [(cfg.key, f.tag, M) for cfg in S.CONFIGS.values() for f in cfg.formats
         for M in cfg.ms]
SAMPLED = {"rwkv7-13.3b"}
FULL_LAYERS = {0, 30, 60}  # checked in full; the head too
SAMPLE_EVERY = 16          # elsewhere one row in 16

_store = {}


def step_weights(cfg, fmt):
    """The workload's packed matrices on the GPU (one workload held at a time)."""
    key = (cfg.key, fmt.tag)
    if key not in _store:
        _store.clear()
        torch.cuda.empty_cache()
        mats = cfg.matrices()
        W = [S.gen_matrix(cfg.key, l, mi, N, K, fmt, device="cuda")
             for (l, mi, N, K) in mats]
        torch.cuda.synchronize()
        _store[key] = (mats, W)
    return _store[key]


def rows_checked(cfg, fmt, l, mi, N, M):
    if cfg.key not in SAMPLED or l in FULL_LAYERS or mi == ST.HEAD:
        return None  # every row
    g = torch.Generator().manual_seed(S.seed_for(cfg.key, l, mi, "rows", fmt.tag, M))
    pick = set(torch.randperm(N, generator=g)[:N // SAMPLE_EVERY].tolist()) | {0, N - 1}
    return sorted(pick)


def oracle_rows(p, x, rows):
    """Oracle (y, bound) for the listed rows of p (all rows when None)."""
    sub = p if rows is None else S.rows_of(p, rows)
    q, s, z = to_np(sub)
    f = p.fmt
    return O.gemv_ref(q, s, z, x.cpu().numpy(), sub.N, p.K, f.bits, f.group, f.layout,
                      threads=THREADS)


def other_entry(p, x, y):
    import gemm_rwkv_decode_amd as rq
    fn = rq.rq_gemm_smallm if x.shape[0] < ST.MFMA_MIN_M else rq.rq_gemv
    f = p.fmt
    fn(p.qweight, p.scales, p.zeros, x, y, x.shape[0], p.N, p.K, f.bits, f.group, f.layout)


@pytest.mark.parametrize("wkey,ftag,M", CASES, ids=[f"{k}-{t}-M{m}" for k, t, m in CASES])
def test_workload_step(wkey, ftag, M):
    cfg = S.CONFIGS[wkey]
    fmt = S.FORMATS[ftag]
    say(f"[workload] {wkey} {ftag} M={M}: generating")
    mats, W = step_weights(cfg, fmt)
    X = [S.gen_x(cfg, l, mi, M, K, device="cuda") for (l, mi, N, K) in mats]
    Y = [torch.full((M, N), float("nan"), device="cuda") for (_, _, N, _) in mats]
    calls = ST.step_calls(mats, W, X, Y, "layer")
    say(f"[workload] {wkey} {ftag} M={M}: {len(mats)} matrices, {len(calls)} launches")
    for c in calls:
        c()
    layer0 = [i for i, m in enumerate(mats) if m[0] == 0]
    Y2 = {i: torch.full_like(Y[i], float("nan")) for i in layer0}
    for i in layer0:
        other_entry(W[i], X[i], Y2[i])
    torch.cuda.synchronize()
    say(f"[workload] {wkey} {ftag} M={M}: GPU done, checking against the oracle")

    checked = 0
    for i, (l, mi, N, K) in enumerate(mats):
        rows = rows_checked(cfg, fmt, l, mi, N, M)
        y_ref, bound = oracle_rows(W[i], X[i], rows)
        got = Y[i] if rows is None else Y[i][:, rows]
        what = f"{wkey} {ftag} M={M} layer {l} matrix {S.MAT_NAMES[mi]} ({N}x{K})"
        assert_close(got, y_ref, bound, what)
        if i in Y2:
            assert_close(Y2[i], y_ref, bound, what + " via the other entry point")
        checked += got.numel()
    say(f"[workload] {wkey} {ftag} M={M}: {checked} outputs match")
