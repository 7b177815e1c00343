"""The decode step's launch sequence (host logic only; the C calls are
replaced by a recorder, so nothing here touches a GPU)."""
from types import SimpleNamespace

import pytest
import torch

import gemm_rwkv_decode_amd as rq
from gemm_rwkv_decode_amd import step as ST
from gemm_rwkv_decode_amd import synth as S


@pytest.fixture
def recorded(monkeypatch):
    log = []

    def fake_prepare(name, *args, stream=None):
        log.append((name, args))
        return lambda: None
    monkeypatch.setattr(rq, "prepare", fake_prepare)
    return log


def fake_step(cfg, M):
    mats = cfg.matrices()
    W = [SimpleNamespace(qweight=("q", i), scales=("s", i), zeros=None, N=N, K=K,
                         fmt=cfg.formats[0]) for i, (_, _, N, K) in enumerate(mats)]
    X = [torch.empty((M, 1)) for _ in mats]  # only the shape is read
    Y = [("y", i) for i in range(len(mats))]
    return mats, W, X, Y


def test_layer_schedule_at_m1(recorded):
    cfg = S.CONFIGS["rwkv7-13.3b"]
    mats, W, X, Y = fake_step(cfg, 1)
    calls = ST.step_calls(mats, W, X, Y, "layer")
    assert len(calls) == 61 * 4 + 1 == len(recorded)
    # every matrix exactly once, layers in order, dependencies respected
    seen = []
    for name, args in recorded:
        if name == "rq_gemv_batched":
            idx = [p[0][1] for p in args[0]]  # receptance, key, value of one layer
            assert idx == [len(seen), len(seen) + 1, len(seen) + 2]
            seen.extend(idx)
        else:
            assert name == "rq_gemv"
            seen.append(args[0][1])
    assert seen == list(range(len(mats)))
    assert recorded[-1][1][6] == 65536  # the head is the last launch


def test_smallm_entry_from_m5(recorded):
    cfg = S.CONFIGS["rwkv7-2.9b"]
    mats, W, X, Y = fake_step(cfg, 16)
    ST.step_calls(mats, W, X, Y, "layer")
    # per layer: grouped receptance/key/value, then three matrix-core launches
    assert [n for n, _ in recorded] == (["rq_gemv_batched"] + ["rq_gemm_smallm"] * 3) * 32
    assert all(a[1] == 16 for n, a in recorded if n == "rq_gemv_batched")
    assert all(a[5] == 16 for n, a in recorded if n == "rq_gemm_smallm")
    assert recorded[1][1][10] == S.LAYOUT_ASYM_SB and recorded[1][1][9] == 32
    del recorded[:]
    ST.step_calls(mats, W, X, Y, "matrix")
    assert [n for n, _ in recorded] == ["rq_gemm_smallm"] * len(mats)


def test_matrix_and_batched_kinds(recorded):
    cfg = S.CONFIGS["rwkv7-0.1b"]
    mats, W, X, Y = fake_step(cfg, 4)
    assert len(ST.step_calls(mats, W, X, Y, "matrix")) == 72
    del recorded[:]
    calls = ST.step_calls(mats, W, X, Y, "batched")
    assert len(calls) == 2 and [len(a[0]) for _, a in recorded] == [64, 8]
    del recorded[:]
    ST.step_calls(mats, W, [torch.empty((16, 1))] * 72, Y, "batched")
    assert [(n, a[1]) for n, a in recorded] == [("rq_gemv_batched", 16)] * 2
    del recorded[:]
    ST.step_calls(mats, W, [torch.empty((5, 1))] * 72, Y, "layer")
    assert [n for n, _ in recorded] == (["rq_gemv_batched"] + ["rq_gemm_smallm"] * 3) * 12
    del recorded[:]
    ST.step_calls(mats, W, X, Y, "layer")
    assert [n for n, _ in recorded] == (["rq_gemv_batched"] + ["rq_gemv"] * 3) * 12
    with pytest.raises(ValueError):
        ST.step_calls(mats, W, X, Y, "fused")
    assert ST.step_calls([], [], [], [], "layer") == []
