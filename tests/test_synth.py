"""The seeded input generators: encodings agree with the oracle's (pinned)
packers, values follow the stated distributions, seeds are reproducible."""
import numpy as np
import pytest
import torch

import oracle as O
from gemm_rwkv_decode_amd import synth as S


def test_pack_nibbles_matches_oracle_packer():
    g = torch.Generator().manual_seed(0)
    for layout, lo, hi in [(S.LAYOUT_SYM, -8, 7), (S.LAYOUT_ASYM_SB, 0, 15)]:
        codes = torch.randint(lo, hi + 1, (13, 96), generator=g, dtype=torch.int16)
        codes = codes.to(torch.int8)
        mine = S.pack_nibbles(codes).numpy()
        ref = O.pack_codes(codes.numpy(), 4, layout)
        assert np.array_equal(mine, ref)


def test_pack_records_matches_oracle_packer():
    g = torch.Generator().manual_seed(1)
    base = (torch.rand((5, 3), generator=g) * 10).half()
    base[0, 0] = float.fromhex("0x1p-24")  # subnormal
    base[1, 1] = -2.5
    sub = torch.randint(0, 64, (5, 3, 8), generator=g, dtype=torch.int16).to(torch.uint8)
    rec = S.pack_records(base, sub).numpy()
    bb = base.view(torch.int16).numpy().view(np.uint16)
    for n in range(5):
        for b in range(3):
            assert np.array_equal(rec[n, b], O.pack_record(int(bb[n, b]), sub[n, b].numpy()))


@pytest.mark.parametrize("fmt", [S.INT4_G64, S.INT8_G16, S.ASYM4_G32])
def test_gen_matrix_decodes_to_its_codes(fmt):
    N, K = 24, 512
    p, codes = S.gen_matrix("t9", 0, 0, N, K, fmt, keep_codes=True)
    got = O.unpack_codes(p.qweight.numpy(), N, K, fmt.bits, fmt.layout)
    assert np.array_equal(got, codes.numpy())
    lo, hi = fmt.code_range()
    assert codes.min().item() >= lo and codes.max().item() <= hi
    # every value of the range occurs
    assert len(torch.unique(codes)) == hi - lo + 1
    if fmt.layout == S.LAYOUT_SYM:
        s = p.scales.float()
        assert p.scales.dtype == torch.float16 and p.scales.shape == (N, K // fmt.group)
        assert s.min().item() >= 1e-3 * (1 - 2 ** -10) and s.max().item() <= 1e-1 * (1 + 2 ** -10)
        assert p.zeros is None
    else:
        assert p.scales.shape == (N, K // 256, 8) and p.zeros.shape == (N, K // 256, 8)
        for rec in (p.scales, p.zeros):
            base, sub = O.unpack_record(rec[0, 0].numpy())
            v = O.half_to_double(base)
            assert 1e-4 * (1 - 2 ** -10) <= v <= 2e-3 * (1 + 2 ** -10)
            assert sub.max() <= 63


def test_seeds_are_reproducible_and_distinct():
    a = S.gen_matrix("rwkv7-13.3b", 3, 1, 8, 256, S.INT4_G64)
    b = S.gen_matrix("rwkv7-13.3b", 3, 1, 8, 256, S.INT4_G64)
    c = S.gen_matrix("rwkv7-13.3b", 3, 2, 8, 256, S.INT4_G64)
    assert torch.equal(a.qweight, b.qweight) and torch.equal(a.scales, b.scales)
    assert not torch.equal(a.qweight, c.qweight)
    s = {S.seed_for("rwkv7-13.3b", l, m, r, "int4g64", 1) for l in range(3) for m in range(7)
         for r in ("codes", "scales", "x")}
    assert len(s) == 3 * 7 * 3


def test_massive_channels_fixed():
    cfg = S.CONFIGS["rwkv7-1.5b"]
    x = S.gen_x(cfg, 0, 0, 4, 2048)
    plain = S.gen_x(S.CONFIGS["rwkv7-1.5b"], 0, 0, 4, 2048).float()
    chans, mult = S.massive_channels(cfg, 0, 0, 2048)
    assert chans == [1202] and mult == 50.0
    assert torch.equal(x.float(), plain)
    # channel 1202 is ~50x larger than the rest on average
    big = x[:, 1202].float().abs().mean().item()
    rest = x.float().abs().mean().item()
    assert big > 10 * rest


def test_massive_channel_outside_the_input_is_refused():
    """A recipe's fixed channel past K raises on the host, before any tensor
    is indexed (on the GPU an index past the end would not be checked)."""
    with pytest.raises(ValueError):
        S.massive_channels(S.CONFIGS["rwkv7-1.5b"], 0, 0, 768)   # channel 1202
    with pytest.raises(ValueError):
        S.gen_x(S.CONFIGS["rwkv7-1.5b"], 0, 0, 1, 768)
    with pytest.raises(ValueError):
        S.massive_channels(S.CONFIGS["rwkv7-2.9b"], 0, 0, 512)   # forced channel 517
    assert S.massive_channels(S.CONFIGS["rwkv7-2.9b"], 0, 0, 2560)[0][0] == 517


@pytest.mark.parametrize("wkey,K,share", [("rwkv7-2.9b", 2560, 0.98),
                                          ("rwkv7-2.9b", 10240, 0.98),
                                          ("rwkv7-13.3b", 4096, 0.99),
                                          ("rwkv7-13.3b", 16384, 0.99)])
def test_massive_channels_energy_share(wkey, K, share):
    cfg = S.CONFIGS[wkey]
    chans, alpha = S.massive_channels(cfg, 5, 3, K)
    assert len(chans) == 8 and len(set(chans)) == 8 and max(chans) < K
    if wkey == "rwkv7-2.9b":
        assert 517 in chans
    x = S.gen_x(cfg, 5, 3, 64, K).double()
    e = (x ** 2).sum(dim=1)
    em = (x[:, chans] ** 2).sum(dim=1)
    # expected share over 64 rows: within a few percent of f
    assert abs((em.sum() / e.sum()).item() - share) < 0.01


def test_step_sizes_match_the_configs():
    # 13.3B shape: 61 layers x (4 x 4096^2 + 2 x 16384x4096) int4 g64
    c = S.CONFIGS["rwkv7-13.3b"]
    assert c.step_weight_bytes(S.INT4_G64, with_head=False) == \
        61 * (4 * 4096 * 4096 + 2 * 16384 * 4096) * 17 // 32
    assert len(c.matrices(with_head=False)) == 366
    # with the 65536 x 4096 head: about 6.7 GB per step
    assert len(c.matrices()) == 367 and c.matrices()[-1] == (61, 6, 65536, 4096)
    assert c.step_weight_bytes(S.INT4_G64) == \
        (61 * (4 * 4096 * 4096 + 2 * 16384 * 4096) + 65536 * 4096) * 17 // 32
    assert 6.6e9 < c.step_weight_bytes(S.INT4_G64) < 6.7e9
    assert len(S.CONFIGS["rwkv7-0.1b"].matrices()) == 72
    assert S.CONFIGS["gemv768"].matrices() == [(0, 0, 768, 768)]
    # int8 g16 carries 9 bits per weight, asym 4.5
    assert S.INT8_G16.weight_bytes(2048, 2048) * 8 == 2048 * 2048 * 9
    assert S.ASYM4_G32.weight_bytes(2560, 2560) * 8 == 2560 * 2560 * 9 // 2
