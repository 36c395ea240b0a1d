"""Seeded input generators: shapes, dtypes, determinism and distribution sanity."""
import numpy as np
import torch

from fp4_quantization_precision_amd import inputs


def test_zipf_counts_sum_and_order():
    c = inputs.zipf_counts(32, 16384, 1.1)
    assert sum(c) == 16384 and len(c) == 32
    assert all(c[i] >= c[i + 1] for i in range(31))
    # largest-remainder rounding of 16384 * e^-1.1 / H, e = 1..32
    assert c[:4] == [4649, 2169, 1388, 1012] and c[-2:] == [106, 103]
    c64 = inputs.zipf_counts(64, 16384, 1.1)
    assert sum(c64) == 16384 and min(c64) > 0


def test_group_offsets():
    off = inputs.group_offsets([3, 0, 5])
    assert off.tolist() == [0, 3, 3, 8] and off.dtype == torch.int32


def test_tiny_roundtrip_deterministic():
    a1, b1 = inputs.tiny_roundtrip()
    a2, b2 = inputs.tiny_roundtrip()
    assert a1.shape == (64, 256) and a1.dtype == torch.float32
    assert torch.equal(a1, a2) and torch.equal(b1, b2)
    rel = ((b1 - a1) / a1).abs()
    assert 5e-4 < rel.median().item() < 2e-3


def test_moe_layer_small():
    xr, xt = inputs.moe_expert_weights_layer(5, experts=2, rows=256, cols=768)
    assert xr.shape == (2, 256, 768) and xr.dtype == torch.bfloat16
    frac = (xr != xt).float().mean().item()
    assert 0.003 < frac < 0.05          # noise mostly below half a bf16 ulp
    big = (xr.float().abs() > 0.2).float().mean().item()
    assert 2e-4 < big < 3e-3             # the x20 entries
    xr2, _ = inputs.moe_expert_weights_layer(5, experts=2, rows=256, cols=768)
    assert torch.equal(xr, xr2)
    xr3, _ = inputs.moe_expert_weights_layer(6, experts=2, rows=256, cols=768)
    assert not torch.equal(xr, xr3)


def test_activations_small():
    xr, xt, ch = inputs.activations(tokens=256, hidden=512)
    assert xr.shape == (256, 512) and ch.numel() == 8
    col_max = xr.float().abs().amax(dim=0)
    assert col_max[ch].min() > col_max[[i for i in range(512) if i not in set(ch.tolist())]].max()
    rel = ((xt.float() - xr.float()) / xr.float()).abs()
    assert rel.max().item() <= 2.0 ** -8 + 2.0 ** -8


def test_random_nvfp4():
    c, s, t = inputs.random_nvfp4(2, 32, 64, zero_block_frac=0.2)
    assert c.shape == (2, 32, 32) and s.shape == (2, 32, 4) and t.shape == (2,)
    assert s.max().item() <= 0x7E and (s == 0).any()


def test_kv_cache_small():
    kr, kt, vr, vt, ch = inputs.kv_cache(64, 2, 32, outlier_channels=2)
    assert kr.shape == (64, 2, 32) and kr.dtype == torch.bfloat16
    assert ch.shape == (2, 2)
    for h in range(2):
        big = kr[:, h, ch[h]].float().abs().mean()
        rest = kr[:, h].float().abs().mean()
        assert big > 5 * rest
    rel = ((kt.float() - kr.float()).abs() / kr.float().abs().clamp_min(1e-30)).max()
    assert rel <= 2.0 ** -8 + 2.0 ** -8  # noise bound plus one bf16 rounding
    kr2, _, vr2, _, _ = inputs.kv_cache(64, 2, 32, outlier_channels=2)
    assert torch.equal(kr, kr2) and torch.equal(vr, vr2)
