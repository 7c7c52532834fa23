"""The seeded synthetic input recipe (CPU only)."""
import torch

from exact_io_aware_45_amd import inputs


def test_blocksparse_mask_matches_recipe():
    """Band |qb - kb| <= 1 plus seeded off-band tiles, 12.5 % of 128 x 128 tiles."""
    m = inputs.block_mask(16384, 128, band=1, density=0.125, seed=0)
    assert m.shape == (128, 128) and m.dtype == torch.uint8 and int(m.sum()) == 2048
    idx = torch.arange(128)
    band = (idx[:, None] - idx[None, :]).abs() <= 1
    assert bool(m[band].all()) and int(band.sum()) == 382
    assert torch.equal(m, inputs.block_mask(16384, 128, band=1, density=0.125, seed=0))
    assert not torch.equal(m, inputs.block_mask(16384, 128, band=1, density=0.125, seed=1))


def test_qkv_is_seeded_and_standard_normal():
    a = inputs.qkv(2, 3, 100, 64, torch.float32, seed=4, with_dout=True)
    b = inputs.qkv(2, 3, 100, 64, torch.float32, seed=4, with_dout=True)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    assert all(x.shape == (2, 3, 100, 64) for x in a)
    x = torch.cat([t.flatten() for t in a])
    assert abs(float(x.mean())) < 0.02 and abs(float(x.std()) - 1.0) < 0.02
    h = inputs.qkv(2, 3, 100, 64, torch.bfloat16, seed=4)
    assert h[0].dtype == torch.bfloat16 and torch.equal(h[0], a[0].to(torch.bfloat16))


def test_workload_shapes():
    w = inputs.WORKLOADS
    assert (w["long_d128_causal"].B, w["long_d128_causal"].H, w["long_d128_causal"].N,
            w["long_d128_causal"].d) == (1, 32, 8192, 128)
    assert (w["bwd_d128_causal"].B, w["bwd_d128_causal"].H, w["bwd_d128_causal"].N) == (4, 16, 4096)
    assert w["bwd_d128_causal"].backward and w["long_d128_causal"].causal
    assert w["blocksparse_d64"].sparse and w["blocksparse_d64"].N == 16384
    assert w["single_head_f32"].dtype == "f32"


def test_fp8_inputs_quantize_the_same_draws():
    ref = inputs.qkv(1, 2, 100, 64, torch.float32, seed=3)
    for (codes, descale), x in zip(inputs.qkv_fp8(1, 2, 100, 64, seed=3), ref):
        assert codes.dtype == torch.float8_e4m3fn and codes.shape == x.shape
        real = codes.to(torch.float64) * descale
        assert float(codes.to(torch.float32).abs().max()) <= inputs.FP8_MAX
        # e4m3 rounding: relative error <= 2^-4 in the normal range, absolute
        # <= 2^-10 * descale below it
        err = (real - x.to(torch.float64)).abs()
        bound = 2.0 ** -4 * x.to(torch.float64).abs() + 2.0 ** -10 * descale + 1e-12
        assert bool((err <= bound).all())
        assert abs(float(x.abs().max()) / inputs.FP8_MAX - descale) <= 1e-6 * descale
