"""Checks of the seeded input generator (CPU only): reproducibility, distributions, and the
encoders' round-to-nearest-even against torch's own conversions."""
import numpy as np
import torch

from synth import synth as S


def test_streams_are_reproducible_and_independent():
    a = S.normal_f64(1, S.TAG_GATE_UP, 3, 1000)
    b = S.normal_f64(1, S.TAG_GATE_UP, 3, 1000)
    c = S.normal_f64(1, S.TAG_GATE_UP, 4, 1000)
    assert (a == b).all() and not np.allclose(a, c)
    # counter-based: any window equals the same range of the whole stream
    np.testing.assert_array_equal(S.normal_f64(1, S.TAG_GATE_UP, 3, 100, start=450), a[450:550])


def test_normal_moments():
    v = S.normal_f64(2, S.TAG_X, 0, 400_000)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1) < 0.01
    assert abs(((v > 1.96).mean()) - 0.025) < 0.002


def test_bf16_tokens_are_rne_of_normals():
    x = S.tokens(3, 8, 64)
    ref = torch.from_numpy(S.normal_f64(3, S.TAG_X, 0, 8 * 64)).float().to(torch.bfloat16)
    assert (torch.from_numpy(x.reshape(-1)).view(torch.bfloat16) == ref).all()


def test_nvfp4_scales_are_rne_e4m3_of_group_amax():
    H, I = 256, 32
    b = S.routed_bank(4, "nvfp4", 1, H, I)
    w = S.normal_f64(4, S.TAG_GATE_UP, 0, 2 * I * H, S.WEIGHT_SIGMA).reshape(2 * I, H)
    G = (np.abs(w).max(1) / (6 * 448)).astype(np.float32)
    np.testing.assert_array_equal(b.gate_up_global[0], G)
    want = torch.from_numpy(np.abs(w).reshape(2 * I, -1, 16).max(2) / 6 / G[:, None].astype(np.float64))
    want = want.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(b.gate_up_scale[0], want)


def test_fp8blk_codes_are_rne_e4m3():
    H, I = 256, 128
    b = S.routed_bank(5, "fp8blk", 1, H, I)
    w = S.normal_f64(5, S.TAG_DOWN, 0, H * I, S.WEIGHT_SIGMA).reshape(H, I)
    si = np.repeat(np.repeat(b.down_scale[0], 128, 0), 128, 1).astype(np.float64)
    want = torch.from_numpy(w / si).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(b.down[0], want)


def test_mxfp4_scale_exponents():
    H, I = 128, 64
    b = S.routed_bank(6, "mxfp4", 1, H, I)
    w = S.normal_f64(6, S.TAG_GATE_UP, 0, 2 * I * H, S.WEIGHT_SIGMA).reshape(2 * I, H)
    amax = np.abs(w).reshape(2 * I, -1, 32).max(2)
    np.testing.assert_array_equal(b.gate_up_scale[0].astype(int), np.floor(np.log2(amax)).astype(int) - 2 + 127)


def test_zipf_bias_is_a_permuted_zipf_law():
    bias = S.zipf_bias(7, 256, 1.1)
    p = np.sort(np.exp(bias.astype(np.float64)))[::-1]
    r = np.arange(1, 257)
    ref = r ** -1.1 / (r ** -1.1).sum()
    np.testing.assert_allclose(p, ref, rtol=1e-6)
    assert not (np.argsort(-bias) == np.arange(256)).all()


def test_configs_are_the_stated_workloads():
    c = S.CONFIGS
    assert (c[1].H, c[1].E, c[1].k, c[1].I, c[1].Ts) == (256, 8, 2, 128, (16,))
    assert (c[2].H, c[2].E, c[2].k, c[2].I, c[2].shared, c[2].Ts) == (2048, 256, 8, 512, True, (1, 8, 32, 64))
    assert c[3].Ts == (8192,) and c[3].zipf_s == 1.1
    assert c[4].fmt == "fp8blk" and c[4].Ts == (1, 64, 4096) and c[4].slices[0] == (0, 256)
    assert (c[5].H, c[5].I, c[5].slices[0], c[5].fmt) == (4096, 2048, (0, 1024), "mxfp4")
