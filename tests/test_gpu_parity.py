"""GPU parity of the HIP path (through the C ABI) against the fp64 CPU oracle.

Routing selection and alignment are compared bit for bit; expert outputs must meet
max|delta| <= 1e-2 * max|ref| + 1e-3.  Inputs come from the seeded generator or from the
oracle, never from the GPU path.
"""
import dataclasses

import numpy as np
import pytest
import torch

import quantized_moe_expert_topk_amd as qm
from oracle import oracle as O
from synth import synth as S
from tests.gpu_util import align_np, bf16_dev, check_close, device_bank, tile16_np, to_dev

pytestmark = pytest.mark.gpu

NEAR_TIE = 1e-5  # fp32 logit gap below which the k-th/(k+1)-th choice is not pinned


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    qm.lib()
    yield


_cache = {}


def inputs_for(cid, T, batch=0, experts="routed"):
    """Layer inputs of config `cid` for T tokens with only the experts the oracle routes to
    materialised (plus the oracle routing).  Cached per (cid, T, batch)."""
    key = (cid, T, batch)
    if key not in _cache:
        cfg = S.CONFIGS[cid]
        base = S.layer_inputs(cfg, T, batch=batch, experts=[])
        lg, ids, w, gap = O.route(base.x, base.router, base.bias, cfg.k, cfg.renormalize)
        inp = S.layer_inputs(cfg, T, batch=batch, experts=np.unique(ids))
        _cache[key] = (inp, dict(logits=lg, ids=ids, w=w, gap=gap))
    return _cache[key]


def dev_banks(inp):
    key = ("dev", id(inp))
    if key not in _cache:
        _cache[key] = (device_bank(inp.routed), device_bank(inp.shared) if inp.shared is not None else None)
    return _cache[key]


# ----------------------------------------------------------------------------- routing

@pytest.mark.parametrize("T,E,k,renorm,with_bias", [
    (1, 256, 8, True, False), (16, 8, 2, True, False), (300, 256, 8, True, True), (77, 1000, 64, True, False),
    (33, 64, 6, False, False), (5, 3, 3, True, False),
])
def test_route_from_logits_selection_is_bit_exact(T, E, k, renorm, with_bias):
    lg = S.logits_f32(7, E + k, T, E)
    lg[:, E // 2] = lg[:, 1]                      # exact ties: index 1 must rank first
    if T > 3:
        lg[3, :] = np.float32(0.25)               # a row of all-equal logits
    bias = S.zipf_bias(8, E, 1.1) if with_bias else None
    eff = lg + bias if with_bias else lg          # the fp32 add the kernel does
    ids_ref, w_ref, _ = O.topk(eff.astype(np.float64), k, renorm)
    ids, w = qm.moe_route_from_logits(to_dev(lg), k, to_dev(bias), renorm)
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    assert np.abs(w.cpu().numpy() - w_ref).max() <= 2e-6


@pytest.mark.parametrize("k", [1, 2, 3])
def test_route_from_logits_signed_zeros_are_one_score(k):
    """-0.0 and +0.0 are the same logit: the lower index ranks first whichever of the two
    carries the sign bit (the stated tie rule), with and without a bias that is zero."""
    T, E = 6, 40
    lg = -1.0 - S.logits_f32(21, 3, T, E) ** 2     # every other logit is below -1
    lg = lg.astype(np.float32)
    lg[0, 5], lg[0, 9] = np.float32(-0.0), np.float32(0.0)    # lower index negative zero
    lg[1, 5], lg[1, 9] = np.float32(0.0), np.float32(-0.0)    # lower index positive zero
    lg[2, [3, 7, 30]] = np.float32(-0.0)                     # three negative zeros
    lg[3, [3, 7, 30]] = [np.float32(0.0), np.float32(-0.0), np.float32(0.0)]
    lg[4, 0], lg[4, E - 1] = np.float32(-0.0), np.float32(0.0)
    lg[5, :] = np.float32(-0.0)
    lg[5, ::2] = np.float32(0.0)
    assert np.signbit(lg[0, 5]) and not np.signbit(lg[0, 9])
    ids_ref, w_ref, _ = O.topk(lg.astype(np.float64), k, True)
    for bias in (None, np.zeros(E, np.float32)):
        ids, w = qm.moe_route_from_logits(to_dev(lg), k, to_dev(bias), True)
        np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
        assert np.abs(w.cpu().numpy() - w_ref).max() <= 2e-6
    assert (ids_ref[0, 0], ids_ref[1, 0], ids_ref[4, 0], ids_ref[5, 0]) == (5, 5, 0, 0)


@pytest.mark.parametrize("cid,T", [(1, 16), (2, 1), (2, 64), (4, 64), (5, 16), (3, 8192)])
def test_route_matches_oracle(cid, T):
    cfg = S.CONFIGS[cid]
    x = S.tokens(cfg.seed, T, cfg.H)
    wr = S.router_weight(cfg.seed, cfg.E, cfg.H)
    bias = S.zipf_bias(cfg.seed, cfg.E, cfg.zipf_s) if cfg.zipf_s else None
    lg_ref, ids_ref, w_ref, gap = O.route(x, wr, bias, cfg.k, cfg.renormalize)
    lg, ids, w = qm.moe_route(bf16_dev(x), bf16_dev(wr), to_dev(bias), cfg.k, cfg.renormalize)
    lerr = np.abs(lg.cpu().numpy() - lg_ref).max()
    assert lerr <= 5e-6, lerr
    sure = gap > NEAR_TIE
    print(f"[route] cfg{cid} T={T}: max logit err {lerr:.2e}, near-tie tokens {int((~sure).sum())}", flush=True)
    ids_g = ids.cpu().numpy()
    np.testing.assert_array_equal(ids_g[sure], ids_ref[sure])
    assert np.abs(w.cpu().numpy()[sure] - w_ref[sure]).max() <= 1e-5
    # near-tie tokens: the picks must still be a valid top-k within the tie window
    for t in np.nonzero(~sure)[0]:
        kth = np.sort(lg_ref[t])[::-1][cfg.k - 1]
        assert (lg_ref[t][ids_g[t]] >= kth - 2 * NEAR_TIE).all()


@pytest.mark.parametrize("T,E,H,k,with_bias", [(1500, 200, 1024, 6, True), (1024, 256, 4096, 8, False),
                                               (2077, 64, 384, 4, False), (1031, 100, 256, 64, True),
                                               (1100, 300, 512, 8, True),
                                               # E % 4 != 0: the output tile's direct stores instead of
                                               # the LDS-staged 16-byte ones
                                               (1030, 61, 256, 3, True), (1040, 130, 512, 8, False)])
def test_tiled_router_shapes_match_oracle(T, E, H, k, with_bias):
    """Batches of 1024 tokens and more run the router on the LDS-tiled GEMM (split over
    K): ragged token and expert tiles, k up to 64, more than 256 experts, with and without a
    bias."""
    x = S.tokens(3, T, H)
    wr = S.router_weight(3, E, H)
    bias = S.zipf_bias(3, E, 1.1) if with_bias else None
    lg_ref, ids_ref, w_ref, gap = O.route(x, wr, bias, k, True)
    lg, ids, w = qm.moe_route(bf16_dev(x), bf16_dev(wr), to_dev(bias), k, True)
    lerr = np.abs(lg.cpu().numpy() - lg_ref).max()
    assert lerr <= 5e-6, lerr
    sure = gap > NEAR_TIE
    np.testing.assert_array_equal(ids.cpu().numpy()[sure], ids_ref[sure])
    assert np.abs(w.cpu().numpy()[sure] - w_ref[sure]).max() <= 1e-5


def test_route_is_deterministic():
    cfg = S.CONFIGS[3]
    x = bf16_dev(S.tokens(cfg.seed, 4096, cfg.H))
    wr = bf16_dev(S.router_weight(cfg.seed, cfg.E, cfg.H))
    a = qm.moe_route(x, wr, None, 8)
    b = qm.moe_route(x, wr, None, 8)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


# ----------------------------------------------------------------------------- alignment

@pytest.mark.parametrize("T,k,E,bm,kind", [
    (16, 2, 8, 16, "rand"), (1, 8, 256, 16, "rand"), (64, 8, 256, 16, "rand"), (8192, 8, 256, 64, "rand"),
    (4096, 8, 256, 32, "rand"), (130, 8, 1000, 16, "rand"), (3000, 4, 7, 128, "rand"), (1, 1, 1, 16, "rand"),
    (500, 8, 256, 16, "one_expert"), (257, 3, 256, 256, "two_experts"), (8192, 8, 256, 16, "zipf"),
    (8192, 8, 256, 128, "zipf"), (100, 2, 600, 128, "rand"), (4096, 8, 256, 128, "one_expert"),
    # one workgroup with four rows of 64 pairs per wave (1024 < T*k <= 4096, E <= 256), and
    # the sizes just past it
    (256, 8, 256, 16, "rand"), (512, 8, 256, 64, "zipf"), (129, 8, 256, 16, "rand"), (300, 8, 200, 128, "one_expert"),
    (1000, 4, 3, 32, "two_experts"), (513, 8, 256, 16, "rand"), (250, 8, 257, 16, "rand"),
    # block sizes that are not powers of two (divisions instead of shifts)
    (16, 2, 8, 48, "rand"), (300, 8, 200, 80, "rand"), (1, 8, 256, 208, "rand"), (5000, 2, 64, 112, "rand"),
])
def test_align_is_bit_exact(T, k, E, bm, kind):
    if kind == "rand":
        ids = S.randint(13, T * 31 + E, T * k, E).reshape(T, k)
    elif kind == "one_expert":
        ids = np.full((T, k), E // 3, np.int32)
    elif kind == "two_experts":
        ids = np.where(np.arange(T * k) % 5 == 0, 0, E - 1).astype(np.int32).reshape(T, k)
    else:
        cfg = S.CONFIGS[3]
        x = S.tokens(cfg.seed, T, cfg.H)
        _, ids, _, _ = O.route(x, S.router_weight(cfg.seed, E, cfg.H), S.zipf_bias(cfg.seed, E, 1.1), k)
    ref = O.align(ids, E, bm)
    out = qm.moe_align(to_dev(ids), E, bm)
    got = align_np(out)
    for key in ref:
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    again = align_np(qm.moe_align(to_dev(ids), E, bm))
    for key in ref:
        np.testing.assert_array_equal(again[key], got[key], err_msg=key)


@pytest.mark.parametrize("T,E,k,H,with_bias,renorm,bm", [
    (1, 256, 8, 2048, False, True, 16), (2, 8, 2, 256, True, True, 16), (5, 3, 3, 128, False, False, 32),
    (16, 512, 16, 384, True, True, 64), (16, 64, 64, 256, False, True, 128), (4, 1, 1, 128, False, True, 16),
    (8, 100, 6, 640, True, False, 256),
    (17, 256, 8, 2048, False, True, 16), (64, 256, 8, 2048, True, True, 16), (1, 513, 4, 256, False, True, 16),
    (16, 128, 64, 128, False, True, 16), (1500, 200, 6, 1024, True, True, 128),
    # larger batches on both sides of 1024 pairs, the tiled router (T = 1024) and E = 512
    (128, 256, 8, 2048, True, True, 16), (129, 256, 8, 2048, False, True, 16), (37, 256, 8, 1024, True, False, 32),
    (1024, 64, 1, 256, False, True, 16), (100, 512, 10, 384, True, True, 64),
    # block sizes that are not powers of two
    (3, 256, 8, 2048, True, True, 48), (40, 256, 8, 1024, False, True, 176)])
def test_route_align_equals_route_then_align(T, E, k, H, with_bias, renorm, bm):
    """moe_route_align (one top-k + align workgroup for T <= 8, E <= 512, T*k <= 1024) gives
    exactly the outputs of moe_route followed by moe_align, on both sides of that boundary."""
    x, wr = bf16_dev(S.tokens(5, T, H)), bf16_dev(S.router_weight(5, E, H))
    bias = to_dev(S.zipf_bias(5, E, 1.1)) if with_bias else None
    lg1, ids1, w1 = qm.moe_route(x, wr, bias, k, renorm)
    al1 = align_np(qm.moe_align(ids1, E, bm))
    lg2, ids2, w2, al2 = qm.moe_route_align(x, wr, bias, k, bm, renorm)
    assert torch.equal(lg1, lg2) and torch.equal(ids1, ids2) and torch.equal(w1, w2)
    al2 = align_np(al2)
    for key in al1:
        np.testing.assert_array_equal(al2[key], al1[key], err_msg=key)
    # and against the oracle's selection and alignment where the picks are pinned
    _, ids_ref, _, gap = O.route(S.tokens(5, T, H), S.router_weight(5, E, H),
                                 S.zipf_bias(5, E, 1.1) if with_bias else None, k, renorm)
    if (gap > NEAR_TIE).all():
        np.testing.assert_array_equal(ids2.cpu().numpy(), ids_ref)
        ref = O.align(ids_ref, E, bm)
        for key in ref:
            np.testing.assert_array_equal(al2[key], ref[key], err_msg=key)


@pytest.mark.parametrize("seed", range(24))
def test_random_route_then_align(seed):
    """Seeded random routing problems (expert counts 1..1000, k up to 64, hidden sizes up to
    2048, small and tiled-router batch sizes, with and without bias and renormalisation): the
    GPU top-k against the oracle's (bit for bit away from near-ties), then the GPU alignment of
    the GPU's picks against the oracle's alignment of the same picks, at a random block size."""
    rng = np.random.default_rng(2000 + seed)
    E = int(rng.choice([1, 2, 3, 7, 8, 64, 100, 256, 513, 1000]))
    k = int(rng.integers(1, min(E, 64) + 1)) if rng.random() < 0.2 else int(rng.integers(1, min(E, 8) + 1))
    H = 128 * int(rng.integers(1, 17))
    T = int(rng.choice([1, 5, 16, 17, 64, 300, 1024, 1500]))
    with_bias, renorm = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    bm = 16 * int(rng.integers(1, 17))
    x, wr = S.tokens(seed, T, H), S.router_weight(seed, E, H)
    bias = S.zipf_bias(seed, E, 1.1) if with_bias else None
    name = f"E={E} k={k} H={H} T={T} bias={with_bias} renorm={renorm} bm={bm}"
    lg_ref, ids_ref, w_ref, gap = O.route(x, wr, bias, k, renorm)
    lg, ids, w = qm.moe_route(bf16_dev(x), bf16_dev(wr), to_dev(bias), k, renorm)
    lerr = np.abs(lg.cpu().numpy() - lg_ref).max()
    assert lerr <= 5e-6, (name, lerr)
    sure = gap > NEAR_TIE
    ids_g = ids.cpu().numpy()
    np.testing.assert_array_equal(ids_g[sure], ids_ref[sure], err_msg=name)
    assert np.abs(w.cpu().numpy()[sure] - w_ref[sure]).max() <= 1e-5, name
    for t in np.nonzero(~sure)[0]:
        kth = np.sort(lg_ref[t])[::-1][k - 1]
        assert (lg_ref[t][ids_g[t]] >= kth - 2 * NEAR_TIE).all(), name
    ref = O.align(ids_g, E, bm)
    got = align_np(qm.moe_align(ids, E, bm))
    for key in ref:
        np.testing.assert_array_equal(got[key], ref[key], err_msg=f"{name} {key}")


# ----------------------------------------------------------------------------- expert layer

# ----------------------------------------------------------------------------- weight layout

@pytest.mark.parametrize("fmt,E,H,I", [("nvfp4", 3, 256, 128), ("fp8blk", 2, 256, 256), ("mxfp4", 3, 512, 192),
                                       ("bf16", 2, 256, 96)])
def test_pack_bank_is_the_tile16_permutation(fmt, E, H, I):
    """moe_pack_bank puts every code and FP4 scale byte at its MOE_LAYOUT_TILE16 position
    (bit-exact against the index transform of the row-major arrays) and leaves the
    order-free arrays (FP8 block scales, NVFP4 globals) as they are."""
    b = S.routed_bank(11, fmt, E, H, I)
    pk = device_bank(b, packed=True)
    torch.cuda.synchronize()
    assert pk.layout == qm.MOE_LAYOUT_TILE16

    def rows2d(a):  # byte rows
        a = np.ascontiguousarray(a)
        return a.view(np.uint8).reshape(a.shape[0] * a.shape[1], -1)

    def got(t):
        a = t.cpu().numpy()
        return a.view(np.uint8).reshape(a.shape[0] * a.shape[1], -1)

    np.testing.assert_array_equal(got(pk.gate_up), tile16_np(rows2d(b.gate_up), 16))
    np.testing.assert_array_equal(got(pk.down), tile16_np(rows2d(b.down), 16))
    if fmt == "fp8blk":
        np.testing.assert_array_equal(pk.gate_up_scale.cpu().numpy(), b.gate_up_scale)
        np.testing.assert_array_equal(pk.down_scale.cpu().numpy(), b.down_scale)
    elif fmt != "bf16":
        unit = 2 if fmt == "nvfp4" else 1
        np.testing.assert_array_equal(got(pk.gate_up_scale), tile16_np(rows2d(b.gate_up_scale), unit))
        np.testing.assert_array_equal(got(pk.down_scale), tile16_np(rows2d(b.down_scale), unit))
    if fmt == "nvfp4":
        np.testing.assert_array_equal(pk.gate_up_global.cpu().numpy(), b.gate_up_global)
        np.testing.assert_array_equal(pk.down_global.cpu().numpy(), b.down_global)


def q4_0_pieces_np(a: np.ndarray) -> np.ndarray:
    """The MOE_LAYOUT_TILE16 bytes of row-major q4_0 codes [rows, H/2], written from the layout's
    definition: piece (s, g) of a row holds one little-endian dword per block 4s+q, made of that
    block's elements 8g..8g+7 (element 8g+2i at bit 4i, element 8g+2i+1 at bit 16+4i), and the
    pieces go to their tile-16 places like any 16-byte unit."""
    R, P = a.shape
    blk = a.reshape(R, P // 16, 16)
    el = np.concatenate([blk & 0xF, blk >> 4], axis=2).astype(np.uint32)  # [R, block, element]
    el = el.reshape(R, P // 64, 4, 4, 8)                                    # [R, s, q, g, j]
    j = np.arange(8)
    shift = np.where(j % 2 == 0, 4 * (j // 2), 16 + 4 * (j // 2)).astype(np.uint32)
    dw = (el << shift).sum(axis=-1, dtype=np.uint32)                        # disjoint bits
    rows = np.ascontiguousarray(dw.transpose(0, 1, 3, 2)).astype("<u4").reshape(R, -1).view(np.uint8)
    return tile16_np(rows, 16)


def test_pack_bank_q4_0_regroups_nibbles():
    """Q4_0 codes are regrouped per 16-byte piece (bit-exact against the layout written out
    above); the fp16 scales move in units of one step's 4 scales (8 bytes)."""
    b = S.routed_bank(19, "q4_0", 3, 256, 128)
    pk = device_bank(b, packed=True)
    torch.cuda.synchronize()

    def rows2d(a):
        a = np.ascontiguousarray(a)
        return a.view(np.uint8).reshape(a.shape[0] * a.shape[1], -1)

    def got(t):
        a = t.cpu().numpy()
        return a.view(np.uint8).reshape(a.shape[0] * a.shape[1], -1)

    np.testing.assert_array_equal(got(pk.gate_up), q4_0_pieces_np(rows2d(b.gate_up)))
    np.testing.assert_array_equal(got(pk.down), q4_0_pieces_np(rows2d(b.down)))
    np.testing.assert_array_equal(got(pk.gate_up_scale), tile16_np(rows2d(b.gate_up_scale), 8))
    np.testing.assert_array_equal(got(pk.down_scale), tile16_np(rows2d(b.down_scale), 8))


def _transposed_mx(b):
    """The MOE_LAYOUT_MXFP4_T arrays of a row-major MXFP4 bank: codes [E, K/2, N], scales [E, K/32, N]."""
    return tuple(np.ascontiguousarray(a.transpose(0, 2, 1)) for a in (b.gate_up, b.gate_up_scale, b.down, b.down_scale))


def _dev_transposed(b, arrays, I=None):
    gu, gus, dn, dns = (to_dev(a) for a in arrays)
    return qm.DeviceBank("mxfp4", b.E, b.H, b.I if I is None else I, gu, gus, dn, dns, layout=qm.MOE_LAYOUT_MXFP4_T)


def test_pack_bank_from_transposed_mxfp4_equals_row_major():
    """An MXFP4 bank stored transposed (blocks_t [K/2, N], scales [K/32, N]) packs to exactly
    the bytes of the same bank stored row-major."""
    b = S.routed_bank(13, "mxfp4", 3, 512, 192)
    want = device_bank(b)
    got = qm.moe_pack_bank(_dev_transposed(b, _transposed_mx(b)))
    torch.cuda.synchronize()
    for name in ("gate_up", "gate_up_scale", "down", "down_scale"):
        assert torch.equal(getattr(got, name), getattr(want, name)), name


def test_transposed_mxfp4_rank_slice_matches_full_bank():
    """A rank's own storage of a transposed MXFP4 bank: gate_up columns [lo,hi) and [I+lo,I+hi)
    of blocks_t and its scales, down rows [lo/2,hi/2) of blocks_t and [lo/32,hi/32) of its scales
    (the slice is along N for gate_up and along K for down).  Packed, it gives the same result as
    the full bank's slice [lo, hi), and both match the oracle."""
    E, H, I, k, T, lo, hi = 8, 512, 256, 2, 12, 64, 192
    b, sh = S.routed_bank(17, "mxfp4", E, H, I), S.shared_bank(17, "mxfp4", H, I)
    x = S.tokens(17, T, H)
    _, ids, w, _ = O.route(x, S.router_weight(17, E, H), None, k, True)
    ref = O.expert_forward(b, sh, x, ids, w, lo, hi)

    def rank(bank):
        gu, gus, dn, dns = _transposed_mx(bank)
        cols = np.r_[lo:hi, I + lo:I + hi]
        own = (gu[:, :, cols], gus[:, :, cols], dn[:, lo // 2:hi // 2, :], dns[:, lo // 32:hi // 32, :])
        return qm.moe_pack_bank(_dev_transposed(bank, [np.ascontiguousarray(a) for a in own], I=hi - lo))

    al = qm.moe_align(to_dev(ids.astype(np.int32)), E, 16)
    xd, wd = bf16_dev(x), to_dev(w.astype(np.float32))
    full = qm.moe_expert_forward(device_bank(b), device_bank(sh), xd, wd, al, lo, hi).cpu().numpy()
    own = qm.moe_expert_forward(rank(b), rank(sh), xd, wd, al, 0, hi - lo).cpu().numpy()
    np.testing.assert_array_equal(own, full)
    check_close("transposed MXFP4 rank slice", own, ref)


def test_forward_rejects_row_major_bank():
    inp, r = inputs_for(1, 8)
    rows = device_bank(inp.routed, packed=False)
    dev = "cuda"
    al = qm.moe_align(to_dev(r["ids"].astype(np.int32), dev), inp.routed.E, 16)
    with pytest.raises(qm.MoeError, match="TILE16"):
        qm.moe_expert_forward(rows, None, bf16_dev(inp.x), to_dev(r["w"].astype(np.float32), dev), al, 0, 128)


def _forward_gpu(inp, ids, w, lo, hi, bm=None, out_dtype=torch.float32, banks=None):
    cfg = inp.cfg
    T = ids.shape[0]
    bm = bm or qm.choose_block_m(T, cfg.k, cfg.E)
    rb, sb = banks or dev_banks(inp)
    al = qm.moe_align(to_dev(ids), cfg.E, bm)
    out = qm.moe_expert_forward(rb, sb, bf16_dev(inp.x), to_dev(w.astype(np.float32)), al, lo, hi,
                                out_dtype=out_dtype)
    return out.float().cpu().numpy()


FORWARD_CASES = [(1, 16, (0, 128)), (1, 16, (0, 64)), (1, 16, (64, 128)),
                 (2, 1, (0, 256)), (2, 8, (0, 256)), (2, 32, (0, 256)), (2, 64, (0, 256)), (2, 64, (0, 512)),
                 (2, 1, (0, 512)),
                 (4, 1, (0, 256)), (4, 64, (0, 256)), (4, 64, (0, 512)),
                 (5, 1, (0, 1024)), (5, 16, (0, 1024)), (5, 16, (1024, 2048)),
                 # MXFP4 slices off the 128-wide chunk grid: a masked K tail, unaligned scale spans
                 (5, 16, (0, 96)), (5, 16, (32, 160)), (5, 1, (992, 2048)),
                 # MXFP4 with 64 slice columns per gate_up workgroup (>= 4 pairs per expert), a
                 # last column group half past the slice
                 (5, 256, (0, 96)), (5, 256, (32, 160)), (5, 256, (1024, 2048)),
                 # MXFP4 slices of 3, 4 and 8 K steps, with K tails inside a step
                 (5, 16, (0, 480)), (5, 64, (512, 896)), (5, 256, (32, 1024)),
                 # bf16 stacked experts (issue #62 "Suggested staging" item 1)
                 (6, 1, (0, 256)), (6, 64, (0, 256)), (6, 16, (32, 160)), (6, 8, (0, 512)),
                 # q4_0 experts (issue #62 "Suggested staging" item 3), no shared expert
                 (7, 1, (0, 256)), (7, 64, (0, 256)), (7, 16, (128, 384)), (7, 8, (0, 512)), (7, 3, (384, 512)),
                 # q4_0 slices on its 32-element block (issue #62 "What it touches" item 2): down's K
                 # range starts or ends inside a 128-wide step
                 (7, 16, (32, 160)), (7, 8, (96, 512)), (7, 1, (0, 32)), (7, 64, (224, 480)), (7, 5, (480, 512))]


@pytest.mark.parametrize("cid,T,sl", FORWARD_CASES)
def test_expert_forward_matches_oracle(cid, T, sl):
    """Oracle routing fed to both sides; GPU align + gate_up + down + combine vs oracle."""
    inp, r = inputs_for(cid, T)
    lo, hi = sl
    ref = O.expert_forward(inp.routed, inp.shared, inp.x, r["ids"], r["w"], lo, hi)
    got = _forward_gpu(inp, r["ids"], r["w"], lo, hi)
    check_close(f"cfg{cid} T={T} slice=[{lo},{hi})", got, ref)


def test_large_activation_rows_stay_exact():
    """Two rows of x scaled by 2^16 (exact in bf16; h grows by 2^32), far beyond what a 16-bit
    float with 5 exponent bits holds: the bf16 operands of every kernel keep both the scaled
    rows and the others within the tolerance."""
    inp, r = inputs_for(2, 8)
    x = inp.x.copy()
    rows = [0, 5]
    big = (x[rows].astype(np.uint32) << 16).view(np.float32) * np.float32(65536.0)  # exact in bf16
    x[rows] = (big.view(np.uint32) >> 16).astype(np.uint16)
    assert np.abs(big).max() > 65504
    ref = O.expert_forward(inp.routed, inp.shared, x, r["ids"], r["w"], 0, 256)
    got = _forward_gpu(dataclasses.replace(inp, x=x), r["ids"], r["w"], 0, 256, banks=dev_banks(inp))
    rest = [t for t in range(8) if t not in rows]
    check_close("large rows", got[rows], ref[rows])
    check_close("other rows", got[rest], ref[rest])


@pytest.mark.parametrize("cid,T,scale_exp", [(2, 8, -20), (2, 8, -16), (2, 64, -30), (4, 64, -20), (5, 16, -20),
                                             (6, 8, -20), (7, 8, -20)])
def test_tiny_activation_rows_keep_their_precision(cid, T, scale_exp):
    """Token rows scaled by 2^scale_exp (exact in bf16), so that x and h fall far below the
    range of a 16-bit float with 5 exponent bits: every format must keep those rows' relative
    accuracy (bf16 operands and fp32 accumulation have fp32's exponent range).  Each scaled row is checked against 1e-2 * its own max|ref|, without
    the absolute floor of the layer-wide tolerance, which would hide any error at this size."""
    inp, r = inputs_for(cid, T)
    x = inp.x.copy()
    rows = [1, T - 2] if T > 2 else [0]
    f = (x[rows].astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** scale_exp)
    x[rows] = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert ((x[rows].astype(np.uint32) << 16).view(np.float32) == f).all()  # exact
    hi = inp.cfg.I // 2
    ref = O.expert_forward(inp.routed, inp.shared, x, r["ids"], r["w"], 0, hi)
    got = _forward_gpu(dataclasses.replace(inp, x=x), r["ids"], r["w"], 0, hi, banks=dev_banks(inp))
    for t in rows:
        err = float(np.abs(got[t] - ref[t]).max())
        bound = 1e-2 * float(np.abs(ref[t]).max())
        print(f"[tiny] cfg{cid} T={T} 2^{scale_exp} row {t}: max|d| {err:.3e}, bound {bound:.3e}, "
              f"ratio {err / bound:.3f}", flush=True)
        assert bound > 0 and err <= bound, (t, err, bound)
    rest = [t for t in range(T) if t not in rows]
    check_close(f"cfg{cid} rows beside the tiny ones", got[rest], ref[rest])


@pytest.mark.parametrize("bm", [16, 128])
def test_ids_outside_the_bank_leave_other_tokens_exact(bm):
    """A caller error: ids outside [0, E) in two tokens.  moe_align drops those pairs (they
    appear nowhere in its output) and the forward pass leaves every other token's row as the
    oracle computes it."""
    inp, r = inputs_for(2, 32)
    E = inp.cfg.E
    ids = r["ids"].copy()
    ids[3, 2], ids[17, 7] = -1, E
    al = qm.moe_align(to_dev(ids), E, bm)
    got_al = align_np(al)
    ok = np.ones(ids.shape, bool)
    ok[3, 2] = ok[17, 7] = False
    sid = got_al["sorted_ids"]
    real = np.sort(sid[sid < ids.size])
    np.testing.assert_array_equal(real, np.flatnonzero(ok.ravel()))
    assert got_al["counts"].sum() == ids.size - 2
    rb, sb = dev_banks(inp)
    out = qm.moe_expert_forward(rb, sb, bf16_dev(inp.x), to_dev(r["w"].astype(np.float32)), al, 0, 256)
    got = out.cpu().numpy()
    good = [t for t in range(32) if t not in (3, 17)]
    sub = dataclasses.replace(inp, x=np.ascontiguousarray(inp.x[good]))
    ref = O.expert_forward(sub.routed, sub.shared, sub.x, r["ids"][good], r["w"][good], 0, 256)
    check_close(f"tokens without dropped pairs bm={bm}", got[good], ref)


@pytest.mark.parametrize("bm", [16, 32, 64, 128])
def test_expert_forward_any_block_m(bm):
    inp, r = inputs_for(2, 64)
    ref = O.expert_forward(inp.routed, inp.shared, inp.x, r["ids"], r["w"], 0, 256)
    check_close(f"cfg2 T=64 bm={bm}", _forward_gpu(inp, r["ids"], r["w"], 0, 256, bm=bm), ref)


TILED_CASES = [(1, 16, (0, 128)), (1, 16, (32, 96)), (2, 64, (0, 256)), (2, 32, (0, 96)), (2, 8, (64, 512)),
               (4, 64, (0, 256)), (4, 64, (256, 512)), (6, 64, (0, 256)), (6, 32, (32, 160))]


@pytest.mark.parametrize("cid,T,sl", TILED_CASES)
def test_tiled_kernels_match_oracle(cid, T, sl):
    """128-row align blocks select the prefill GEMMs (NVFP4, fp8-block, bf16); small cases
    cover partial column tiles and a 32-wide K tail."""
    inp, r = inputs_for(cid, T)
    lo, hi = sl
    ref = O.expert_forward(inp.routed, inp.shared, inp.x, r["ids"], r["w"], lo, hi)
    check_close(f"tiled cfg{cid} T={T} [{lo},{hi})", _forward_gpu(inp, r["ids"], r["w"], lo, hi, bm=128), ref)


@pytest.mark.parametrize("fmt,H,I,sl,T,bm", [
    ("nvfp4", 384, 224, (0, 224), 300, 128), ("nvfp4", 384, 224, (32, 160), 257, 256),
    ("nvfp4", 256, 128, (0, 128), 1, 128), ("nvfp4", 640, 96, (0, 96), 700, 128),
    ("fp8blk", 384, 256, (0, 256), 300, 128), ("fp8blk", 640, 384, (128, 384), 257, 256),
    ("fp8blk", 256, 128, (0, 128), 1, 128),
    ("bf16", 384, 224, (32, 160), 257, 256), ("bf16", 640, 96, (0, 96), 700, 128)])
def test_wide_kernels_ragged_shapes(fmt, H, I, sl, T, bm):
    """Prefill GEMMs on shapes that leave partial work everywhere: a last down column group
    half past H (H = 384, 640), a last gate_up column group partly past the slice and a down K
    tail (slice widths 224, 128 and 96 are not multiples of 128), shared-expert rows ending inside a
    32-row tile, align blocks of 256 rows, and a single token.  fp8-block slices are multiples of
    the 128-wide scale block."""
    E, k, seed = 6, 2, 23
    b, sh = S.routed_bank(seed, fmt, E, H, I), S.shared_bank(seed, fmt, H, I)
    x = S.tokens(seed, T, H)
    _, ids, w, _ = O.route(x, S.router_weight(seed, E, H), None, k, True)
    lo, hi = sl
    ref = O.expert_forward(b, sh, x, ids, w, lo, hi)
    al = qm.moe_align(to_dev(ids.astype(np.int32)), E, bm)
    got = qm.moe_expert_forward(device_bank(b), device_bank(sh), bf16_dev(x), to_dev(w.astype(np.float32)), al,
                                lo, hi).float().cpu().numpy()
    check_close(f"wide {fmt} H={H} I={I} [{lo},{hi}) T={T} bm={bm}", got, ref)


def _random_case(seed):
    """A seeded draw of format, shapes, slice, routing width, token count, align block size and
    shared expert, inside the constraints the ABI states for each format."""
    rng = np.random.default_rng(1000 + seed)
    fmt = S.FORMATS[seed % len(S.FORMATS)]
    unit = {"nvfp4": 32, "fp8blk": 128, "mxfp4": 32, "bf16": 32, "q4_0": 128}[fmt]
    E = int(rng.integers(2, 17))
    H = 128 * int(rng.integers(1, 7))
    I = unit * int(rng.integers(1, max(2, 768 // unit) + 1))
    a, b = sorted(rng.choice(I // unit + 1, 2, replace=False))
    lo, hi = unit * int(a), unit * int(b)
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.choice([0, 1, 2, 7, 16, 33, 64, 129, 300]))
    bm = int(rng.choice([16, 32, 64, 128]))
    shared = bool(rng.integers(0, 2))
    return fmt, E, H, I, lo, hi, k, T, bm, shared


@pytest.mark.parametrize("seed", range(30))
def test_random_shapes_match_oracle(seed):
    """Seeded random layers over every format: the forward pass on the GPU against the oracle
    (the streaming kernels for align blocks below 128 and for MXFP4 / Q4_0, the prefill GEMMs
    otherwise), including T = 0, single tokens, slices anywhere in [0, I) and odd expert counts."""
    fmt, E, H, I, lo, hi, k, T, bm, shared = _random_case(seed)
    b = S.routed_bank(seed, fmt, E, H, I)
    sh = S.shared_bank(seed, fmt, H, I) if shared else None
    x = S.tokens(seed, T, H)
    _, ids, w, _ = O.route(x, S.router_weight(seed, E, H), None, k, True)
    ref = O.expert_forward(b, sh, x, ids, w, lo, hi)
    al = qm.moe_align(to_dev(ids.astype(np.int32).reshape(T, k)), E, bm)
    got = qm.moe_expert_forward(device_bank(b), device_bank(sh) if sh is not None else None, bf16_dev(x),
                                to_dev(w.astype(np.float32).reshape(T, k)), al, lo, hi).float().cpu().numpy()
    assert got.shape == (T, H)
    check_close(f"random {fmt} E={E} H={H} I={I} [{lo},{hi}) k={k} T={T} bm={bm} shared={shared}", got, ref)


@pytest.mark.parametrize("fmt,E,H,I,lo,hi,k,T,shared", [
    ("mxfp4", 40, 1152, 640, 0, 640, 6, 100, True),     # 5 column groups, the last one half outside H
    ("nvfp4", 24, 2304, 1024, 128, 768, 8, 70, False),  # 9 column groups, slice inside I
    ("q4_0", 16, 1280, 512, 0, 512, 4, 130, True),      # 5 column groups
])
def test_down_column_groups_on_one_xcd(fmt, E, H, I, lo, hi, k, T, shared):
    """Slices of at least 512 with at least 512 pairs launch the streaming kernels with the column
    group as the fastest grid index, and down then maps its linear workgroup index so that the
    column groups of a sub-block share one XCD.  Column-group and sub-block counts that are not
    multiples of 8 exercise the remap and the plain order past the last whole group of 8."""
    assert hi - lo >= 512 and T * k >= 512
    seed = 71
    b = S.routed_bank(seed, fmt, E, H, I)
    sh = S.shared_bank(seed, fmt, H, I) if shared else None
    x = S.tokens(seed, T, H)
    _, ids, w, _ = O.route(x, S.router_weight(seed, E, H), None, k, True)
    ref = O.expert_forward(b, sh, x, ids, w, lo, hi)
    al = qm.moe_align(to_dev(ids.astype(np.int32).reshape(T, k)), E, 16)
    got = qm.moe_expert_forward(device_bank(b), device_bank(sh) if sh is not None else None, bf16_dev(x),
                                to_dev(w.astype(np.float32).reshape(T, k)), al, lo, hi).float().cpu().numpy()
    check_close(f"down XCD order {fmt} E={E} H={H} [{lo},{hi}) k={k} T={T}", got, ref)


@pytest.mark.parametrize("sl", [(0, 384), (128, 384)])
def test_fp8_prefill_zero_block_scales(sl):
    """fp8-block scales of 0 (an all-zero weight block) with nonzero codes: the block adds
    nothing.  Zeros sit at the first K block of a tile, inside a tile's K run, over a whole
    tile row of blocks (its gate output is 0) and in the shared expert; the prefill kernels keep
    each tile's accumulators in units of its current block scale, so every one of these is a
    separate path."""
    E, H, I, T, k, seed = 4, 512, 384, 300, 2, 31
    b, sh = S.routed_bank(seed, "fp8blk", E, H, I), S.shared_bank(seed, "fp8blk", H, I)
    b.gate_up_scale[:, 0, 0] = 0            # gate rows [0,128): first K block
    b.gate_up_scale[1:, 4, 2] = 0           # up rows [I+128, I+256): a middle K block
    b.gate_up_scale[2, 1, :] = 0            # expert 2, gate rows [128,256): every K block
    b.gate_up_scale[3, 3, 0:2] = 0          # expert 3, up rows [I, I+128): two leading blocks
    b.down_scale[:, 1, 1] = 0               # down rows [128,256), K block 1
    b.down_scale[0, 2, 0] = 0               # expert 0, down rows [256,384), first K block
    sh.gate_up_scale[0, 0, 3] = 0           # shared expert, gate rows [0,128), last K block
    sh.down_scale[0, 0, :] = 0              # shared expert, down rows [0,128): every K block
    x = S.tokens(seed, T, H)
    _, ids, w, _ = O.route(x, S.router_weight(seed, E, H), None, k, True)
    lo, hi = sl
    ref = O.expert_forward(b, sh, x, ids, w, lo, hi)
    al = qm.moe_align(to_dev(ids.astype(np.int32)), E, 128)
    got = qm.moe_expert_forward(device_bank(b), device_bank(sh), bf16_dev(x), to_dev(w.astype(np.float32)), al,
                                lo, hi).float().cpu().numpy()
    check_close(f"fp8 zero block scales [{lo},{hi})", got, ref)
    assert np.isfinite(got).all()


_oracle_cache = {}


def oracle_forward(cid, T, lo, hi):
    """The whole-layer oracle output for config `cid`, T tokens, slice [lo, hi), with the
    oracle's own routing (computed once per case: it is the slow part)."""
    key = (cid, T, lo, hi)
    if key not in _oracle_cache:
        inp, r = inputs_for(cid, T)
        _oracle_cache[key] = O.expert_forward(inp.routed, inp.shared, inp.x, r["ids"], r["w"], lo, hi)
    return _oracle_cache[key]


@pytest.mark.parametrize("cid,T,sl,bm", [(3, 8192, (0, 512), 128), (3, 8192, (0, 256), 128),
                                         (4, 4096, (0, 256), 128), (3, 8192, (0, 512), 64),
                                         (6, 8192, (0, 512), 128), (5, 256, (0, 1024), None)])
def test_prefill_full_size_every_row(cid, T, sl, bm):
    """Full-size layers at the block size the benchmark runs them with (align blocks of 128:
    the prefill GEMMs; 64 for config 3 runs the streaming kernels at full size), every token
    row compared element by element with the whole-layer oracle.  Config 3 has the Zipf-skewed
    routing, so its hot experts span many row blocks and their last blocks are ragged."""
    inp, r = inputs_for(cid, T)
    lo, hi = sl
    print(f"[prefill] cfg{cid} T={T} [{lo},{hi}) bm={bm}: oracle ...", flush=True)
    ref = oracle_forward(cid, T, lo, hi)
    got = _forward_gpu(inp, r["ids"], r["w"], lo, hi, bm=bm)
    assert np.isfinite(got).all()
    check_close(f"prefill cfg{cid} T={T} [{lo},{hi}) bm={bm} all {T} rows", got, ref)


@pytest.mark.parametrize("cid,T,sl", [(1, 16, (0, 128)), (2, 64, (0, 256)), (5, 16, (0, 1024)),
                                      # one token: the whole-layer call's in-kernel routing
                                      (2, 1, (0, 256)), (4, 1, (0, 256)), (5, 1, (0, 1024)), (6, 1, (0, 256)),
                                      (7, 1, (0, 256))])
def test_full_layer_matches_oracle(cid, T, sl):
    """The whole GPU path (route -> align -> forward) against the whole oracle layer,
    excluding tokens whose k-th/(k+1)-th logit gap is inside the near-tie window."""
    inp, r = inputs_for(cid, T)
    cfg = inp.cfg
    lo, hi = sl
    rb, sb = dev_banks(inp)
    bias = to_dev(inp.bias) if inp.bias is not None else None
    layer = qm.MoeLayer(rb, sb, bf16_dev(inp.router), bias, T, cfg.k, lo, hi, cfg.renormalize)
    got = layer(bf16_dev(inp.x)).cpu().numpy()
    sure = r["gap"] > NEAR_TIE
    np.testing.assert_array_equal(layer.ids.cpu().numpy()[sure], r["ids"][sure])
    ref = O.expert_forward(inp.routed, inp.shared, inp.x, r["ids"], r["w"], lo, hi)
    check_close(f"full layer cfg{cid} T={T} [{lo},{hi})", got[sure], ref[sure])


# fmt, E, H, I, k, T, slice, shared, bias, renormalize, block_m (None: the library's choice)
LAYER_CALL_CASES = [
    ("nvfp4", 256, 2048, 512, 8, 1, (0, 256), True, False, True, None),     # the Qwen3.6-shaped decode layer
    ("nvfp4", 8, 1024, 128, 8, 1, (0, 128), False, True, False, None),      # k = E: every expert picked
    ("nvfp4", 8, 1024, 128, 1, 1, (32, 96), True, True, True, None),        # k = 1
    ("fp8blk", 256, 2048, 512, 8, 1, (0, 256), True, True, True, None),
    ("mxfp4", 256, 4096, 2048, 8, 1, (0, 1024), True, False, True, None),   # the DeepSeek-V4-Flash-shaped layer
    ("bf16", 64, 1024, 256, 6, 1, (0, 256), True, False, False, None),
    ("q4_0", 100, 1024, 256, 8, 1, (32, 224), False, True, True, None),
    ("nvfp4", 1000, 1024, 128, 64, 1, (0, 128), False, True, True, None),   # E = 1000, k = 64
    # paths that enqueue the two calls: another block size, H without an 8-wave K split, T > 1
    ("nvfp4", 256, 2048, 512, 8, 1, (0, 256), True, False, True, 32),
    ("nvfp4", 8, 256, 128, 2, 1, (0, 128), False, False, True, None),
    ("nvfp4", 256, 2048, 512, 8, 5, (0, 256), True, True, True, None),
    ("mxfp4", 256, 4096, 2048, 8, 16, (0, 1024), True, False, True, None),
    # mid-size batches: 1024 pairs, a block size of 48, E = 1000
    ("nvfp4", 256, 2048, 512, 8, 128, (0, 512), True, True, True, None),
    ("nvfp4", 256, 2048, 512, 8, 40, (256, 512), False, True, False, 48),
    ("nvfp4", 1000, 1024, 128, 10, 100, (0, 128), False, True, True, None),
    # MXFP4's activation planes written by the split-K router GEMM (T = 256), and by the
    # activation kernel after the tiled router (T = 1024)
    ("mxfp4", 256, 4096, 2048, 8, 256, (0, 1024), True, False, True, None),
    ("mxfp4", 64, 512, 256, 4, 1024, (32, 256), True, True, True, None),
    # MXFP4 with fewer than 64 experts: waves of the router's first expert group that have no
    # experts still write their share of the activation planes (at H = 4096 the router splits K
    # 16 ways, 256 each: waves 0 and 1 own a 128-wide step; E <= 16 leaves wave 1 without experts)
    ("mxfp4", 16, 4096, 256, 4, 1, (0, 256), True, True, True, None),
    ("mxfp4", 16, 4096, 256, 4, 5, (0, 256), True, False, True, None),
    ("mxfp4", 8, 4096, 256, 2, 64, (32, 256), False, True, True, None),
    ("mxfp4", 40, 4096, 256, 4, 64, (0, 256), False, False, True, None),
]


@pytest.mark.parametrize("case", LAYER_CALL_CASES, ids=lambda c: "-".join(str(v) for v in c))
@pytest.mark.parametrize("ties", [False, True])
def test_layer_forward_equals_the_two_calls(case, ties):
    """moe_layer_forward gives exactly the outputs of moe_route_align followed by
    moe_expert_forward (logits, ids, weights, every alignment array and the layer output, bit
    for bit), both where one token's routing runs inside the gate_up kernel and where the call
    enqueues the two calls.  ties: three router rows are one scaled row, so three experts
    share the top logit (the lower index must rank first)."""
    fmt, E, H, I, k, T, (lo, hi), shared, with_bias, renorm, bm = case
    seed = 61
    b = S.routed_bank(seed, fmt, E, H, I)
    sh = S.shared_bank(seed, fmt, H, I) if shared else None
    rb, sb = device_bank(b), (device_bank(sh) if sh is not None else None)
    wr_np = S.router_weight(seed, E, H)
    x_np = S.tokens(seed, T, H)
    tied = sorted({E - 1, E // 2, 1 % E})
    if ties:  # 8 times row 0, signed so that token 0's logit is large and positive (exact in bf16)
        sgn = 1.0 if float(np.dot(x_np[0].astype(np.float64), wr_np[0].astype(np.float64))) >= 0 else -1.0
        for e in tied:
            wr_np[e] = (8 * sgn) * wr_np[0]
    x, wr = bf16_dev(x_np), bf16_dev(wr_np)
    bias = to_dev(S.zipf_bias(seed, E, 1.1) if not ties else np.zeros(E, np.float32)) if with_bias else None
    bm = bm or qm.choose_block_m(T, k, E, fmt)
    lg1, ids1, w1, al1 = qm.moe_route_align(x, wr, bias, k, bm, renorm)
    out1 = qm.moe_expert_forward(rb, sb, x, w1, al1, lo, hi)
    layer = qm.MoeLayer(rb, sb, wr, bias, T, k, lo, hi, renorm, block_m=bm)
    for buf in (layer.logits, layer.w, layer.out):
        buf.fill_(float("nan"))
    for buf in (layer.ids, layer.align.sorted_ids, layer.align.block_expert, layer.align.counts,
                layer.align.offsets, layer.align.total_padded):
        buf.fill_(-7)
    for buf in (layer.ws, layer.route_ws):  # no byte the call should write is left over (0xFF: e4m3 NaN)
        buf.fill_(0xFF)
    out2 = layer(x)
    torch.cuda.synchronize()
    assert torch.equal(layer.logits, lg1) and torch.equal(layer.ids, ids1) and torch.equal(layer.w, w1)
    a1, a2 = align_np(al1), align_np(layer.align)
    for key in a1:
        np.testing.assert_array_equal(a2[key], a1[key], err_msg=key)
    assert torch.equal(out2, out1)
    if ties:  # equal logits rank by index
        row = [int(e) for e in ids1[0].cpu().numpy()]
        picked = [e for e in row if e in tied]
        assert picked == sorted(picked), row
        if row[0] in tied:
            assert row[0] == tied[0], row


@pytest.mark.parametrize("cid,T,cuts,bm", [
    (1, 16, (0, 64, 128), None), (2, 64, (0, 256, 512), None), (4, 64, (0, 256, 512), None),
    (2, 8, (0, 128, 384, 512), None), (5, 16, (0, 96, 1024, 2048), None), (7, 16, (0, 128, 384, 512), None),
    (7, 16, (0, 32, 96, 288, 512), None), (5, 256, (0, 96, 1024, 2048), None),
    # the prefill GEMMs (align blocks of 128): full-size Zipf prefill, fp8-block at T = 4096, and
    # bf16 cut at 96 and 352 (slices of 96, 256 and 160: K tails inside a 64-wide stage)
    (3, 8192, (0, 256, 512), 128), (4, 4096, (0, 256, 512), 128), (6, 8192, (0, 96, 352, 512), 128),
    (2, 64, (0, 32, 160, 512), 128)])
def test_gpu_slices_sum_to_gpu_full(cid, T, cuts, bm):
    """Linearity in the intermediate index on the GPU: disjoint slices tiling [0, I) sum to
    the unsliced GPU result (issue #520 section 4), for both kernel families."""
    inp, r = inputs_for(cid, T)
    full = _forward_gpu(inp, r["ids"], r["w"], 0, inp.cfg.I, bm=bm)
    parts = sum(_forward_gpu(inp, r["ids"], r["w"], lo, hi, bm=bm) for lo, hi in zip(cuts[:-1], cuts[1:]))
    check_close(f"slice sum cfg{cid} T={T} cuts={cuts} bm={bm}", parts, full.astype(np.float64))


@pytest.mark.parametrize("cid", [2, 6, 7])
def test_pre_sliced_bank_equals_slice_of_full_bank(cid):
    """A rank's own storage [0, Il) gives bit-identical results to [lo, hi) of the full bank
    (NVFP4 with a shared expert, bf16, q4_0)."""
    inp, r = inputs_for(cid, 32)
    for lo, hi in ((0, 256), (256, 512), (128, 384)):
        full = _forward_gpu(inp, r["ids"], r["w"], lo, hi)
        own = (device_bank(S.slice_bank(inp.routed, lo, hi)),
               device_bank(S.slice_bank(inp.shared, lo, hi)) if inp.shared is not None else None)
        mine = _forward_gpu(inp, r["ids"], r["w"], 0, hi - lo, banks=own)
        np.testing.assert_array_equal(mine, full)


def test_negative_control_mis_sliced_up_rows_fails_parity():
    """Up rows taken at Il+lo instead of I+lo (a mis-sliced bank handed to the GPU) must be
    caught by the parity check: the check is sensitive (issue #520 section 5)."""
    inp, r = inputs_for(2, 32)
    lo, hi = 0, 256
    ref = O.expert_forward(inp.routed, inp.shared, inp.x, r["ids"], r["w"], lo, hi)
    bad = S.slice_bank(inp.routed, lo, hi)
    bad.gate_up[:, 256:] = inp.routed.gate_up[:, 256:512]
    bad.gate_up_scale[:, 256:] = inp.routed.gate_up_scale[:, 256:512]
    bad.gate_up_global[:, 256:] = inp.routed.gate_up_global[:, 256:512]
    got = _forward_gpu(inp, r["ids"], r["w"], 0, hi - lo,
                       banks=(device_bank(bad), device_bank(S.slice_bank(inp.shared, lo, hi))))
    err = np.abs(got - ref).max()
    tol = 1e-2 * np.abs(ref).max() + 1e-3
    print(f"[negative control] max|d|={err:.3e} vs tol {tol:.3e}", flush=True)
    assert err > tol


def test_forward_is_deterministic_and_bf16_output_matches():
    inp, r = inputs_for(2, 64)
    a = _forward_gpu(inp, r["ids"], r["w"], 0, 256)
    b = _forward_gpu(inp, r["ids"], r["w"], 0, 256)
    np.testing.assert_array_equal(a, b)
    c = _forward_gpu(inp, r["ids"], r["w"], 0, 256, out_dtype=torch.bfloat16)
    ref = O.expert_forward(inp.routed, inp.shared, inp.x, r["ids"], r["w"], 0, 256)
    check_close("cfg2 T=64 bf16 out", c, ref)
    np.testing.assert_array_equal(c, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_zero_tokens_is_a_no_op():
    inp, r = inputs_for(1, 16)
    rb, sb = dev_banks(inp)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    al = qm.moe_align(ids, 8, 16)
    out = qm.moe_expert_forward(rb, None, x, torch.empty((0, 2), device="cuda"), al, 0, 128)
    assert out.shape == (0, 256)
    lg, i2, w2 = qm.moe_route(x, bf16_dev(inp.router), None, 2)
    assert i2.shape == (0, 2)


@pytest.mark.parametrize("cid,T,bm", [(2, 32, None), (3, 8192, 128), (4, 64, 128), (5, 16, None), (6, 64, 128),
                                       (7, 16, None), (2, 1, None), (5, 1, None)])
def test_graph_replays_match_eager(cid, T, bm):
    """The three calls captured in a HIP graph, for every format and every kernel family
    (streaming, the one-token down + combine at T = 1, and the prefill GEMMs at align blocks
    of 128): every replay (with eager work and synchronisations in between) reproduces the
    eager result bit for bit."""
    inp, r = inputs_for(cid, T)
    cfg = inp.cfg
    rb, sb = dev_banks(inp)
    bias = to_dev(inp.bias) if inp.bias is not None else None
    half = cfg.I // 2
    layer = qm.MoeLayer(rb, sb, bf16_dev(inp.router), bias, T, cfg.k, 0, half, cfg.renormalize, block_m=bm)
    x = bf16_dev(inp.x)
    eager = layer(x).clone()
    ids_eager = layer.ids.clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(x)
    other = qm.MoeLayer(rb, sb, bf16_dev(inp.router), bias, T, cfg.k, half, cfg.I, cfg.renormalize, block_m=bm)
    for _ in range(3):
        layer.out.zero_()
        layer.ids.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.out, eager) and torch.equal(layer.ids, ids_eager)
        other(x)  # eager work between replays
        torch.cuda.synchronize()
