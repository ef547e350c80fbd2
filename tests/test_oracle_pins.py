"""Pins of the fp64 CPU oracle against things other than itself (CPU only).

Each test ties one part of the oracle to an independent source: a public format table, a
library routine (torch dtype conversions, numpy matmul/sort, scipy softmax), a closed form,
brute force on tiny inputs, the raw normals the quantized weights were drawn from, or a
number the FreeToken pages print.  A plausible mistake in the oracle (dropped term, wrong
sign, index or operand) fails at least one of them.
"""
import itertools
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import oracle as O
from synth import synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if line:
            rows.append(line.split()[:2])
    return rows


def _bf16_to_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).to(torch.float64).numpy()


# ------------------------------------------------------------------ format tables

def test_e2m1_matches_ocp_table():
    for code, val in _golden("ocp_fp4_e2m1.txt"):
        v = O.e2m1(int(code))
        assert v == float(val) and np.signbit(v) == val.startswith("-"), (code, v, val)


def test_e2m1_matches_bitfield_formula():
    # OCP MX v1.0 FP4: value = (-1)^s * 2^(e-1) * (1 + m/2) for e > 0, (-1)^s * 0.5 * m for e = 0
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        ref = (2.0 ** (e - 1)) * (1 + m / 2) if e else 0.5 * m
        assert O.e2m1(code) == (-ref if s else ref)


def test_e4m3fn_all_codes_match_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([O.e4m3fn(b) for b in range(256)])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all() and nan.sum() == 2  # 0x7F and 0xFF
    assert (got[~nan] == ref[~nan]).all()
    assert (np.signbit(got[~nan]) == np.signbit(ref[~nan])).all()


def test_e4m3fn_spot_values():
    for code, val in _golden("ocp_fp8_e4m3_spot.txt"):
        assert O.e4m3fn(int(code, 16)) == float(val), code


def test_e8m0_all_codes_match_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([O.e8m0(b) for b in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert (got[:255] == ref[:255]).all()
    assert O.e8m0(127) == 1.0 and O.e8m0(0) == 2.0 ** -127


def test_f16_all_codes_match_numpy():
    """The q4_0 block scale decoder against numpy's binary16 for all 65536 codes."""
    codes = np.arange(65536, dtype=np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    got = np.array([O.f16(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    np.testing.assert_array_equal(got[~nan], ref[~nan])


def test_q4_0_one_hot_probe_locates_nibble_and_block_scale():
    """q4_0: a single code 9 (value 1 * d) at element c of row r, scale d = 2^-(b % 5) for block
    b, every other code 8 (zero): the oracle reads c through the block's nibble order (element j
    in byte j's low nibble, j + 16 in its high nibble) and the block's fp16 scale."""
    H, I = 128, 64
    b = S.routed_bank(1, "q4_0", 1, H, I)
    b.gate_up[:] = 0x88
    for blk in range(H // 32):
        b.gate_up_scale[0, :, blk] = np.float16(2.0 ** -(blk % 5)).view(np.uint16)
    for r, c in ((0, 0), (3, 15), (5, 16), (7, 31), (2 * I - 1, 70), (9, 127)):
        blk, j = c // 32, c % 32
        byte = 16 * blk + (j % 16)
        old = int(b.gate_up[0, r, byte])
        b.gate_up[0, r, byte] = (old & 0xF0) | 9 if j < 16 else (old & 0x0F) | 0x90
        W = O.dequant_gate_up(b, 0)
        assert W[r, c] == 2.0 ** -(blk % 5), (r, c)
        W[r, c] = 0
        assert (W == 0).all(), (r, c)
        b.gate_up[0, r, byte] = old


def test_bf16_matches_torch():
    bits = np.array([0, 0x3F80, 0xBF80, 0x0001, 0x7F7F, 0xC2F7, 0x3E4C, 0x8000], np.uint16)
    ref = _bf16_to_f64(bits)
    assert all(O.bf16(int(b)) == r for b, r in zip(bits, ref))


# ------------------------------------------------------------------ dequantization and layout

def _empty_bank(fmt, E, H, I):
    return S._alloc_bank(fmt, E, H, I)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_fp4_one_hot_probe_locates_nibble_scale_and_global(fmt):
    """One nonzero code: it must read back at exactly (row, col) with its own group scale
    (and per-row global) and nowhere else.  Pins the even-index-in-low-nibble packing, the
    group index c/16 (NVFP4) or c/32 (MXFP4), and the per-row global."""
    E, H, I = 2, 64, 32
    b = _empty_bank(fmt, E, H, I)
    grp = 16 if fmt == "nvfp4" else 32
    rng = np.random.default_rng(0)
    if fmt == "nvfp4":
        b.gate_up_scale[:] = rng.integers(0x08, 0x70, b.gate_up_scale.shape)  # positive e4m3
        b.gate_up_global[:] = rng.uniform(0.5, 2.0, b.gate_up_global.shape).astype(np.float32)
        b.down_scale[:] = rng.integers(0x08, 0x70, b.down_scale.shape)
        b.down_global[:] = rng.uniform(0.5, 2.0, b.down_global.shape).astype(np.float32)
    else:
        b.gate_up_scale[:] = rng.integers(120, 134, b.gate_up_scale.shape)
        b.down_scale[:] = rng.integers(120, 134, b.down_scale.shape)
    for (e, r, c, code) in [(1, 5, 37, 0x7), (0, 2 * I - 1, H - 1, 0xB), (1, 0, 0, 0x3), (0, 40, 18, 0xE)]:
        b.gate_up[:] = 0
        b.gate_up[e, r, c // 2] = code << 4 if c % 2 else code
        W = O.dequant_gate_up(b, e)
        scale = (torch.tensor([int(b.gate_up_scale[e, r, c // grp])], dtype=torch.uint8)
                 .view(torch.float8_e4m3fn if fmt == "nvfp4" else torch.float8_e8m0fnu)
                 .to(torch.float64).item())
        glob = float(b.gate_up_global[e, r]) if fmt == "nvfp4" else 1.0
        want = np.zeros_like(W)
        want[r, c] = [0, .5, 1, 1.5, 2, 3, 4, 6][code & 7] * (-1 if code & 8 else 1) * scale * glob
        np.testing.assert_array_equal(W, want)
        assert not O.dequant_gate_up(b, 1 - e).any()
    for (e, n, i, code) in [(0, 3, 17, 0x5), (1, H - 1, I - 1, 0x9)]:
        b.down[:] = 0
        b.down[e, n, i // 2] = code << 4 if i % 2 else code
        W = O.dequant_down(b, e)
        scale = (torch.tensor([int(b.down_scale[e, n, i // grp])], dtype=torch.uint8)
                 .view(torch.float8_e4m3fn if fmt == "nvfp4" else torch.float8_e8m0fnu)
                 .to(torch.float64).item())
        glob = float(b.down_global[e, n]) if fmt == "nvfp4" else 1.0
        want = np.zeros_like(W)
        want[n, i] = [0, .5, 1, 1.5, 2, 3, 4, 6][code & 7] * (-1 if code & 8 else 1) * scale * glob
        np.testing.assert_array_equal(W, want)


def test_fp8blk_one_hot_probe_locates_block_scale():
    E, H, I = 1, 256, 256
    b = _empty_bank("fp8blk", E, H, I)
    b.gate_up_scale[:] = np.arange(b.gate_up_scale.size, dtype=np.float32).reshape(b.gate_up_scale.shape) + 1
    b.down_scale[:] = 10 * (np.arange(b.down_scale.size, dtype=np.float32).reshape(b.down_scale.shape) + 1)
    for (r, c) in [(0, 0), (130, 5), (300, 200), (511, 255)]:
        b.gate_up[:] = 0
        b.gate_up[0, r, c] = 0x38  # 1.0
        W = O.dequant_gate_up(b, 0)
        want = np.zeros_like(W)
        want[r, c] = b.gate_up_scale[0, r // 128, c // 128]
        np.testing.assert_array_equal(W, want)
    b.down[:] = 0
    b.down[0, 200, 129] = 0xC0  # -2.0
    W = O.dequant_down(b, 0)
    assert W[200, 129] == -2.0 * b.down_scale[0, 1, 1] and np.count_nonzero(W) == 1


@pytest.mark.parametrize("fmt,H,I", [("nvfp4", 256, 64), ("fp8blk", 256, 128), ("mxfp4", 256, 64), ("bf16", 128, 64),
                                     ("q4_0", 256, 64)])
def test_dequant_reconstructs_generated_normals(fmt, H, I):
    """The oracle's decode of the generator's codes reproduces the N(0, 0.02) weights the
    generator drew, within each format's rounding bound.  Decoder and encoder are separate
    code; a wrong nibble order, scale index or global would blow the bound."""
    seed = 77
    b = S.routed_bank(seed, fmt, 2, H, I)
    for e in range(2):
        w_gu = S.normal_f64(seed, S.TAG_GATE_UP, e, 2 * I * H, S.WEIGHT_SIGMA).reshape(2 * I, H)
        w_dn = S.normal_f64(seed, S.TAG_DOWN, e, H * I, S.WEIGHT_SIGMA).reshape(H, I)
        for W, ref in ((O.dequant_gate_up(b, e), w_gu), (O.dequant_down(b, e), w_dn)):
            err = np.abs(W - ref)
            if fmt == "bf16":  # round to nearest with 8 significant bits: half an ulp <= 2^-8 |w|
                bound = np.abs(ref) * 2.0 ** -8 * 1.0001
            elif fmt == "q4_0":  # levels -8..7 of step d = amax/8: half a step, except that an
                # element near -amax's opposite extreme clamps to +7 (one full step off)
                amax = np.repeat(np.abs(ref).reshape(ref.shape[0], -1, 32).max(axis=2), 32, axis=1)
                bound = amax / 8 * (1 + 2.0 ** -10) * 1.0001 + amax * 2.0 ** -11
            elif fmt == "fp8blk":
                # e4m3 relative step 2^-3 -> |err| <= 2^-4 |w| (normals), plus subnormal floor
                si = np.repeat(np.repeat(np.abs(ref).reshape(ref.shape[0] // 128, 128, -1, 128)
                                         .max(axis=(1, 3)) / 448, 128, 0), 128, 1)
                bound = np.maximum(np.abs(ref) * 2.0 ** -4, si * 2.0 ** -10) * 1.0001
            else:
                g = 16 if fmt == "nvfp4" else 32
                amax = np.repeat(np.abs(ref).reshape(ref.shape[0], -1, g).max(axis=2), g, axis=1)
                # e2m1 step at most 2 units (between 4 and 6) -> half-step 1 unit = amax/6 (NVFP4:
                # the e4m3 scale adds <= 1/16 relative; MXFP4: one unit is amax/4 at most)
                bound = amax / 6 * (1 + 1 / 16) * 1.0001 + 1e-12 if fmt == "nvfp4" else amax / 4 * 1.0001
            assert (err <= bound).all(), (fmt, float((err / bound).max()))
            rel = np.linalg.norm(W - ref) / np.linalg.norm(ref)
            assert rel < {"nvfp4": 0.1, "mxfp4": 0.15, "fp8blk": 0.04, "bf16": 0.003, "q4_0": 0.12}[fmt], rel


# ------------------------------------------------------------------ routing

def test_router_logits_match_numpy_matmul():
    seed = 5
    x = S.tokens(seed, 7, 96)
    wr = S.router_weight(seed, 12, 96)
    bias = np.linspace(-1, 1, 12).astype(np.float32)
    got = O.router_logits(x, wr, bias)
    ref = _bf16_to_f64(x) @ _bf16_to_f64(wr).T + bias.astype(np.float64)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


def test_topk_brute_force_all_permutations_e8_k2():
    """Brute force over all ordered pairs: exactly one ordered k-tuple has every member
    ranking before every non-member and its members in rank order (rank: larger score,
    then lower index); it must be the oracle's selection."""
    rng = np.random.default_rng(1)
    score = np.round(rng.normal(size=(200, 8)), 1)  # rounding creates many exact ties
    ids, w, gap = O.topk(score, 2, True)
    for t in range(score.shape[0]):
        s = score[t]

        def before(a, b):
            return s[a] > s[b] or (s[a] == s[b] and a < b)

        winners = [p for p in itertools.permutations(range(8), 2)
                   if before(p[0], p[1]) and all(before(p[1], u) for u in range(8) if u not in p)]
        assert winners == [tuple(int(v) for v in ids[t])], (t, s, ids[t])
        np.testing.assert_allclose(w[t], scipy.special.softmax(s[list(ids[t])]), rtol=1e-14)
        third = max((u for u in range(8) if u not in winners[0]), key=lambda u: (s[u], -u))
        assert gap[t] == s[ids[t][1]] - s[third]


def test_topk_matches_numpy_lexsort_and_scipy_softmax():
    rng = np.random.default_rng(2)
    score = rng.normal(size=(64, 256))
    score[:, 17] = score[:, 3]  # exact ties: expert 3 must come first
    for renorm in (True, False):
        ids, w, _ = O.topk(score, 8, renorm)
        for t in range(score.shape[0]):
            order = np.lexsort((np.arange(256), -score[t]))[:8]
            assert (ids[t] == order).all()
            sm = scipy.special.softmax(score[t][order]) if renorm else scipy.special.softmax(score[t])[order]
            np.testing.assert_allclose(w[t], sm, rtol=1e-12)
        if renorm:
            np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-14)
    pos3 = [list(r).index(3) for r in ids if 3 in r and 17 in r]
    pos17 = [list(r).index(17) for r in ids if 3 in r and 17 in r]
    assert all(a < b for a, b in zip(pos3, pos17))


def test_topk_k_equals_e_is_dense_softmax():
    score = np.random.default_rng(3).normal(size=(5, 6))
    ids, w, gap = O.topk(score, 6, True)
    for t in range(5):
        np.testing.assert_allclose(w[t], scipy.special.softmax(score[t])[ids[t]], rtol=1e-14)
    assert np.isinf(gap).all()


def test_route_duplicate_router_rows_tie_to_lower_index():
    seed = 9
    x = S.tokens(seed, 32, 64)
    wr = S.router_weight(seed, 8, 64)
    wr[6] = wr[1]  # identical rows -> identical logits for every token
    _, ids, _, _ = O.route(x, wr, None, 8, True)
    for row in ids:
        assert list(row).index(1) + 1 == list(row).index(6)


def test_route_rounds_logits_to_fp32_before_selection():
    """Two logits equal in fp32 but not in fp64: the decision is taken in fp32 (lower index)."""
    x = np.zeros((1, 2), np.uint16)
    x[0, 0] = 0x3F80  # 1.0
    wr = np.zeros((3, 2), np.uint16)
    bias = np.array([0.0, 0.0, 0.0], np.float32)
    bias[0] = np.float32(1.0)
    bias[2] = np.float32(1.0)
    wr[1, 0] = 0x3F80  # expert 1 logit = 1.0 (bf16 weight) + 0
    _, ids, _, gap = O.route(x, wr, bias, 1, True)
    assert ids[0, 0] == 0 and gap[0] == 0.0


# ------------------------------------------------------------------ align

def _align_brute(ids, E, BM):
    """Definition by a library stable sort."""
    T, k = ids.shape
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    padded = -(-counts // BM) * BM
    offsets = np.concatenate([[0], np.cumsum(padded)])
    cap = O.align_capacity(T, k, E, BM)
    sorted_ids = np.full(cap, T * k, np.int64)
    be = np.full(cap // BM, -1, np.int64)
    pos = 0
    for e in range(E):
        run = order[pos:pos + counts[e]]
        sorted_ids[offsets[e]:offsets[e] + counts[e]] = run
        be[offsets[e] // BM:offsets[e + 1] // BM] = e
        pos += counts[e]
    return dict(sorted_ids=sorted_ids, block_expert=be, counts=counts, offsets=offsets,
                total_padded=np.array([offsets[-1]]))


@pytest.mark.parametrize("T,k,E,BM,kind", [
    (16, 2, 8, 16, "rand"), (64, 8, 256, 16, "rand"), (1, 8, 256, 16, "rand"), (0, 8, 256, 16, "rand"),
    (100, 4, 32, 64, "rand"), (50, 3, 8, 1, "rand"), (40, 8, 256, 32, "one_expert"), (33, 2, 9, 8, "two_experts"),
])
def test_align_matches_stable_sort_definition(T, k, E, BM, kind):
    if kind == "rand":
        ids = S.randint(11, T, T * k, E).reshape(T, k)
    elif kind == "one_expert":
        ids = np.full((T, k), E - 1, np.int32)
    else:
        ids = np.where(np.arange(T * k) % 3 == 0, 0, E - 1).astype(np.int32).reshape(T, k)
    got = O.align(ids, E, BM)
    ref = _align_brute(ids, E, BM)
    for key in ref:
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    # invariants
    assert got["counts"].sum() == T * k
    real = got["sorted_ids"][got["sorted_ids"] < T * k]
    assert sorted(real.tolist()) == list(range(T * k))
    assert (got["offsets"] % BM == 0).all()
    for e in range(E):
        run = got["sorted_ids"][got["offsets"][e]:got["offsets"][e + 1]]
        r = run[run < T * k]
        assert (np.diff(r) > 0).all() and (ids.reshape(-1)[r] == e).all()


@pytest.mark.parametrize("T,k,E,BM,cap", [
    # worked by hand: every expert's run can carry BM - 1 padding rows, then round up to BM
    (16, 2, 8, 16, 160),      # 32 pairs + 8*15 = 152 -> 160
    (1, 8, 256, 16, 3856),    # 8 + 256*15 = 3848 -> 3856
    (8192, 8, 256, 128, 98048),  # 65536 + 256*127 = 98048, already a multiple of 128
    (0, 8, 256, 16, 3840),    # no pairs: 256*15 = 3840
    (3, 1, 1, 4, 8),          # 3 + 3 = 6 -> 8
    (5, 2, 3, 1, 10),         # BM = 1: exactly the pairs
])
def test_align_capacity_hand_values(T, k, E, BM, cap):
    assert O.align_capacity(T, k, E, BM) == cap


@pytest.mark.parametrize("T,k,E,BM", [(2, 2, 3, 4), (3, 1, 3, 2), (1, 3, 4, 3), (4, 1, 2, 5)])
def test_align_capacity_bounds_every_routing(T, k, E, BM):
    """Brute force over every assignment of the T*k pairs to E experts: the padded total never
    exceeds the capacity, the capacity is a multiple of BM, and the worst assignment comes
    within one block of it when there are at least as many pairs as experts (one pair in each
    of E - 1 experts, the rest in the last, pads every run but one by BM - 1)."""
    cap = O.align_capacity(T, k, E, BM)
    assert cap % BM == 0
    worst = 0
    for ids in itertools.product(range(E), repeat=T * k):
        counts = np.bincount(np.array(ids), minlength=E)
        worst = max(worst, int((-(-counts // BM) * BM).sum()))
    assert worst <= cap
    if T * k >= E:
        assert cap - worst <= BM, (cap, worst)


# ------------------------------------------------------------------ expert layer

def _dense_swiglu(x64, Wgu, Wd, lo, hi, I):
    g = x64 @ Wgu[lo:hi].T
    u = x64 @ Wgu[I + lo:I + hi].T
    return (g / (1 + np.exp(-g)) * u) @ Wd[:, lo:hi].T


@pytest.mark.parametrize("fmt,H,I", [("nvfp4", 128, 64), ("fp8blk", 256, 256), ("mxfp4", 128, 64), ("bf16", 128, 64),
                                     ("q4_0", 128, 128)])
def test_forward_single_expert_is_dense_swiglu(fmt, H, I):
    """E=1, k=1, weight 1: a plain SwiGLU FFN on the dequantized matrices (numpy matmul)."""
    b = S.routed_bank(21, fmt, 1, H, I)
    x = S.tokens(21, 5, H)
    ids = np.zeros((5, 1), np.int32)
    w = np.ones((5, 1))
    lo, hi = (0, I)
    got = O.expert_forward(b, None, x, ids, w, lo, hi)
    ref = _dense_swiglu(_bf16_to_f64(x), O.dequant_gate_up(b, 0), O.dequant_down(b, 0), lo, hi, I)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)


def test_forward_k_equals_e_is_dense_softmax_mixture_plus_shared():
    H, I, E = 64, 32, 4
    b = S.routed_bank(31, "nvfp4", E, H, I)
    sh = S.shared_bank(31, "nvfp4", H, I)
    x = S.tokens(31, 6, H)
    wr = S.router_weight(31, E, H)
    _, ids, w, _ = O.route(x, wr, None, E, True)
    got = O.expert_forward(b, sh, x, ids, w, 0, I)
    x64 = _bf16_to_f64(x)
    lg = (x64 @ _bf16_to_f64(wr).T).astype(np.float32).astype(np.float64)
    p = scipy.special.softmax(lg, axis=1)
    ref = sum(p[:, [e]] * _dense_swiglu(x64, O.dequant_gate_up(b, e), O.dequant_down(b, e), 0, I, I)
              for e in range(E))
    ref = ref + _dense_swiglu(x64, O.dequant_gate_up(sh, 0), O.dequant_down(sh, 0), 0, I, I)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-14)


def test_forward_all_ones_closed_form():
    """Every code 1.0, every scale 1.0, every global 1.0: W = all-ones, so
    g = u = sum(x), a = silu(s)*s and y_n = Il * a for every n, weighted by w."""
    H, I, E = 32, 32, 4
    b = _empty_bank("nvfp4", E, H, I)
    b.gate_up[:] = 0x22
    b.down[:] = 0x22
    b.gate_up_scale[:] = 0x38
    b.down_scale[:] = 0x38
    b.gate_up_global[:] = 1.0
    b.down_global[:] = 1.0
    x = S.tokens(41, 3, H)
    ids = np.array([[0, 3], [2, 1], [1, 0]], np.int32)
    w = np.array([[0.7, 0.3], [0.5, 0.5], [0.9, 0.1]])
    for lo, hi in ((0, 32), (16, 32)):
        got = O.expert_forward(b, None, x, ids, w, lo, hi)
        s = _bf16_to_f64(x).sum(1)
        a = s / (1 + np.exp(-s)) * s
        want = np.repeat(((hi - lo) * a * w.sum(1))[:, None], H, axis=1)
        np.testing.assert_allclose(got, want, rtol=1e-13)


@pytest.mark.parametrize("fmt,H,I,cuts", [("nvfp4", 128, 128, (0, 16, 64, 128)),
                                          ("fp8blk", 256, 384, (0, 128, 384)),
                                          ("mxfp4", 128, 128, (0, 32, 96, 128)),
                                          ("bf16", 128, 96, (0, 32, 64, 96)),
                                          ("q4_0", 128, 256, (0, 128, 256))])
def test_forward_slices_sum_to_full(fmt, H, I, cuts):
    """Linearity in the intermediate index (issue #520 section 4): the partials of disjoint
    slices tiling [0, I) sum to the unsliced layer, routed and shared alike."""
    E = 6
    b = S.routed_bank(51, fmt, E, H, I)
    sh = S.shared_bank(51, fmt, H, I)
    x = S.tokens(51, 9, H)
    _, ids, w, _ = O.route(x, S.router_weight(51, E, H), None, 2, True)
    full = O.expert_forward(b, sh, x, ids, w, 0, I)
    parts = sum(O.expert_forward(b, sh, x, ids, w, lo, hi) for lo, hi in zip(cuts[:-1], cuts[1:]))
    assert np.abs(parts - full).max() <= 1e-12 * np.abs(full).max()


def test_forward_pre_sliced_bank_equals_slice_of_full_bank():
    """A rank's own storage (gate rows [lo,hi), up rows [I+lo,I+hi), down columns [lo,hi),
    globals split / replicated per the companion rule) is the slice [0, Il) of itself."""
    H, I, E = 128, 128, 4
    for fmt in ("nvfp4", "mxfp4"):
        b = S.routed_bank(61, fmt, E, H, I)
        x = S.tokens(61, 4, H)
        ids = np.array([[0, 1], [2, 3], [3, 0], [1, 2]], np.int32)
        w = np.full((4, 2), 0.5)
        for lo, hi in ((0, 64), (64, 128), (32, 96)):
            ref = O.expert_forward(b, None, x, ids, w, lo, hi)
            got = O.expert_forward(S.slice_bank(b, lo, hi), None, x, ids, w, 0, hi - lo)
            np.testing.assert_array_equal(got, ref)


def test_forward_negative_control_wrong_up_rows_is_detected():
    """Mis-slicing up rows at Il+lo instead of I+lo (the token-salad failure of issue #520
    section 3(c)) changes the result: the slice-sum check is sensitive to it."""
    H, I, E = 64, 64, 2
    b = S.routed_bank(71, "nvfp4", E, H, I)
    x = S.tokens(71, 4, H)
    ids = np.array([[0], [1], [0], [1]], np.int32)
    w = np.ones((4, 1))
    full = O.expert_forward(b, None, x, ids, w, 0, I)
    wrong = S.slice_bank(b, 0, 32)
    wrong.gate_up[:, 32:] = b.gate_up[:, 32:64]  # "up" rows taken from gate rows [32, 64)
    wrong.gate_up_scale[:, 32:] = b.gate_up_scale[:, 32:64]
    wrong.gate_up_global[:, 32:] = b.gate_up_global[:, 32:64]
    bad = O.expert_forward(wrong, None, x, ids, w, 0, 32) + O.expert_forward(b, None, x, ids, w, 32, 64)
    tol = 1e-2 * np.abs(full).max() + 1e-3 * np.abs(full).max()
    assert np.abs(bad - full).max() > tol


def test_forward_one_hot_token_reads_single_weight_column():
    """x = e_h, one expert, down = one-hot at (n, i): out[n] = silu(Wg[i,h]) Wu[I+i,h] Wd[n,i]."""
    H, I = 64, 32
    b = S.routed_bank(81, "nvfp4", 1, H, I)
    b.down[:] = 0
    b.down[0, 10, 7 // 2] = 0x2 << 4  # i = 7 (odd -> high nibble), value 1.0 * scale * global
    x = np.zeros((1, H), np.uint16)
    x[0, 23] = 0x3F80
    out = O.expert_forward(b, None, x, np.zeros((1, 1), np.int32), np.ones((1, 1)), 0, I)
    g = O.weight_gate_up(b, 0, 7, 23)
    u = O.weight_gate_up(b, 0, I + 7, 23)
    d = O.weight_down(b, 0, 10, 7)
    assert d != 0
    want = np.zeros(H)
    want[10] = g / (1 + np.exp(-g)) * u * d
    np.testing.assert_allclose(out[0], want, rtol=1e-14, atol=0)


# ------------------------------------------------------------------ layout numbers on the pages

def test_bank_layout_matches_page_byte_counts():
    g = {k: float(v) for k, v in _golden("page_layout_numbers.txt")}
    # NVFP4 expert (codes + e4m3 group scales) of the Qwen3.6 layer, both projections
    b = S._alloc_bank("nvfp4", 1, int(g["qwen36_hidden"]), int(g["qwen36_moe_intermediate"]))
    per_expert = b.gate_up[0].nbytes + b.gate_up_scale[0].nbytes + b.down[0].nbytes + b.down_scale[0].nbytes
    bank_gib = per_expert * g["qwen36_experts"] * g["qwen36_layers"] / 2 ** 30
    shared_gib = per_expert * g["qwen36_layers"] / 2 ** 30
    assert abs(bank_gib + shared_gib - g["qwen36_nvfp4_bank_gib"]) / g["qwen36_nvfp4_bank_gib"] < 0.005
    # DSV4 routed FP4 with 32-element scale blocks fits the TP=1 host footprint; 16-element
    # e4m3 groups would not
    m = S._alloc_bank("mxfp4", 1, 4096, 2048)
    mx = m.gate_up[0].nbytes + m.gate_up_scale[0].nbytes + m.down[0].nbytes + m.down_scale[0].nbytes
    assert mx * g["dsv4_total_experts"] / 2 ** 30 <= g["dsv4_host_gib_tp1"]
    assert 3 * 2048 * 4096 * (1 / 2 + 1 / 16) * g["dsv4_total_experts"] / 2 ** 30 > g["dsv4_host_gib_tp1"]
    assert g["dsv4_total_experts"] % 256 == 0
    # partial-sum payload bs*H*2 bytes: 8 KiB at H = 4096, 5,120 B at H = 2560
    assert 1 * 4096 * 2 == g["dsv4_allreduce_bytes_bs1"]
    assert 1 * g["r9700_allreduce_hidden"] * 2 == g["r9700_allreduce_bytes"]
