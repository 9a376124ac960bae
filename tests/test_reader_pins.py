"""Pins of the channel-selection reader's oracle (CPU only): the rotation, the
ternary sketch and its byte format, the partial scan, the output-level score
and top K, and the rank-32 recovery map, each against something other than
the oracle itself (the dense Sylvester matrix, hand-derived values, a limit
in which the sketch is exact, brute force, an independent singular value
decomposition, the page's figures)."""
import json
import math
import os

import numpy as np
import pytest

import oracle as O
from oracle import reader as Rd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_bf16(rng, shape, scale=0.02):
    f = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------- rotation

@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128])
def test_fast_transform_equals_dense_sylvester_matrix(n):
    rng = np.random.default_rng(n)
    H = Rd.hadamard(n)
    # Sylvester matrices: entries +-1, rows orthogonal, H H^T = n I
    assert set(np.unique(H)) <= {-1.0, 1.0}
    np.testing.assert_array_equal(H @ H.T, n * np.eye(n))
    v = rng.integers(-1000, 1000, (5, n)).astype(np.float64)  # exact arithmetic
    np.testing.assert_array_equal(Rd.fwht(v), v @ H.T)
    np.testing.assert_array_equal(Rd.fwht(Rd.fwht(v)), n * v)  # H^2 = n I


def test_rotation_preserves_dot_products():
    """R = H diag(sigma) / sqrt(128) per block is orthogonal: g . x = (R g) . (R x);
    the unnormalised rotation gives g . x = (u . x'') / 128."""
    rng = np.random.default_rng(1)
    signs = np.where(rng.integers(0, 2, (4, 128)) == 1, 1, -1).astype(np.int8)
    g = rng.standard_normal((3, 512))
    x = rng.standard_normal(512)
    u = Rd.rotate(g, signs).reshape(3, 512)
    xr = Rd.rotate(x[None, :], signs).reshape(512)
    np.testing.assert_allclose(u @ xr / 128.0, g @ x, rtol=1e-12, atol=1e-12)
    # against the dense matrix, block by block
    Hm = Rd.hadamard(128)
    for b in range(4):
        np.testing.assert_allclose(Rd.rotate(x[None, :], signs)[0, b], Hm @ (signs[b] * x[128 * b:128 * (b + 1)]),
                                   rtol=0, atol=1e-12)


# ---------------------------------------------------------------- ternary code

def test_ternary_code_hand_derived():
    u = np.zeros(128)
    u[:4] = [4.0, -3.0, 1.0, 0.5]
    # sum |u| = 8.5, Delta = 0.7 * 8.5 / 128 = 0.046484375: all four kept
    c, s = Rd.ternary_code(u)
    np.testing.assert_array_equal(c[:4], [1, -1, 1, 1])
    assert not c[4:].any()
    assert s == np.float32(2.125 / 128)  # mean of 4, 3, 1, 0.5
    v = np.full(128, 0.1)
    v[0] = 10.0
    # sum = 10 + 12.7 = 22.7, Delta = 0.7 * 22.7 / 128 = 0.12414...: only 10 kept
    c, s = Rd.ternary_code(v)
    assert c[0] == 1 and not c[1:].any()
    assert s == np.float32(10.0 / 128)
    c, s = Rd.ternary_code(np.zeros(128))
    assert not c.any() and s == 0.0
    # equal magnitudes: every coordinate kept with its sign, scale = magnitude
    w = np.where(np.arange(128) % 3 == 0, -0.75, 0.75)
    c, s = Rd.ternary_code(w)
    np.testing.assert_array_equal(c, np.sign(w))
    assert s == np.float32(0.75 / 128)


def test_pair_sum_order_and_value():
    rng = np.random.default_rng(12)
    v = rng.integers(-10 ** 6, 10 ** 6, (4, 128)).astype(np.float64)  # exact in any order
    np.testing.assert_array_equal(Rd.pair_sum(v), v.sum(axis=-1))
    # the order is ((x0 + x1) + (x2 + x3)): for 2^53, 1, 1, -2^53 that gives 1, left to right 0
    w = np.array([2.0 ** 53, 1.0, 1.0, -(2.0 ** 53)])
    assert Rd.pair_sum(w) == 1.0
    assert ((w[0] + w[1]) + w[2]) + w[3] == 0.0


def test_ternary_code_scale_invariance():
    rng = np.random.default_rng(2)
    u = rng.standard_normal((6, 128))
    c1, s1 = Rd.ternary_code(u)
    c2, s2 = Rd.ternary_code(u * 8.0)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s2, s1 * np.float32(8.0))


# ---------------------------------------------------------------- byte format

def test_base3_bytes_hand_derived():
    codes = np.array([1, 0, -1, 1, 1, 0, 0], np.int8)
    row = Rd.pack_codes(codes)
    # digits (2, 1, 0, 2, 2) -> 2 + 1*3 + 0*9 + 2*27 + 2*81 = 221; channels 5, 6 and
    # the padding channels 7..9 are code 0 (digit 1): 1 + 3 + 9 + 27 + 81 = 121
    assert row.shape == (16,)
    assert row[0] == 221 and row[1] == 121 and not row[2:].any()
    assert Rd.sketch_row_bytes(768) == 160 and Rd.sketch_row_bytes(5) == 16 and Rd.sketch_row_bytes(81) == 32


def test_base3_roundtrip():
    rng = np.random.default_rng(3)
    for I in (1, 4, 5, 6, 37, 768):
        c = rng.integers(-1, 2, (3, 7, I)).astype(np.int8)
        rows = Rd.pack_codes(c)
        assert rows.max() < 243
        np.testing.assert_array_equal(Rd.unpack_codes(rows, I), c)


def test_sketch_layout_of_an_expert():
    """Codes come out (block, coordinate, channel) with channel j's codes
    those of its own rotated row."""
    rng = np.random.default_rng(4)
    w = rand_bf16(rng, (9, 256))
    signs = np.where(rng.integers(0, 2, (2, 128)) == 1, 1, -1).astype(np.int8)
    codes, scale = Rd.sketch_expert(w, signs)
    assert codes.shape == (2, 128, 9) and scale.shape == (2, 9)
    for j in (0, 4, 8):
        u = Rd.rotate(O.bf16_to_f64(w[j])[None, :], signs)[0]
        cj, sj = Rd.ternary_code(u)
        np.testing.assert_array_equal(codes[:, :, j], cj)
        np.testing.assert_array_equal(scale[:, j], sj)


# ---------------------------------------------------------------- scan and estimate

def test_scan_picks_largest_magnitudes_ties_to_lower_coordinate():
    rng = np.random.default_rng(5)
    xr = rng.standard_normal((3, 128))
    m = Rd.scan_mask(xr, 80)
    for b in range(3):
        order = np.lexsort((np.arange(128), -np.abs(xr[b])))
        np.testing.assert_array_equal(np.flatnonzero(m[b]), np.sort(order[:80]))
    tie = np.ones((1, 128))
    tie[0, 5] = -1.0
    np.testing.assert_array_equal(np.flatnonzero(Rd.scan_mask(tie, 80)[0]), np.arange(80))
    assert Rd.scan_mask(xr, 128).all()


def test_exact_sketch_full_scan_gives_exact_activation():
    """Rows whose rotated blocks are exactly ternary (u = alpha c): the sketch
    reproduces them and a full scan gives g_hat = g . x exactly."""
    rng = np.random.default_rng(6)
    signs = np.where(rng.integers(0, 2, (2, 128)) == 1, 1, -1).astype(np.int8)
    I = 5
    g = np.zeros((I, 256))
    for j in range(I):
        for b in range(2):
            c = rng.integers(-1, 2, 128).astype(np.float64)
            alpha = 2.0 ** rng.integers(-6, 2)
            u = alpha * c
            # invert the unnormalised rotation: H diag(s) g = u  <=>  g = diag(s) H u / 128
            g[j, 128 * b:128 * (b + 1)] = signs[b] * (Rd.hadamard(128) @ u) / 128.0
    u = Rd.rotate(g, signs)
    codes, scale = Rd.ternary_code(u)
    codes = codes.transpose(1, 2, 0)
    scale = scale.T
    x = rng.standard_normal(256)
    xr = Rd.rotate(x[None, :], signs)[0]
    est = Rd.sketch_estimate(codes, scale, xr, Rd.scan_mask(xr, 128))
    np.testing.assert_allclose(est, g @ x, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- score and top K

def test_select_top_brute_force_and_ties():
    rng = np.random.default_rng(7)
    ids = np.array([5, 2, 9])
    sc = rng.integers(0, 6, (3, 7)).astype(np.float64)  # many exact ties
    for K in (0, 1, 5, 11, 21):
        got = Rd.select_top(sc, ids, K)
        cands = [(-sc[s, j], ids[s], j, s) for s in range(3) for j in range(7)]
        want = sorted(s * 7 + j for (_, _, j, s) in sorted(cands)[:K])
        np.testing.assert_array_equal(got, want)


def test_scores_output_level_closed_form():
    a = np.array([0.25], np.float32)
    g = np.array([[0.0, math.log(3.0), -2.0]])
    v = np.array([[5.0, 2.0, -1.0]])
    dn = np.array([[1.0, 4.0, 0.5]], np.float32)
    sc = Rd.reader_scores(a, g, v, dn)
    # SiLU(0) = 0; SiLU(ln 3) = 0.75 ln 3; SiLU(-2) = -2 / (1 + e^2)
    want = [0.0, 0.25 * 4.0 * 0.75 * math.log(3.0) * 2.0, 0.25 * 0.5 * (2.0 / (1.0 + math.e ** 2))]
    np.testing.assert_allclose(sc[0], want, rtol=1e-14)


def test_reader_all_kept_equals_dense():
    rng = np.random.default_rng(8)
    E, I, H, k = 4, 6, 256, 2
    wg, wu, wd = (rand_bf16(rng, (E, I, H)) for _ in range(3))
    signs = np.where(rng.integers(0, 2, (2, 128)) == 1, 1, -1).astype(np.int8)
    h = rng.standard_normal(H).astype(np.float32)
    ids = np.array([3, 1])
    aff = np.array([0.625, 0.375], np.float32)
    r = Rd.reader_step(h, ids, aff, wg, wu, wd, signs, K=k * I)
    ref = O.dense_forward(h[None, :], ids[None, :], aff.astype(np.float64)[None, :], wg, wu, wd)[0]
    np.testing.assert_allclose(r["y"], ref, rtol=1e-12, atol=1e-15)
    assert len(r["kept"]) == k * I


# ---------------------------------------------------------------- recovery

def test_full_rank_recovery_is_exact():
    """With rank = H and unrounded coefficients U U^T = I, so the recovered
    output of the dropped channels is their exact sum when the estimate is
    exact (exact sketch and full scan are replaced here by p_hat = a)."""
    rng = np.random.default_rng(9)
    E, I, H, k = 3, 5, 16, 2
    wg, wu, wd = (rand_bf16(rng, (E, I, H), 0.3) for _ in range(3))
    h = rng.standard_normal(H).astype(np.float32)
    ids = np.array([2, 0])
    aff = np.array([0.7, 0.3], np.float32)
    U = Rd.recovery_basis(wd, rank=H)
    np.testing.assert_allclose(U.T @ U, np.eye(H), atol=1e-12)
    a = np.stack([O.expert_intermediate(h, wg[e], wu[e]) for e in ids])   # exact activations
    kept = np.array([1, 4, 7])                                              # s * I + j
    dropped = np.ones((k, I), bool)
    dropped.reshape(-1)[kept] = False
    b = np.stack([O.bf16_to_f64(wd[e]) @ U for e in ids])                  # unrounded b_j = U^T d_j
    y = O.channel_sparse_forward(h[None, :], ids[None, :], aff.astype(np.float64)[None, :], wg, wu, wd,
                                 kept[None, :])[0]
    y = y + Rd.recovery_term(U, b, aff.astype(np.float64), a, dropped)
    ref = O.dense_forward(h[None, :], ids[None, :], aff.astype(np.float64)[None, :], wg, wu, wd)[0]
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12)


def test_recovery_basis_against_svd():
    """The top left singular vectors of the stacked down columns (a planted
    rank-3 structure plus noise, so the top 3 are well separated): same
    projector as numpy's SVD, orthonormal, sign convention applied."""
    rng = np.random.default_rng(10)
    E, I, H = 3, 40, 24
    base = rng.standard_normal((H, 3)) * np.array([9.0, 6.0, 4.0])
    cols = base @ rng.standard_normal((3, E * I)) + 0.1 * rng.standard_normal((H, E * I))
    wd = (cols.T.reshape(E, I, H).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    U = Rd.recovery_basis(wd, rank=3)
    D = O.bf16_to_f64(wd).reshape(E * I, H).T
    Us, sv, _ = np.linalg.svd(D, full_matrices=False)
    np.testing.assert_allclose(U @ U.T, Us[:, :3] @ Us[:, :3].T, atol=1e-9)
    np.testing.assert_allclose(U.T @ U, np.eye(3), atol=1e-12)
    for c in range(3):
        assert U[np.argmax(np.abs(U[:, c])), c] > 0
    # captured energy = sum of the squared top singular values (Ky Fan)
    np.testing.assert_allclose(np.sum((U.T @ D) ** 2), np.sum(sv[:3] ** 2), rtol=1e-10)


def test_recovery_coefficients_round_once_to_bf16():
    rng = np.random.default_rng(11)
    U = np.linalg.qr(rng.standard_normal((32, 4)))[0]
    wd = rand_bf16(rng, (6, 32), 0.5)
    b = Rd.recovery_coefs(U, wd)
    exact = O.bf16_to_f64(wd) @ U
    back = O.bf16_to_f64(b)
    assert np.all(np.abs(back - exact) <= np.abs(exact) * 2.0 ** -8 + 1e-30)
    assert Rd.f64_to_bf16_bits(np.array([1.0, -2.0, 1.0 + 2.0 ** -8]))[0] == 0x3F80
    assert Rd.f64_to_bf16_bits(np.array([-2.0]))[0] == 0xC000
    assert Rd.f64_to_bf16_bits(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80      # tie to even
    assert Rd.f64_to_bf16_bits(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82  # tie to even (up)


# ---------------------------------------------------------------- the page's figures

def test_reader_settings_and_byte_figures_of_the_page():
    f = json.load(open(os.path.join(GOLDEN, "reader_settings.json")))
    assert (Rd.BLOCK, Rd.SCAN, Rd.RECOVERY_RANK) == (f["block"], f["scan"], f["rank"])
    H, I = 2048, 768
    assert f["bf16_block_bytes"] == Rd.BLOCK * 2
    # bytes per 128-coordinate block of one channel: its share of the code rows + its scale
    per_block = Rd.BLOCK * Rd.sketch_row_bytes(I) / I + 4
    assert abs(per_block - f["sketch_block_bytes_about"]) <= 2.0
    # sketch of gate and up against the channel's bf16 gate, up and down rows
    ch_bytes = 3 * H * 2
    mem = 2 * (H // Rd.BLOCK) * per_block / ch_bytes * 100
    assert 6.0 <= mem <= 9.0 and abs(mem - f["sketch_memory_percent_about"]) <= 1.5
    # the partial scan reads SCAN of BLOCK code rows per block
    scan = 2 * (H // Rd.BLOCK) * (Rd.SCAN * Rd.sketch_row_bytes(I) / I + 4) / ch_bytes * 100
    assert abs(scan - f["reads_percent"]["sketch"]) <= 0.6
    # 12.3% exact channels of the 8 x 768 candidates
    assert round(f["reads_percent"]["exact"] / 100 * 8 * I) == 756
    r = f["reads_percent"]
    assert abs(r["sketch"] + r["exact"] + r["recovery"] - r["total"]) < 1e-9
    # recovery map: bf16 b_j per channel; reads add the dropped channels' b_j and U (fp32)
    assert abs(Rd.RECOVERY_RANK * 2 / ch_bytes * 100 - f["recovery_memory_percent_about"]) <= 0.1
    routed = 8 * I * ch_bytes
    rec_pp = ((8 * I - 756) * Rd.RECOVERY_RANK * 2 + H * Rd.RECOVERY_RANK * 4) / routed * 100
    lo, hi = f["recovery_reads_pp"]
    assert lo <= rec_pp <= hi + 0.05
