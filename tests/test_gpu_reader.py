"""GPU parity of the channel-selection reader (ternary-sketch screening,
output-level scores, exact top K, rank-32 recovery map) against the fp64
oracle in oracle/reader_oracle.py, through the C ABI.

Comparison rules
  * sketch codes, bytes and scales, the scanned coordinates and their x''
    values: bit-exact (both sides take the same fp64 operations in the same
    order, then round once);
  * estimates g_hat, v_hat: within the rigorous fp32 bound of their sums
    (summation depth <= 80 rows + 64 row groups + 1 scale product + 2 block
    groups);
  * kept list: bit-exact against the oracle's selection applied to the GPU's
    own fp32 scores (the decision taken in the kernel's precision); against
    the oracle's fp64 scores, every difference must lie within the scores'
    error at the K-th score (certified);
  * outputs y: rel-L2 <= 1e-3 and max-abs <= 5e-3 max|y_ref|; the recovery
    term alone (y with the map minus y without, same kept list) likewise.
"""
import numpy as np
import pytest

import oracle as O
import synth
from helpers import check_close, to_dev, upload_layer

R = O.reader
pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


@pytest.fixture(scope="module")
def mb():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_bound_routed_amd as m
    return m


def say(*a):
    print(*a, flush=True)


def reader_tables(mb, cfg, dev, signs, rank=0, iters=40):
    """Load-time arrays of the reader, built on the device from the weights."""
    import torch
    E, I, H = cfg.E, cfg.I, cfg.H
    nb, rowb = H // 128, mb.moe_sketch_row_bytes(I)
    dev["rot_signs"] = to_dev(np.ascontiguousarray(signs, np.int8).reshape(-1))
    dev["sketch"] = torch.empty(E * 2 * nb * 128 * rowb, dtype=torch.uint8, device="cuda")
    dev["sketch_scale"] = torch.empty((E, 2, nb, I), dtype=torch.float32, device="cuda")
    dev["down_norm"] = torch.empty((E, I), dtype=torch.float32, device="cuda")
    mb.moe_reader_sketch(cfg, dev["w_gate"], dev["w_up"], dev["rot_signs"], dev["sketch"], dev["sketch_scale"])
    mb.moe_down_norms(cfg, dev["w_down"], dev["down_norm"])
    if rank:
        dev["rec_basis"] = torch.empty((H, rank), dtype=torch.float32, device="cuda")
        dev["rec_coef"] = torch.empty((E, I, rank), dtype=torch.int16, device="cuda")
        mb.moe_recovery_basis(cfg, dev["w_down"], rank, iters, dev["rec_basis"])
        mb.moe_recovery_coefs(cfg, dev["rec_basis"], rank, dev["w_down"], dev["rec_coef"])
    torch.cuda.synchronize()
    return dev


def gpu_sketch(mb, dev, cfg):
    nb, rowb = cfg.H // 128, mb.moe_sketch_row_bytes(cfg.I)
    sk = dev["sketch"].cpu().numpy().reshape(cfg.E, 2, nb, 128, rowb)
    sc = dev["sketch_scale"].cpu().numpy()
    return sk, sc


def check_sketch(mb, dev, cfg, inp, signs, experts):
    """Codes, bytes and scales of the given experts: bit-exact."""
    sk, sc = gpu_sketch(mb, dev, cfg)
    out = {}
    for e in experts:
        for P, name in enumerate(("w_gate", "w_up")):
            codes, scale = R.sketch_expert(inp[name][e], signs)
            np.testing.assert_array_equal(sk[e, P], R.pack_codes(codes), err_msg="sketch bytes e%d P%d" % (e, P))
            np.testing.assert_array_equal(sc[e, P], scale, err_msg="sketch scale e%d P%d" % (e, P))
            out[(e, P)] = (codes, scale)
    return out


def make_reader_layer(mb, wl, inp, signs, max_tokens, K, rank=0, iters=40):
    dev = upload_layer(inp)
    cfg = mb.make_config(wl.H, wl.I, wl.E, wl.k, wl.block_b, max_tokens, max_keep=K, reader=1, rec_rank=rank)
    reader_tables(mb, cfg, dev, signs, rank, iters)
    return cfg, dev, mb.Layer(cfg, dev)


def inspect(mb, layer, cfg, h_np, ids_np, w_np, K):
    """moe_reader_inspect for given routes: xsel, xval, est, score, kept."""
    import torch
    M = h_np.shape[0]
    nb = cfg.H // 128
    h = to_dev(h_np)
    ids = to_dev(np.ascontiguousarray(ids_np, np.int32))
    w = to_dev(np.ascontiguousarray(w_np, np.float32))
    xsel = torch.empty((M, nb, 80), dtype=torch.uint8, device="cuda")
    xval = torch.empty((M, nb, 80), dtype=torch.float32, device="cuda")
    est = torch.empty((M, cfg.top_k, 2, cfg.I), dtype=torch.float32, device="cuda")
    score = torch.empty((M, cfg.top_k, cfg.I), dtype=torch.float32, device="cuda")
    kept = torch.empty((M, K), dtype=torch.int32, device="cuda")
    mb.moe_reader_inspect(layer.ctx, h, M, ids, w, K, xsel, xval, est, score, kept)
    torch.cuda.synchronize()
    return {"xsel": xsel.cpu().numpy(), "xval": xval.cpu().numpy(), "est": est.cpu().numpy(),
            "score": score.cpu().numpy(), "kept": kept.cpu().numpy().astype(np.int64)}


def est_bound(codes_scale, xr, mask, ids_t, I):
    """Rigorous bound on |fp32 estimate - exact| per (slot, P, channel):
    gamma_147 * sum over blocks of |scale| * sum over scanned |x''|."""
    n = 80 + 64 + 1 + 2
    gam = n * U32 / (1 - n * U32)
    ax = np.where(mask, np.abs(xr), 0.0).sum(axis=1)   # [nb]
    out = np.zeros((len(ids_t), 2, I))
    for s, e in enumerate(ids_t):
        for P in range(2):
            sc = codes_scale[(int(e), P)][1].astype(np.float64)    # [nb][I]
            out[s, P] = gam * (np.abs(sc) * ax[:, None]).sum(axis=0) + 1e-30
    return out


def check_token(mb, g, t, cfg, h_t, ids_t, w_t, cs, signs, K):
    """Stages 1-3 of one token against the oracle.  Returns (kept, oracle
    scores, estimate error bound)."""
    nb = cfg.H // 128
    xr = R.rotate(np.asarray(h_t, np.float64)[None, :], signs)[0]
    mask = R.scan_mask(xr)
    for b in range(nb):
        sel = np.nonzero(mask[b])[0]
        np.testing.assert_array_equal(g["xsel"][t, b], sel, err_msg="scan block %d" % b)
        np.testing.assert_array_equal(g["xval"][t, b], xr[b, sel].astype(np.float32), err_msg="x'' block %d" % b)
    k = len(ids_t)
    est_ref = np.zeros((k, 2, cfg.I))
    for s, e in enumerate(ids_t):
        for P in range(2):
            codes, scale = cs[(int(e), P)]
            est_ref[s, P] = R.sketch_estimate(codes, scale, xr, mask)
    bnd = est_bound(cs, xr, mask, ids_t, cfg.I)
    err = np.abs(g["est"][t].astype(np.float64) - est_ref)
    assert np.all(err <= bnd), "estimate error %.3e above its bound (ratio %.2f)" % (err.max(), (err / bnd).max())
    # scores in the kernel's precision: fp32 w * dn * |SiLU(g) v| from the GPU's estimates
    dn = np.stack([np.asarray(cs[("dn", int(e))], np.float32) for e in ids_t])
    ge, ve = g["est"][t, :, 0].astype(np.float64), g["est"][t, :, 1].astype(np.float64)
    sc_ref = R.reader_scores(w_t, ge, ve, dn)
    np.testing.assert_allclose(g["score"][t], sc_ref, rtol=4e-6, atol=1e-30)
    own = R.select_top(g["score"][t].astype(np.float64), ids_t, K)
    np.testing.assert_array_equal(g["kept"][t], own)
    # certified against the oracle's fp64 scores
    sc_or = R.reader_scores(w_t, est_ref[:, 0], est_ref[:, 1], dn)
    ref_kept = R.select_top(sc_or, ids_t, K)
    diff = np.setxor1d(own, ref_kept)
    if diff.size:
        thr = np.sort(sc_or.ravel())[::-1][K - 1]
        tol = 1e-4 * thr + 1e-30
        gap = np.abs(sc_or.ravel()[diff] - thr)
        assert np.all(gap <= tol), "kept set differs from the oracle's beyond the score error"
        say("  token %d: %d candidates at the K-th score differ (within %.1e)" % (t, diff.size, tol))
    return own


def oracle_tables(inp, signs, experts, mb, dev, cfg):
    cs = check_sketch(mb, dev, cfg, inp, signs, experts)
    dn_gpu = dev["down_norm"].cpu().numpy()
    for e in experts:
        ref = R.down_norms(inp["w_down"][e])
        ulp = np.abs(dn_gpu[e].view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
        assert ulp.max() <= 1, "down norms differ by %d ulp" % ulp.max()
        cs[("dn", int(e))] = dn_gpu[e]
    return cs


def routes_of(mb, layer, h_np):
    import torch
    M = h_np.shape[0]
    layer.route(to_dev(h_np), M)
    torch.cuda.synchronize()
    return layer.ids[:M].cpu().numpy().astype(np.int64), layer.w[:M].cpu().numpy()


# ----------------------------------------------------------------------------

SMALL = [
    # name, H, I, E, k, M, K
    ("h256_i128_e16_k2_m1", 256, 128, 16, 2, 1, 40),
    ("h384_i100_e8_k3_m3", 384, 100, 8, 3, 3, 77),       # 3 blocks (row groups left idle), ragged I
    ("h1024_i333_e32_k4_m2", 1024, 333, 32, 4, 2, 200),
    ("h256_i64_e264_k4_m2", 256, 64, 264, 4, 2, 30),     # E > 256: routing outside the screening
    ("h128_i40_e8_k2_m2_all", 128, 40, 8, 2, 2, 80),     # K = k * I: every channel kept
    ("h256_i96_e16_k2_m2_one", 256, 96, 16, 2, 2, 1),    # K = 1
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_reader_small_shapes(mb, case):
    import torch
    name, H, I, E, k, M, K = case
    say("reader", name)
    wl = synth.small_workload("reader_" + name, H=H, I=I, E=E, k=k, M=M, seed=4100 + H + I + E)
    inp = synth.layer_inputs(wl, 0)
    signs = synth.rotation_signs(wl, 0)
    cfg, dev, layer = make_reader_layer(mb, wl, inp, signs, M, K)
    cs = oracle_tables(inp, signs, range(E), mb, dev, cfg)
    h = inp["h"]
    ids, w = routes_of(mb, layer, h)
    g = inspect(mb, layer, cfg, h, ids, w, K)
    kept = np.stack([check_token(mb, g, t, cfg, h[t], ids[t], w[t], cs, signs, K) for t in range(M)])
    # the step through moe_expert_forward: same kept list, y from the kept channels
    layer.forward(to_dev(h), M, keep=K)
    torch.cuda.synchronize()
    y = layer.y[:M].cpu().numpy()
    np.testing.assert_array_equal(layer.kept.view(-1)[: M * K].view(M, K).cpu().numpy(), kept)
    ref = O.channel_sparse_forward(h, ids, w.astype(np.float64), inp["w_gate"], inp["w_up"], inp["w_down"], kept)
    say("  y vs oracle on the kept list", check_close(y, ref))
    if K == k * I:
        dense = O.dense_forward(h, ids, w.astype(np.float64), inp["w_gate"], inp["w_up"], inp["w_down"])
        say("  all kept vs dense", check_close(y, dense))
    # the one-call decode step: same routing, kept list and y, bit for bit
    y1 = layer.decode_step(to_dev(h), M, keep=K).cpu().numpy()
    np.testing.assert_array_equal(layer.ids[:M].cpu().numpy(), ids)
    np.testing.assert_array_equal(layer.w[:M].cpu().numpy(), w)
    np.testing.assert_array_equal(layer.kept.view(-1)[: M * K].view(M, K).cpu().numpy(), kept)
    np.testing.assert_array_equal(y1, y)
    assert mb.moe_read_device_error(layer.ctx) == 0
    layer.close()


def test_reader_full_size(mb):
    """The sketch reader at H=2048, I=768, E=128, top-8, one token, K=756."""
    import torch
    wl = synth.WORKLOADS["reader_h2048_i768_e128_k8_m1_keep756"]
    say(wl.name, "layer 0 (full size)")
    inp = synth.layer_inputs(wl, 0)
    signs = synth.rotation_signs(wl, 0)
    cfg, dev, layer = make_reader_layer(mb, wl, inp, signs, 1, wl.keep)
    for step in range(2):
        h = synth.hidden(wl, 0, step)
        ids, w = routes_of(mb, layer, h)
        cs = oracle_tables(inp, signs, sorted(set(ids.ravel().tolist())), mb, dev, cfg)
        g = inspect(mb, layer, cfg, h, ids, w, wl.keep)
        kept = check_token(mb, g, 0, cfg, h[0], ids[0], w[0], cs, signs, wl.keep)[None, :]
        y1 = layer.decode_step(to_dev(h), 1, keep=wl.keep).cpu().numpy()
        np.testing.assert_array_equal(layer.ids[:1].cpu().numpy(), ids)
        np.testing.assert_array_equal(layer.kept.view(-1)[: wl.keep].view(1, -1).cpu().numpy(), kept)
        ref = O.channel_sparse_forward(h, ids, w.astype(np.float64), inp["w_gate"], inp["w_up"], inp["w_down"],
                                       kept)
        say("  step", step, "kept per slot", np.bincount(kept[0] // wl.I, minlength=wl.k).tolist(),
            check_close(y1, ref))
        # end to end against the oracle's own reader (fp64 scores) where the kept sets agree
        full = R.reader_step(h[0], ids[0], w[0], inp["w_gate"], inp["w_up"], inp["w_down"], signs, wl.keep)
        if np.array_equal(full["kept"], kept[0]):
            say("  end to end (oracle kept set identical)", check_close(y1[0], full["y"]))
    assert mb.moe_read_device_error(layer.ctx) == 0
    layer.close()


def bf16_ulp(bits: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at each value (2^(exponent - 7))."""
    v = np.abs(O.bf16_to_f64(bits))
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_coefs(b_gpu: np.ndarray, U: np.ndarray, wd_e: np.ndarray) -> float:
    """b = U^T d_j rounded to bf16: the GPU's fp32 sum (H terms) may differ
    from the exact one by gamma_H * sum |U_i d_i|, then each side rounds once
    to bf16 (half an ulp each).  Returns the fraction of differing entries."""
    d = O.bf16_to_f64(wd_e)
    ref = R.recovery_coefs(U, wd_e)
    H = d.shape[1]
    gam = H * U32 / (1 - H * U32)
    bound = gam * (np.abs(d) @ np.abs(U)) + 0.5 * (bf16_ulp(b_gpu) + bf16_ulp(ref)) + 1e-30
    err = np.abs(O.bf16_to_f64(b_gpu) - O.bf16_to_f64(ref))
    assert np.all(err <= bound), "coefficients off by %.2f of their bound" % (err / bound).max()
    return float((b_gpu != ref).mean())


def planted_down(E, I, H, seed, rank=64, decay=0.9, noise=1e-4):
    """bf16 down columns with a planted spectrum: d_j = sum_r decay^r a_jr u_r
    + noise, orthonormal u_r (a seeded QR), so that the top-32 eigenvectors of
    sum d d^T are well separated."""
    U = np.linalg.qr(synth.normal_f32(seed, "planted/u", (H, rank)).astype(np.float64))[0]
    # orthogonal coefficient columns: the planted eigenvalues are exactly
    # 0.0025 N decay^(2r), consecutive ratio decay^2
    a = np.linalg.qr(synth.normal_f32(seed, "planted/a", (E * I, rank)).astype(np.float64))[0] * np.sqrt(E * I)
    n = synth.normal_f32(seed, "planted/n", (E * I, H)).astype(np.float64)
    d = (a * decay ** np.arange(rank)) @ U.T * 0.05 + noise * n
    return R.f64_to_bf16_bits(d).reshape(E, I, H)


def test_recovery_basis_planted_spectrum(mb):
    """moe_recovery_basis against the oracle's symmetric eigensolver on down
    columns with a planted, well-separated spectrum; and the coefficients."""
    import torch
    E, I, H, rank = 8, 128, 256, 32
    wd = planted_down(E, I, H, 4201)
    cfg = mb.make_config(H, I, E, 2)
    dwd = to_dev(wd)
    U = torch.empty((H, rank), dtype=torch.float32, device="cuda")
    mb.moe_recovery_basis(cfg, dwd, rank, 60, U)
    b = torch.empty((E, I, rank), dtype=torch.int16, device="cuda")
    mb.moe_recovery_coefs(cfg, U, rank, dwd, b)
    torch.cuda.synchronize()
    Ug = U.cpu().numpy().astype(np.float64)
    Uo = R.recovery_basis(wd, rank)
    np.testing.assert_allclose(Ug.T @ Ug, np.eye(rank), atol=2e-5)
    err = np.abs(Ug - Uo).max()
    say("  basis max-abs vs eigh %.2e" % err)
    assert err <= 2e-4
    bg = b.cpu().numpy().view(np.uint16)
    frac = max(check_coefs(bg[e], Ug, wd[e]) for e in range(E))
    say("  coefficients differing from the fp64 rounding: %.2e" % frac)


@pytest.mark.parametrize("case", ["small", "full"])
def test_reader_recovery_map(mb, case):
    """y with the recovery map = y without it + U sum over dropped of w p_hat b
    (oracle on the GPU's U, b, estimates and kept list)."""
    import torch
    if case == "small":
        wl = synth.small_workload("reader_rec_small", H=512, I=160, E=16, k=4, M=3, seed=4300)
        K, rank, iters = 120, 16, 30
        inp = synth.layer_inputs(wl, 0)
    else:
        wl = synth.WORKLOADS["reader_h2048_i768_e128_k8_m1_keep756_r32"]
        K, rank, iters = wl.keep, wl.rec_rank, 8
        inp = synth.layer_inputs(wl, 0)
    say("reader recovery", wl.name)
    M = wl.M
    signs = synth.rotation_signs(wl, 0)
    cfg, dev, layer = make_reader_layer(mb, wl, inp, signs, M, K, rank, iters)
    cfg0 = mb.make_config(wl.H, wl.I, wl.E, wl.k, wl.block_b, M, max_keep=K, reader=1)
    layer0 = mb.Layer(cfg0, dev)
    h = inp["h"]
    hd = to_dev(h)
    y = layer.decode_step(hd, M, keep=K).cpu().numpy()
    y0 = layer0.decode_step(hd, M, keep=K).cpu().numpy()
    ids = layer.ids[:M].cpu().numpy().astype(np.int64)
    w = layer.w[:M].cpu().numpy()
    kept = layer.kept.view(-1)[: M * K].view(M, K).cpu().numpy().astype(np.int64)
    np.testing.assert_array_equal(layer0.kept.view(-1)[: M * K].view(M, K).cpu().numpy(), kept)
    g = inspect(mb, layer, cfg, h, ids, w, K)
    Ug = dev["rec_basis"].cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(Ug.T @ Ug, np.eye(rank), atol=2e-5)
    bg = dev["rec_coef"].cpu().numpy().view(np.uint16)
    for t in range(M):
        np.testing.assert_array_equal(g["kept"][t], kept[t])
        est = g["est"][t].astype(np.float64)
        p_hat = O.silu(est[:, 0]) * est[:, 1]
        dropped = np.ones((wl.k, wl.I), bool)
        dropped.reshape(-1)[kept[t]] = False
        rec = R.recovery_term(Ug, bg[ids[t]], w[t].astype(np.float64), p_hat, dropped)
        say("  token", t, "recovery term", check_close(y[t] - y0[t], rec, "recovery"),
            "|rec|/|y| %.3f" % (np.linalg.norm(rec) / np.linalg.norm(y0[t])))
        for e in sorted(set(ids[t].tolist())):
            check_coefs(bg[e], Ug, inp["w_down"][e])
    assert mb.moe_read_device_error(layer.ctx) == 0
    layer.close()
    layer0.close()


def test_reader_bitwise_repeat(mb):
    """Two calls of the reader decode step give bitwise the same outputs."""
    import torch
    wl = synth.WORKLOADS["reader_h2048_i768_e128_k8_m1_keep756_r32"]
    inp = synth.layer_inputs(wl, 0)
    signs = synth.rotation_signs(wl, 0)
    cfg, dev, layer = make_reader_layer(mb, wl, inp, signs, 1, wl.keep, wl.rec_rank, 8)
    hd = to_dev(inp["h"])
    outs = []
    for _ in range(3):
        y = layer.decode_step(hd, 1, keep=wl.keep).clone()
        torch.cuda.synchronize()
        outs.append((y.cpu().numpy(), layer.kept.cpu().numpy().copy()))
    for y, kp in outs[1:]:
        np.testing.assert_array_equal(y.view(np.uint32), outs[0][0].view(np.uint32))
        np.testing.assert_array_equal(kp, outs[0][1])
    layer.close()
