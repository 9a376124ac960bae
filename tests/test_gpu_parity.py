"""GPU parity: the HIP library, called through its C ABI, against the fp64
oracle on the same seeded inputs.

Comparison rules
  * integer outputs (top-k ids, alignment plan, kept channel list) are
    compared bit-exactly: stage-isolated (each stage fed the GPU's previous
    outputs, the oracle stage given the same inputs) always, and end-to-end
    wherever the certified margin of the router decision holds;
  * the GPU top-k must equal the oracle's top-k applied to the GPU's own fp32
    logits (the decision taken in the kernel's precision);
  * floating outputs: rel-L2 <= 1e-3 and max-abs <= 5e-3 * max|y_ref|.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle as O
import synth
from helpers import (certified_tokens, check_close, logit_error_bound, to_dev, upload_layer)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mb():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_bound_routed_amd as m
    return m


def say(*a):
    print(*a, flush=True)


def channel_tables(mb, cfg, dev):
    """Load-time table of the channel-sparse mode, computed on the device:
    the static channel norms."""
    import torch
    norms = torch.empty((cfg.E, cfg.I), dtype=torch.float32, device="cuda")
    mb.moe_channel_norms(cfg, dev["w_gate"], dev["w_up"], dev["w_down"], norms)
    dev["chan_norm"] = norms
    return norms


def make_layer(mb, wl, inp, max_tokens, max_keep=0):
    dev = upload_layer(inp)
    if wl.vq:
        cfg = mb.make_config(wl.H, wl.I, wl.E, wl.k, wl.block_b, max_tokens, mb.MOE_WFORMAT_VQLR, wl.vq_d, wl.vq_K,
                             wl.lr_r, max_keep)
    else:
        cfg = mb.make_config(wl.H, wl.I, wl.E, wl.k, wl.block_b, max_tokens, max_keep=max_keep)
    return mb.Layer(cfg, dev)


def run_step(mb, layer, h_np, keep=0):
    import torch
    M = h_np.shape[0]
    h = to_dev(h_np)
    layer.route(h, M, logits=True)
    if not keep:
        layer.align(M)
    layer.forward(h, M, keep=keep)
    torch.cuda.synchronize()
    out = {
        "ids": layer.ids[:M].cpu().numpy().astype(np.int64),
        "w": layer.w[:M].cpu().numpy(),
        "logits": layer.logits[:M].cpu().numpy(),
        "y": layer.y[:M].cpu().numpy().copy(),
    }
    if not keep:
        cnt = layer.counts.cpu().numpy()
        out["num_blocks"], out["num_padded"] = int(cnt[0]), int(cnt[1])
        out["sorted_routes"] = layer.sorted_routes[: cnt[1]].cpu().numpy().astype(np.int64)
        out["block_expert"] = layer.block_expert[: cnt[0]].cpu().numpy().astype(np.int64)
    else:
        out["kept"] = layer.kept.view(-1)[: M * keep].view(M, keep).cpu().numpy().astype(np.int64)
    out["err"] = mb.moe_read_device_error(layer.ctx)
    return out


def check_router(g, inp, k, H):
    """Ids: exact in the kernel's precision; exact vs fp64 where certified."""
    ref_l = O.router_logits(inp["h"], inp["router_w"], inp.get("router_bias"))
    bound = logit_error_bound(inp["h"], inp["router_w"], H, inp.get("router_bias"))
    err = np.abs(g["logits"].astype(np.float64) - ref_l)
    assert np.all(err <= bound), "logit error above the fp32 bound"
    own = O.topk_select(g["logits"].astype(np.float64), k)
    np.testing.assert_array_equal(g["ids"], own)
    np.testing.assert_allclose(g["w"], O.affinities(g["logits"].astype(np.float64), own), rtol=2e-6, atol=1e-7)
    ok = certified_tokens(ref_l, bound, k)
    ref_ids = O.topk_select(ref_l, k)
    for t in range(len(ok)):
        if ok[t]:
            np.testing.assert_array_equal(g["ids"][t], ref_ids[t])
        else:
            say("  token %d: top-%d not certified by the fp32 bound (ill-posed seed); ids %s vs oracle %s"
                % (t, k, g["ids"][t], ref_ids[t]))
    return ref_l, ok


def check_plan(g, E, b):
    al = O.align_blocks(g["ids"], E, b)
    assert g["num_blocks"] == al["num_blocks"] and g["num_padded"] == al["num_padded"]
    np.testing.assert_array_equal(g["sorted_routes"], al["sorted_routes"])
    np.testing.assert_array_equal(g["block_expert"], al["block_expert"])


# ----------------------------------------------------------------------------

def test_tiny_end_to_end(mb):
    wl = synth.WORKLOADS["tiny_h256_i128_e16_k2"]
    say("tiny_h256_i128_e16_k2 layer 0")
    inp = synth.layer_inputs(wl, 0)
    layer = make_layer(mb, wl, inp, 1)
    g = run_step(mb, layer, inp["h"])
    assert g["err"] == 0
    _, ok = check_router(g, inp, wl.k, wl.H)
    check_plan(g, wl.E, wl.block_b)
    ref = O.dense_forward(inp["h"], g["ids"], g["w"].astype(np.float64), inp["w_gate"], inp["w_up"], inp["w_down"])
    say("  stage-isolated", check_close(g["y"], ref))
    if ok.all():
        full = O.moe_step(inp, wl.k)
        say("  end-to-end", check_close(g["y"], full["y"]))
    layer.close()


def test_dense_b1_full_layer(mb):
    wl = synth.WORKLOADS["dense_h2048_i768_e128_k8_m1"]
    say("dense_h2048_i768_e128_k8_m1 layer 0 (full size)")
    inp = synth.layer_inputs(wl, 0)
    layer = make_layer(mb, wl, inp, 1)
    for step in range(3):  # three independent tokens on the same layer
        h = synth.hidden(wl, 0, step)
        g = run_step(mb, layer, h)
        assert g["err"] == 0
        stage_inp = dict(inp, h=h)
        _, ok = check_router(g, stage_inp, wl.k, wl.H)
        check_plan(g, wl.E, wl.block_b)
        assert g["num_blocks"] == wl.k and g["num_padded"] == 8 * wl.k
        ref = O.dense_forward(h, g["ids"], g["w"].astype(np.float64), inp["w_gate"], inp["w_up"], inp["w_down"])
        say("  step", step, "stage-isolated", check_close(g["y"], ref))
        if ok.all():
            full = O.moe_step(stage_inp, wl.k)
            check_close(g["y"], full["y"])
    layer.close()


def test_aligned_m21_hot_experts_and_plan_injection(mb):
    import torch
    wl = synth.WORKLOADS["aligned_h2048_i768_e128_k8_m21"]
    say("aligned_h2048_i768_e128_k8_m21 layer 0 (full size)")
    inp = synth.layer_inputs(wl, 0)
    layer = make_layer(mb, wl, inp, wl.M)
    g = run_step(mb, layer, inp["h"])
    assert g["err"] == 0
    check_router(g, inp, wl.k, wl.H)
    check_plan(g, wl.E, wl.block_b)
    hot = np.nonzero(inp["router_bias"])[0]
    frac = float(np.isin(g["ids"], hot).mean())
    say("  hot-expert share of routes %.3f, blocks %d, rows %d, distinct experts %d"
        % (frac, g["num_blocks"], g["num_padded"], len(set(g["ids"].ravel()))))
    ref = O.dense_forward(inp["h"], g["ids"], g["w"].astype(np.float64), inp["w_gate"], inp["w_up"], inp["w_down"])
    say("  stage-isolated", check_close(g["y"], ref))

    # plan injection: valid non-canonical plans give bitwise the same y
    M = wl.M
    h = to_dev(inp["h"])
    base = g["y"]
    rows = g["sorted_routes"].copy()
    blocks = g["block_expert"].copy()
    cap = mb.moe_align_capacity(M, wl.k, wl.E, wl.block_b)

    def forward_with(rows_np):
        sr = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
        sr[: rows_np.size] = torch.from_numpy(rows_np.astype(np.int32)).cuda()
        be = torch.from_numpy(blocks.astype(np.int32)).cuda()
        ct = torch.tensor([g["num_blocks"], g["num_padded"]], dtype=torch.int32, device="cuda")
        st, why = mb.moe_validate_plan(g["ids"], M, wl.k, wl.E, wl.block_b, rows_np, blocks,
                                       np.array([g["num_blocks"], g["num_padded"]]))
        assert st == 0, why
        layer.forward(h, M, plan=(sr, be, ct))
        torch.cuda.synchronize()
        assert mb.moe_read_device_error(layer.ctx) == 0
        return layer.y[:M].cpu().numpy()

    # within-block permutation: reverse the valid rows of every block
    perm = rows.copy()
    R = M * wl.k
    for blk in range(g["num_blocks"]):
        seg = perm[blk * 8:(blk + 1) * 8]
        valid = seg[seg != R]
        seg[: valid.size] = valid[::-1]
    assert np.array_equal(forward_with(perm), base)
    # cross-boundary exchange: swap rows across two blocks of one expert
    multi = [e for e in set(blocks.tolist()) if (blocks == e).sum() >= 2]
    assert multi, "expected an expert with more than one block"
    e = multi[0]
    b0 = int(np.nonzero(blocks == e)[0][0])
    swap = rows.copy()
    swap[b0 * 8], swap[(b0 + 1) * 8] = rows[(b0 + 1) * 8], rows[b0 * 8]
    mem_a = O.block_membership(rows, blocks, R)
    mem_b = O.block_membership(swap, blocks, R)
    assert mem_a != mem_b
    assert np.array_equal(forward_with(swap), base)
    layer.close()


def test_chansparse_keep799(mb):
    import torch
    wl = synth.WORKLOADS["chansparse_h2048_i768_e128_k8_m1_keep799"]
    say("chansparse_h2048_i768_e128_k8_m1_keep799 layer 0 (full size)")
    inp = synth.layer_inputs(wl, 0)
    dev = upload_layer(inp)
    cfg = mb.make_config(wl.H, wl.I, wl.E, wl.k, wl.block_b, 1, max_keep=wl.keep)
    norms = channel_tables(mb, cfg, dev)
    torch.cuda.synchronize()
    gn = norms.cpu().numpy()
    ref_n = O.channel_norms(inp["w_gate"], inp["w_up"], inp["w_down"], experts=range(0, wl.E, 9))
    sel = list(range(0, wl.E, 9))
    ulp = np.abs(gn[sel].view(np.int32).astype(np.int64) - ref_n[sel].view(np.int32).astype(np.int64))
    assert ulp.max() <= 1, "norms differ by %d ulp" % ulp.max()
    layer = mb.Layer(cfg, dev)
    for step in range(2):
        h = synth.hidden(wl, 0, step)
        g = run_step(mb, layer, h, keep=wl.keep)
        assert g["err"] == 0
        _, ok = check_router(g, dict(inp, h=h), wl.k, wl.H)
        routed = sorted(set(g["ids"].ravel().tolist()))
        ref_r = O.channel_norms(inp["w_gate"], inp["w_up"], inp["w_down"], experts=routed)
        ulp_r = np.abs(gn[routed].view(np.int32).astype(np.int64) - ref_r[routed].view(np.int32).astype(np.int64))
        assert ulp_r.max() <= 1, "norms of the routed experts differ by %d ulp" % ulp_r.max()
        kept_ref = O.channel_select(g["w"], g["ids"], gn, wl.keep)
        np.testing.assert_array_equal(g["kept"], kept_ref)
        per_slot = np.bincount(g["kept"][0] // wl.I, minlength=wl.k)
        say("  step", step, "kept per slot", per_slot.tolist())
        ref = O.channel_sparse_forward(h, g["ids"], g["w"].astype(np.float64), inp["w_gate"], inp["w_up"],
                                       inp["w_down"], kept_ref)
        say("  stage-isolated", check_close(g["y"], ref))
    layer.close()


def test_channel_exact_selection(mb):
    """The selection against the oracle's top K, with caller affinities that
    are zero, negative or equal, with tied norms (a whole expert at one value,
    pairs of equal channels) and with one expert in two slots."""
    import torch
    wl = synth.small_workload("cs_ranks", H=256, I=96, E=16, k=4, M=3, seed=61)
    M, I, k = wl.M, wl.I, wl.k
    inp = synth.layer_inputs(wl, 0)
    h_np = synth.hidden(wl, 0, 0, M=M)
    h = to_dev(h_np)
    dev = upload_layer(inp)
    cfg = mb.make_config(wl.H, I, wl.E, k, 8, M, max_keep=k * I)
    norms = channel_tables(mb, cfg, dev)
    torch.cuda.synchronize()
    layer = mb.Layer(cfg, dev)
    layer.route(h, M)
    torch.cuda.synchronize()
    ids = layer.ids[:M].cpu().numpy().astype(np.int64)
    w = layer.w[:M].cpu().numpy()

    def select(keep, ids_np=ids, w_np=w):
        layer.kept.fill_(-5)
        layer.forward(h, M, keep=keep, ids=to_dev(ids_np.astype(np.int32)), w=to_dev(w_np.astype(np.float32)))
        torch.cuda.synchronize()
        assert mb.moe_read_device_error(layer.ctx) == 0
        got = layer.kept.view(-1)[: M * keep].view(M, keep).cpu().numpy().astype(np.int64)
        ref = O.channel_select(w_np, ids_np, norms.cpu().numpy(), keep)
        np.testing.assert_array_equal(got, ref)
        return got

    for keep in (1, 37, 200, k * I):
        select(keep)
    kept = select(150)
    ref_y = O.channel_sparse_forward(h_np, ids, w.astype(np.float64), inp["w_gate"], inp["w_up"], inp["w_down"], kept)
    say("  keep 150:", check_close(layer.y[:M].cpu().numpy(), ref_y))

    w2 = w.copy()
    w2[0, 1] = 0.0
    w2[1, 0] = -w2[1, 0]
    w2[2, :] = 0.25
    say("  caller affinities: zero, negative, equal")
    select(150, w_np=w2)
    select(k * I - 3, w_np=w2)

    ids2 = ids.copy()
    ids2[1, 2] = ids2[1, 0]
    w3 = w.copy()
    w3[1, 2] = w3[1, 0]
    say("  one expert in two slots")
    select(150, ids_np=ids2, w_np=w3)

    say("  tied norms")
    tied = norms.clone()
    tied[int(ids[0, 0])] = 0.5
    tied[int(ids[0, 1]), 1::2] = tied[int(ids[0, 1]), 0::2]
    norms.copy_(tied)
    torch.cuda.synchronize()
    for keep in (60, 150, 300):
        select(keep)
    layer.close()


@pytest.mark.parametrize("case", ["n8192_k8", "k1", "k32", "k3_i700"])
def test_channel_selection_shapes(mb, case):
    """The selection at its size limits: k * I = 8192 candidates (every
    thread's eight), one slot, 32 slots, and a channel count that is not a
    multiple of 8 (candidates of one thread in two slots); kept lists against
    the oracle's, y within tolerance, both entry points."""
    import torch
    shape = {"n8192_k8": dict(H=256, I=1024, E=16, k=8, M=2, keep=1100),
             "k1": dict(H=264, I=200, E=8, k=1, M=3, keep=37),
             "k32": dict(H=256, I=256, E=64, k=32, M=2, keep=2000),
             "k3_i700": dict(H=512, I=700, E=24, k=3, M=2, keep=701)}[case]
    keep = shape.pop("keep")
    wl = synth.small_workload("cs_" + case, seed=71, **shape)
    M = wl.M
    say("channel selection shape", case, shape, "keep", keep)
    inp = synth.layer_inputs(wl, 0)
    h_np = synth.hidden(wl, 0, 0, M=M)
    h = to_dev(h_np)
    dev = upload_layer(inp)
    cfg = mb.make_config(wl.H, wl.I, wl.E, wl.k, 8, M, max_keep=keep)
    norms = channel_tables(mb, cfg, dev)
    layer = mb.Layer(cfg, dev)
    layer.decode_step(h, M, keep=keep, logits=True)
    torch.cuda.synchronize()
    assert mb.moe_read_device_error(layer.ctx) == 0
    ids = layer.ids[:M].cpu().numpy().astype(np.int64)
    w = layer.w[:M].cpu().numpy()
    check_router({"ids": ids, "w": w, "logits": layer.logits[:M].cpu().numpy()}, dict(inp, h=h_np), wl.k, wl.H)
    kept = layer.kept.view(-1)[: M * keep].view(M, keep).cpu().numpy().astype(np.int64)
    ref_kept = O.channel_select(w, ids, norms.cpu().numpy(), keep)
    np.testing.assert_array_equal(kept, ref_kept)
    y1 = layer.y[:M].cpu().numpy()
    ref = O.channel_sparse_forward(h_np, ids, w.astype(np.float64), inp["w_gate"], inp["w_up"], inp["w_down"], ref_kept)
    say("  ", check_close(y1, ref))
    # the separate selection entry point on the same routing: same kept list, same y bits
    layer.kept.fill_(-5)
    layer.forward(h, M, keep=keep)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(layer.kept.view(-1)[: M * keep].view(M, keep).cpu().numpy(), ref_kept)
    assert np.array_equal(layer.y[:M].cpu().numpy().view(np.int32), y1.view(np.int32))
    layer.close()


def test_chansparse_all_channels_equals_dense(mb):
    import torch
    wl = synth.small_workload("sparse_all", H=264, I=40, E=16, k=3, M=2, seed=77)
    inp = synth.layer_inputs(wl, 0)
    inp["h"] = synth.hidden(wl, 0, 0, M=2)
    dev = upload_layer(inp)
    cfg = mb.make_config(wl.H, wl.I, wl.E, wl.k, 8, 2, max_keep=wl.k * wl.I)
    norms = channel_tables(mb, cfg, dev)
    layer = mb.Layer(cfg, dev)
    gs = run_step(mb, layer, inp["h"], keep=wl.k * wl.I)
    np.testing.assert_array_equal(gs["kept"], np.tile(np.arange(wl.k * wl.I), (2, 1)))
    gd = run_step(mb, layer, inp["h"])
    ref = O.dense_forward(inp["h"], gd["ids"], gd["w"].astype(np.float64), inp["w_gate"], inp["w_up"], inp["w_down"])
    check_close(gs["y"], ref)
    check_close(gd["y"], ref)
    # K = 1: a single channel
    g1 = run_step(mb, layer, inp["h"], keep=1)
    k1 = O.channel_select(g1["w"], g1["ids"], norms.cpu().numpy(), 1)
    np.testing.assert_array_equal(g1["kept"], k1)
    check_close(g1["y"], O.channel_sparse_forward(inp["h"], g1["ids"], g1["w"].astype(np.float64), inp["w_gate"],
                                                  inp["w_up"], inp["w_down"], k1))
    layer.close()


def test_vqlr_b4(mb):
    wl = synth.WORKLOADS["vqlr_h2048_i768_e128_k8_m4_d8_K256_r64"]
    say("vqlr_h2048_i768_e128_k8_m4_d8_K256_r64 layer 0 (full size)")
    inp = synth.layer_inputs(wl, 0)
    layer = make_layer(mb, wl, inp, wl.M)
    g = run_step(mb, layer, inp["h"])
    assert g["err"] == 0
    check_router(g, inp, wl.k, wl.H)
    check_plan(g, wl.E, wl.block_b)
    say("  distinct experts", len(set(g["ids"].ravel())))
    ref = O.vqlr_forward(inp["h"], g["ids"], g["w"].astype(np.float64), inp, inp["w_down"])
    say("  stage-isolated", check_close(g["y"], ref))
    layer.close()


@pytest.mark.parametrize("name", ["vqlr_h2048_i768_e128_k8_m4_d4_K256_r256", "vqlr_h2048_i768_e128_k8_m4_d2_K256_r8",
                                  "vqlr_h2048_i768_e128_k8_m4_d2_K256_r0"])
def test_vqlr_block_length_full_size(mb, name):
    """The 4-bit-rate block-length sweep at full size (d = 4, r = 256;
    d = 2, r = 8; and the page's VQ-only d = 2, r = 0), stage-isolated against
    the oracle; the one-call decode step gives the same bits."""
    wl = synth.WORKLOADS[name]
    say(name, "layer 0 (full size)")
    inp = synth.layer_inputs(wl, 0)
    layer = make_layer(mb, wl, inp, wl.M)
    g = run_step(mb, layer, inp["h"])
    assert g["err"] == 0
    check_router(g, inp, wl.k, wl.H)
    check_plan(g, wl.E, wl.block_b)
    ref = O.vqlr_forward(inp["h"], g["ids"], g["w"].astype(np.float64), inp, inp["w_down"])
    say("  stage-isolated", check_close(g["y"], ref))
    y2 = layer.decode_step(to_dev(inp["h"]), wl.M).cpu().numpy()
    assert np.array_equal(y2.view(np.int32), g["y"].view(np.int32)), "decode step differs from the separate calls"
    layer.close()


@pytest.mark.parametrize("d,H,I,r,K", [(4, 544, 37, 8, 256), (2, 528, 29, 24, 100), (4, 1024, 64, 136, 17),
                                       (2, 2048, 40, 64, 256), (8, 1088, 33, 72, 200)])
def test_vq_block_lengths_ragged(mb, d, H, I, r, K):
    """Block lengths 2, 4 and 8 on hidden sizes off the lane grid, odd channel
    counts, ranks that are not multiples of 64 and code books smaller than 256,
    against the oracle (three tokens, the split path)."""
    say("vq ragged", dict(d=d, H=H, I=I, r=r, K=K))
    wl = synth.small_workload("vq_d%d_%d_%d" % (d, H, I), H=H, I=I, E=16, k=4, M=3, seed=H + I + d, vq=True,
                              vq_d=d, lr_r=r, vq_K=K)
    inp = synth.layer_inputs(wl, 0)
    inp["h"] = synth.hidden(wl, 0, 0, M=3)
    layer = make_layer(mb, wl, inp, 3)
    g = run_step(mb, layer, inp["h"])
    assert g["err"] == 0
    ref = O.vqlr_forward(inp["h"], g["ids"], g["w"].astype(np.float64), inp, inp["w_down"])
    say("  ", check_close(g["y"], ref))
    layer.close()


@pytest.mark.parametrize("d,H,I,r,M", [(8, 2176, 40, 72, 8), (2, 1088, 33, 8, 4), (4, 1600, 24, 0, 9), (8, 2112, 20, 16, 8)])
def test_vq_slices_taken_in_turn(mb, d, H, I, r, M):
    """More (route, projection, slice) units than gate/up workgroups fit on
    the device at once: each workgroup takes several slices of its route in
    turn (uneven counts, a short last slice), against the oracle; the decode
    step gives the separate calls' bits."""
    import torch
    say("vq slices in turn", dict(d=d, H=H, I=I, r=r, M=M))
    wl = synth.small_workload("vq_turn_d%d_%d_%d" % (d, H, I), H=H, I=I, E=64, k=8, M=M, seed=H + I + 7 * d, vq=True,
                              vq_d=d, lr_r=r, vq_K=256)
    nbk = H // d
    nslice = (nbk + 63) // 64
    assert 2 * M * 8 * nslice > 512 and nbk % 64 != 0, "the case must need several slices per workgroup"
    inp = synth.layer_inputs(wl, 0)
    inp["h"] = synth.hidden(wl, 0, 0, M=M)
    layer = make_layer(mb, wl, inp, M)
    g = run_step(mb, layer, inp["h"])
    assert g["err"] == 0
    ref = O.vqlr_forward(inp["h"], g["ids"], g["w"].astype(np.float64), inp, inp["w_down"])
    say("  ", check_close(g["y"], ref))
    y1 = layer.decode_step(to_dev(inp["h"]), M).cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(y1.view(np.int32), np.asarray(g["y"], np.float32).view(np.int32))
    layer.close()


@pytest.mark.parametrize("name", ["dense_h2048_i768_e128_k8_m8", "dense_h2048_i768_e128_k8_m16",
                                  "vqlr_h2048_i768_e128_k8_m8_d8_K256_r64", "vqlr_h2048_i768_e128_k8_m16_d8_K256_r64",
                                  "vqlr_h2048_i768_e128_k8_m4_d8_K256_r64"])
def test_batch_8_16_full_size(mb, name):
    """Batch 8 and 16 decode at full size (dense bf16 and VQ + low rank): the
    plan, the router (certified ids) and y against the oracle, stage-isolated,
    through the one-call decode step and the separate calls, bit for bit."""
    import torch
    wl = synth.WORKLOADS[name]
    say(name, "layer 0 (full size)")
    inp = synth.layer_inputs(wl, 0)
    layer = make_layer(mb, wl, inp, wl.M)
    g = run_step(mb, layer, inp["h"])
    assert g["err"] == 0
    check_router(g, inp, wl.k, wl.H)
    check_plan(g, wl.E, wl.block_b)
    say("  distinct experts", len(set(g["ids"].ravel())))
    if wl.vq:
        ref = O.vqlr_forward(inp["h"], g["ids"], g["w"].astype(np.float64), inp, inp["w_down"])
    else:
        ref = O.dense_forward(inp["h"], g["ids"], g["w"].astype(np.float64), inp["w_gate"], inp["w_up"],
                              inp["w_down"])
    say("  stage-isolated", check_close(g["y"], ref))
    y1 = layer.decode_step(to_dev(inp["h"]), wl.M).cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(y1.view(np.int32), np.asarray(g["y"], np.float32).view(np.int32))
    layer.close()


@pytest.mark.parametrize("d", [8, 4, 2])
def test_vq_exact_codebook_equals_dense_path(mb, d):
    """With C = 0 the VQ weights are exactly bf16 (a code-book lookup), so the
    GPU VQ path and the GPU dense path on the materialised weights must both
    meet the tolerance against one oracle output."""
    wl = synth.small_workload("vq_exact_d%d" % d, H=512, I=48, E=16, k=4, M=3, seed=91, vq=True, lr_r=16, vq_d=d)
    inp = synth.layer_inputs(wl, 0)
    inp["h"] = synth.hidden(wl, 0, 0, M=3)
    for P in ("gate", "up"):
        inp["lr_coef_" + P][:] = 0
    lv = make_layer(mb, wl, inp, 3)
    gv = run_step(mb, lv, inp["h"])
    dense = {k: v for k, v in inp.items() if not k.startswith(("lr_", "vq_"))}
    dense["w_gate"] = inp["vq_book_gate"][inp["vq_idx_gate"].astype(np.int64)].reshape(wl.E, wl.I, wl.H)
    dense["w_up"] = inp["vq_book_up"][inp["vq_idx_up"].astype(np.int64)].reshape(wl.E, wl.I, wl.H)
    wd = synth.small_workload("vq_exact_dense", H=512, I=48, E=16, k=4, M=3, seed=91)
    ld = make_layer(mb, wd, dense, 3)
    gd = run_step(mb, ld, inp["h"])
    np.testing.assert_array_equal(gv["ids"], gd["ids"])
    ref = O.dense_forward(inp["h"], gd["ids"], gd["w"].astype(np.float64), dense["w_gate"], dense["w_up"],
                          dense["w_down"])
    check_close(gv["y"], ref, "vq")
    check_close(gd["y"], ref, "dense")
    check_close(gv["y"], gd["y"], "vq vs dense")
    lv.close()
    ld.close()


@pytest.mark.parametrize("H,I,E,k,M,b", [
    (520, 37, 24, 3, 5, 8),     # ragged hidden tail (not a multiple of 512) and channel tail
    (8, 1, 8, 1, 1, 8),         # smallest shapes
    (4104, 9, 8, 2, 3, 4),      # > 4096 hidden (16-load register tile), block size 4
    (1024, 70, 64, 6, 12, 16),  # block size 16, several tokens
    (256, 33, 16, 16, 2, 8),    # k = E: every expert routed
])
def test_ragged_shapes(mb, H, I, E, k, M, b):
    say("ragged", dict(H=H, I=I, E=E, k=k, M=M, b=b))
    wl = synth.small_workload("ragged_%d_%d_%d_%d_%d" % (H, I, E, k, M), H=H, I=I, E=E, k=k, M=M, seed=H + I, block_b=b)
    inp = synth.layer_inputs(wl, 0)
    inp["h"] = synth.hidden(wl, 0, 0, M=M)
    layer = make_layer(mb, wl, inp, M)
    g = run_step(mb, layer, inp["h"])
    assert g["err"] == 0
    check_router(g, inp, k, H)
    check_plan(g, E, b)
    ref = O.dense_forward(inp["h"], g["ids"], g["w"].astype(np.float64), inp["w_gate"], inp["w_up"], inp["w_down"])
    check_close(g["y"], ref)
    layer.close()


def test_alignment_randomised_stage_isolated(mb):
    import torch
    rng = np.random.default_rng(2024)
    E, k, b, maxM = 128, 8, 8, 64
    wl = synth.small_workload("align_only", H=64, I=8, E=E, k=k, M=1, seed=3)
    inp = synth.layer_inputs(wl, 0)
    layer = make_layer(mb, wl, inp, maxM)
    cap = mb.moe_align_capacity(maxM, k, E, b)
    n = 0
    for trial in range(120):
        # half the trials with at most 64 routes (one-wave path), half up to 512
        M = int(rng.integers(1, maxM + 1)) if trial % 2 else int(rng.integers(1, 64 // k + 2))
        kind = trial % 5
        if kind == 0:
            ids = np.stack([rng.permutation(E)[:k] for _ in range(M)])
        elif kind == 1:
            p = np.ones(E); p[:4] = 60.0
            ids = np.stack([rng.choice(E, k, replace=False, p=p / p.sum()) for _ in range(M)])
        elif kind == 2:
            ids = np.full((M, k), int(rng.integers(E)))
        elif kind == 3:
            ids = rng.integers(0, E, size=(M, k))
        else:
            ids = rng.integers(-3, E + 3, size=(M, k))
        dids = torch.from_numpy(ids.astype(np.int32)).cuda()
        sr = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
        be = torch.full((cap // b,), -7, dtype=torch.int32, device="cuda")
        ct = torch.zeros(2, dtype=torch.int32, device="cuda")
        mb.moe_align_blocks(layer.ctx, dids, M, sr, be, ct)
        torch.cuda.synchronize()
        flags = mb.moe_read_device_error(layer.ctx)
        al = O.align_blocks(ids, E, b)
        c = ct.cpu().numpy()
        assert int(c[0]) == al["num_blocks"] and int(c[1]) == al["num_padded"]
        np.testing.assert_array_equal(sr[: c[1]].cpu().numpy(), al["sorted_routes"])
        np.testing.assert_array_equal(be[: c[0]].cpu().numpy(), al["block_expert"])
        assert np.all(sr[c[1]:].cpu().numpy() == -7), "wrote past num_padded"
        assert (flags == mb.DEVERR_BAD_ROUTE_ID) == (al["invalid_routes"] > 0)
        n += 1
    say("  %d randomised routings matched" % n)
    layer.close()


@pytest.mark.parametrize("E,k,b,maxM", [(1024, 8, 1, 48), (1024, 6, 3, 40), (8, 8, 64, 16), (8, 8, 1, 512),
                                         (136, 8, 5, 96)])
def test_alignment_extremes(mb, E, k, b, maxM):
    """Alignment at the limits of its bit arithmetic: 10-bit expert ids
    (E = 1024, four experts per thread in the block-count scan), E = 8,
    b = 1 (an expert can need 64 blocks), b = 64, and 4096 routes (64
    chunks).  Bit-exact against the oracle's alignment (page "Route-Block
    Membership Selects Packed-AWQ Arithmetic", Sec. 2.1 and Sec. 5.3)."""
    import torch
    rng = np.random.default_rng(7 + E + b)
    wl = synth.small_workload("align_ext", H=64, I=8, E=E, k=k, M=1, seed=11, block_b=b)
    inp = synth.layer_inputs(wl, 0)
    layer = make_layer(mb, wl, inp, maxM)
    cap = mb.moe_align_capacity(maxM, k, E, b)
    for trial in range(24):
        M = [1, maxM, 64 // k, 64 // k + 1][trial] if trial < 4 else int(rng.integers(1, maxM + 1))
        kind = trial % 4
        if kind == 0:
            ids = rng.integers(0, E, size=(M, k))
        elif kind == 1:
            ids = np.full((M, k), E - 1 - int(rng.integers(min(E, 4))))
        elif kind == 2:
            ids = rng.integers(-2, E + 2, size=(M, k))
        else:
            p = np.ones(E); p[-3:] = 40.0
            ids = rng.choice(E, size=(M, k), p=p / p.sum())
        dids = torch.from_numpy(ids.astype(np.int32)).cuda()
        sr = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
        be = torch.full((max(cap // b, 1),), -7, dtype=torch.int32, device="cuda")
        ct = torch.zeros(2, dtype=torch.int32, device="cuda")
        mb.moe_align_blocks(layer.ctx, dids, M, sr, be, ct)
        torch.cuda.synchronize()
        flags = mb.moe_read_device_error(layer.ctx)
        al = O.align_blocks(ids, E, b)
        c = ct.cpu().numpy()
        assert int(c[0]) == al["num_blocks"] and int(c[1]) == al["num_padded"], (trial, M)
        np.testing.assert_array_equal(sr[: c[1]].cpu().numpy(), al["sorted_routes"])
        np.testing.assert_array_equal(be[: c[0]].cpu().numpy(), al["block_expert"])
        assert np.all(sr[c[1]:].cpu().numpy() == -7), "wrote past num_padded"
        assert (flags == mb.DEVERR_BAD_ROUTE_ID) == (al["invalid_routes"] > 0)
    layer.close()


def test_empty_batch_and_max_tokens(mb):
    import torch
    wl = synth.small_workload("edge", H=256, I=32, E=16, k=2, M=6, seed=5)
    inp = synth.layer_inputs(wl, 0)
    inp["h"] = synth.hidden(wl, 0, 0, M=6)
    layer = make_layer(mb, wl, inp, 6)
    h = to_dev(inp["h"])
    layer.y.fill_(123.0)
    layer.counts.fill_(99)
    layer.route(h, 0)
    layer.align(0)
    layer.forward(h, 0)
    torch.cuda.synchronize()
    assert layer.counts.cpu().tolist() == [0, 0]
    assert torch.all(layer.y == 123.0)
    with pytest.raises(mb.MoeError) as ei:
        layer.route(h, 7)
    assert ei.value.status == mb.MOE_ERR_CAPACITY
    g = run_step(mb, layer, inp["h"])     # M == max_tokens
    ref = O.dense_forward(inp["h"], g["ids"], g["w"].astype(np.float64), inp["w_gate"], inp["w_up"], inp["w_down"])
    check_close(g["y"], ref)
    layer.close()


@pytest.mark.parametrize("name", ["aligned_h2048_i768_e128_k8_m21", "fused_h2048_i768_e16_k8_m1"])
def test_bitwise_reproducible_over_repeated_calls(mb, name):
    import torch
    if name.startswith("fused"):   # one token: the plan-reading fused kernel, then the combine kernel
        wl = synth.small_workload(name, H=2048, I=768, E=16, k=8, M=1, seed=41)
    else:
        wl = synth.WORKLOADS[name]
    say("100 repeated steps,", name)
    inp = synth.layer_inputs(wl, 0)
    layer = make_layer(mb, wl, inp, wl.M)
    h = to_dev(inp["h"])
    first = None
    for i in range(100):
        y = layer.step(h, wl.M).clone()
        outs = (y, layer.ids.clone(), layer.w.clone(), layer.sorted_routes.clone(), layer.counts.clone())
        if first is None:
            first = outs
        else:
            for a, b in zip(first, outs):
                assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                                   b.view(torch.int32) if b.dtype == torch.float32 else b)
    torch.cuda.synchronize()
    assert mb.moe_read_device_error(layer.ctx) == 0
    ref = O.dense_forward(inp["h"], layer.ids[: wl.M].cpu().numpy().astype(np.int64),
                          layer.w[: wl.M].cpu().numpy().astype(np.float64), inp["w_gate"], inp["w_up"], inp["w_down"])
    check_close(first[0][: wl.M].cpu().numpy(), ref)
    layer.close()


# The five workloads of the decode step, run through moe_decode_step (the
# benchmarked call): name -> channel top-K (0 = dense / VQ).
FIVE = [("tiny_h256_i128_e16_k2", 0), ("dense_h2048_i768_e128_k8_m1", 0), ("aligned_h2048_i768_e128_k8_m21", 0),
        ("chansparse_h2048_i768_e128_k8_m1_keep799", 799), ("vqlr_h2048_i768_e128_k8_m4_d8_K256_r64", 0)]


def _decode_outputs(layer, M, keep):
    """Every output of one moe_decode_step as int32 tensors (fp32 by bits)."""
    import torch
    out = [layer.y[:M].view(torch.int32), layer.ids[:M], layer.w[:M].view(torch.int32)]
    if keep:
        out.append(layer.kept.view(-1)[: M * keep])
    else:
        out.append(layer.counts)
        n = int(layer.counts[1].item())
        out.append(layer.sorted_routes[:n])
        out.append(layer.block_expert[: int(layer.counts[0].item())])
    return [t.clone() for t in out]


@pytest.mark.parametrize("name,keep", FIVE)
def test_decode_step_bitwise_reproducible_five_workloads(mb, name, keep):
    """100 calls of the one-call decode step on the same inputs give the same
    bits in every output (y, ids, affinities, plan or kept list)."""
    import torch
    wl = synth.WORKLOADS[name]
    say("100 repeated decode steps,", name)
    inp = synth.layer_inputs(wl, 0)
    if keep:
        dev = upload_layer(inp)
        cfg = mb.make_config(wl.H, wl.I, wl.E, wl.k, wl.block_b, wl.M, max_keep=keep)
        channel_tables(mb, cfg, dev)
        layer = mb.Layer(cfg, dev)
    else:
        layer = make_layer(mb, wl, inp, wl.M)
    h = to_dev(inp["h"])
    first = None
    for i in range(100):
        layer.decode_step(h, wl.M, keep=keep)
        outs = _decode_outputs(layer, wl.M, keep)
        if first is None:
            first = outs
        else:
            for a, b in zip(first, outs):
                assert torch.equal(a, b), "call %d differs" % i
    torch.cuda.synchronize()
    assert mb.moe_read_device_error(layer.ctx) == 0
    layer.close()


_HISTORY_SCRIPT = r"""
import hashlib, sys, numpy as np, torch
sys.path.insert(0, sys.argv[1]); sys.path.insert(0, sys.argv[1] + '/tests')
import synth, memory_bound_routed_amd as mb
from helpers import upload_layer, to_dev
keep_alive = []
if sys.argv[2] == 'H1':   # allocate and keep extra tensors before building the layers
    for n in (3, 777, 12345):
        keep_alive.append(torch.randn(n, device='cuda'))
    torch.cuda.synchronize()
for name, keep in [("tiny_h256_i128_e16_k2", 0), ("dense_h2048_i768_e128_k8_m1", 0),
                   ("aligned_h2048_i768_e128_k8_m21", 0), ("chansparse_h2048_i768_e128_k8_m1_keep799", 799),
                   ("vqlr_h2048_i768_e128_k8_m4_d8_K256_r64", 0)]:
    wl = synth.WORKLOADS[name]
    inp = synth.layer_inputs(wl, 0)
    dev = upload_layer(inp)
    if wl.vq:
        cfg = mb.make_config(wl.H, wl.I, wl.E, wl.k, wl.block_b, wl.M, mb.MOE_WFORMAT_VQLR, wl.vq_d, wl.vq_K, wl.lr_r)
    else:
        cfg = mb.make_config(wl.H, wl.I, wl.E, wl.k, wl.block_b, wl.M, max_keep=keep)
    if keep:
        dev['chan_norm'] = torch.empty((wl.E, wl.I), dtype=torch.float32, device='cuda')
        mb.moe_channel_norms(cfg, dev['w_gate'], dev['w_up'], dev['w_down'], dev['chan_norm'])
    layer = mb.Layer(cfg, dev)
    y = layer.decode_step(to_dev(inp['h']), wl.M, keep=keep)
    torch.cuda.synchronize()
    hsh = hashlib.sha256(y.cpu().numpy().tobytes())
    hsh.update(layer.ids[:wl.M].cpu().numpy().tobytes())
    if keep:
        hsh.update(layer.kept.view(-1)[:wl.M * keep].cpu().numpy().tobytes())
    print(name, hsh.hexdigest(), flush=True)
    layer.close()
    del dev, layer
"""


def test_bitwise_identical_across_process_histories(mb):
    """Two fresh processes with different allocation histories give the same
    bits for the decode step of all five workloads."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    hashes = {}
    for hist in ("H0", "H1"):
        say("fresh process, history", hist)
        r = subprocess.run([sys.executable, "-c", _HISTORY_SCRIPT, root, hist], capture_output=True, text=True,
                           timeout=300)
        assert r.returncode == 0, r.stderr[-2000:]
        lines = [ln.split() for ln in r.stdout.strip().splitlines() if len(ln.split()) == 2]
        hashes[hist] = dict(lines)
    say("  ", hashes["H0"])
    assert len(hashes["H0"]) == 5
    assert hashes["H0"] == hashes["H1"]


def test_device_error_flags_on_invalid_ids(mb):
    import torch
    wl = synth.small_workload("bad_ids", H=256, I=16, E=16, k=2, M=3, seed=8)
    inp = synth.layer_inputs(wl, 0)
    inp["h"] = synth.hidden(wl, 0, 0, M=3)
    layer = make_layer(mb, wl, inp, 3)
    ids = torch.tensor([[1, 99], [-1, 2], [3, 4]], dtype=torch.int32, device="cuda")
    w = torch.full((3, 2), 0.5, dtype=torch.float32, device="cuda")
    layer.align(3, ids=ids)
    h = to_dev(inp["h"])
    layer.forward(h, 3, ids=ids, w=w)
    torch.cuda.synchronize()
    flags = mb.moe_read_device_error(layer.ctx)
    assert flags & mb.DEVERR_BAD_ROUTE_ID
    idn = ids.cpu().numpy().astype(np.int64)
    ref = O.dense_forward(inp["h"], idn, w.cpu().numpy().astype(np.float64), inp["w_gate"], inp["w_up"],
                          inp["w_down"])
    check_close(layer.y[:3].cpu().numpy(), ref)
    assert mb.moe_read_device_error(layer.ctx) == 0  # cleared
    layer.close()


@pytest.mark.parametrize("name", ["tiny_h256_i128_e16_k2", "dense_h2048_i768_e128_k8_m1",
                                  "aligned_h2048_i768_e128_k8_m21", "small_m3_e128_k8", "small_m8_e64_k8"])
def test_route_align_matches_separate_calls(mb, name):
    import torch
    if name.startswith("small_m3"):      # 24 routes of one 4-token pass: aligned from the selections in LDS
        wl = synth.small_workload(name, H=256, I=8, E=128, k=8, M=3, seed=31)
    elif name.startswith("small_m8"):    # 64 routes over two passes: aligned from the written ids
        wl = synth.small_workload(name, H=512, I=8, E=64, k=8, M=8, seed=32)
    else:
        wl = synth.WORKLOADS[name]
    say("route+align in one launch vs two launches:", name)
    inp = synth.layer_inputs(wl, 0, experts=[])   # router only: no expert weights needed
    inp["w_gate"] = inp["w_up"] = inp["w_down"] = np.zeros((wl.E, 1, wl.H), np.uint16)
    dev = upload_layer(inp)
    cfg = mb.make_config(wl.H, 1, wl.E, wl.k, wl.block_b, wl.M)
    layer = mb.Layer(cfg, dev)
    h = to_dev(inp["h"])
    layer.route(h, wl.M, logits=True)
    layer.align(wl.M)
    torch.cuda.synchronize()
    a = [t.clone() for t in (layer.ids, layer.w, layer.logits, layer.sorted_routes, layer.block_expert, layer.counts)]
    for t in (layer.ids, layer.w, layer.logits, layer.sorted_routes, layer.block_expert, layer.counts):
        t.fill_(-3)
    layer.route_align(h, wl.M, logits=True)
    torch.cuda.synchronize()
    b = (layer.ids, layer.w, layer.logits, layer.sorted_routes, layer.block_expert, layer.counts)
    n = int(a[5][1])
    for x, y, what in zip(a, b, ("ids", "w", "logits", "rows", "blocks", "counts")):
        if what == "rows":
            x, y = x[:n], y[:n]
        if what == "blocks":
            x, y = x[: n // wl.block_b], y[: n // wl.block_b]
        assert torch.equal(x.view(torch.int32), y.view(torch.int32)), what
    assert mb.moe_read_device_error(layer.ctx) == 0
    layer.close()


@pytest.mark.parametrize("ids,b", [
    ([[3, 3, 5, 3]], 8),          # one token routed three times to expert 3: extra routes in one block
    ([[6, 6, 6, 1, 6, 2]], 2),    # block size 2: expert 6 spans two blocks of the run
])
def test_fused_single_token_with_repeated_experts(mb, ids, b):
    import torch
    ids = np.array(ids)
    k = ids.shape[1]
    wl = synth.small_workload("repeat_%d_%d" % (k, b), H=2048, I=64, E=8, k=k, M=1, seed=31, block_b=b)
    inp = synth.layer_inputs(wl, 0)
    inp["h"] = synth.hidden(wl, 0, 0, M=1)
    layer = make_layer(mb, wl, inp, 1)
    dids = torch.from_numpy(ids.astype(np.int32)).cuda()
    w = np.linspace(0.4, 0.1, k).astype(np.float32).reshape(1, k)
    dw = torch.from_numpy(w).cuda()
    layer.align(1, ids=dids)
    layer.forward(to_dev(inp["h"]), 1, ids=dids, w=dw)
    torch.cuda.synchronize()
    assert mb.moe_read_device_error(layer.ctx) == 0
    ref = O.dense_forward(inp["h"], ids, w.astype(np.float64), inp["w_gate"], inp["w_up"], inp["w_down"])
    check_close(layer.y[:1].cpu().numpy(), ref)
    layer.close()


@pytest.mark.parametrize("b,hot", [
    (16, 10),  # one block holds 10 routes of one expert: two 8-route passes of the down kernel, three gate/up groups
    (8, 12),   # an expert with 12 routes spans two blocks of its run
    (4, 7),    # block size 4: a run of two blocks, the second partly padded
])
def test_split_path_forced_hot_expert(mb, b, hot):
    """Several tokens with forced routes: expert 3 takes `hot` routes, the
    rest are spread; checked against the oracle on the same ids and weights."""
    import torch
    M, k, E = 12, 2, 16
    ids = np.zeros((M, k), dtype=np.int64)
    n = 0
    for t in range(M):
        for s in range(k):
            ids[t, s] = 3 if n < hot and s == 0 else (5 + (t * k + s) % 9)
            n += 1 if s == 0 else 0
    assert all(len(set(r)) == k for r in ids) and (ids == 3).sum() == hot
    wl = synth.small_workload("hot_%d_%d" % (b, hot), H=1032, I=72, E=E, k=k, M=M, seed=101 + b, block_b=b)
    say("split forced", dict(b=b, hot=hot, H=wl.H, I=wl.I))
    inp = synth.layer_inputs(wl, 0)
    inp["h"] = synth.hidden(wl, 0, 0, M=M)
    layer = make_layer(mb, wl, inp, M)
    dids = torch.from_numpy(ids.astype(np.int32)).cuda()
    w = np.tile(np.array([[0.7, 0.3]], dtype=np.float32), (M, 1))
    dw = torch.from_numpy(w).cuda()
    layer.align(M, ids=dids)
    layer.forward(to_dev(inp["h"]), M, ids=dids, w=dw)
    torch.cuda.synchronize()
    assert mb.moe_read_device_error(layer.ctx) == 0
    ref = O.dense_forward(inp["h"], ids, w.astype(np.float64), inp["w_gate"], inp["w_up"], inp["w_down"])
    check_close(layer.y[:M].cpu().numpy(), ref)
    layer.close()


@pytest.mark.parametrize("b,hot", [(16, 10), (8, 12), (4, 7)])
def test_split_down_matrix_cores_forced_hot_expert(mb, b, hot):
    """The split schedule's 256-column down launch (bf16 MFMA tiles of 32
    channels, s split into hi and lo bf16 parts) with forced multi-route
    experts: full 8-route passes, a ragged last channel tile (I = 200) and a
    partial last column block (H = 2056); checked against the oracle."""
    import torch
    M, k, E, H, I = 40, 2, 64, 2056, 200
    ids = np.zeros((M, k), dtype=np.int64)
    for t in range(M):
        ids[t, 0] = 3 if t < hot else 5 + (2 * t) % 9
        ids[t, 1] = 5 + (2 * t + 1) % 9
    assert all(len(set(r)) == k for r in ids) and (ids == 3).sum() == hot
    cap = mb.moe_align_capacity(M, k, E, b)
    assert (cap // b) * ((H + 255) // 256) >= 512, "shape must take the 256-column launch"
    wl = synth.small_workload("mfma_hot_%d_%d" % (b, hot), H=H, I=I, E=E, k=k, M=M, seed=131 + b, block_b=b)
    say("split down matrix cores", dict(b=b, hot=hot, H=H, I=I, E=E, M=M))
    inp = synth.layer_inputs(wl, 0)
    inp["h"] = synth.hidden(wl, 0, 0, M=M)
    layer = make_layer(mb, wl, inp, M)
    dids = torch.from_numpy(ids.astype(np.int32)).cuda()
    w = np.tile(np.array([[0.6, 0.4]], dtype=np.float32), (M, 1))
    dw = torch.from_numpy(w).cuda()
    layer.align(M, ids=dids)
    layer.forward(to_dev(inp["h"]), M, ids=dids, w=dw)
    torch.cuda.synchronize()
    assert mb.moe_read_device_error(layer.ctx) == 0
    ref = O.dense_forward(inp["h"], ids, w.astype(np.float64), inp["w_gate"], inp["w_up"], inp["w_down"])
    check_close(layer.y[:M].cpu().numpy(), ref)
    layer.close()


@pytest.mark.parametrize("b", [8, 4])
def test_vq_forced_multi_route_experts(mb, b):
    """VQ + low-rank path with nine experts routed more than once (expert 3
    six times, eight others twice): more such runs than the kernel shares
    with extra workgroups, so shared and unshared runs are both checked."""
    import torch
    M, k = 12, 2
    ids = np.array([[3, 5 + t] for t in range(6)] + [[5 + (t - 6), 12 + (t % 4)] for t in range(6, 12)],
                   dtype=np.int64)
    assert all(len(set(r)) == k for r in ids)
    wl = synth.small_workload("vq_multi_%d" % b, H=1024, I=40, E=16, k=k, M=M, seed=131 + b, vq=True, lr_r=16,
                              block_b=b)
    say("vq forced", dict(b=b))
    inp = synth.layer_inputs(wl, 0)
    inp["h"] = synth.hidden(wl, 0, 0, M=M)
    layer = make_layer(mb, wl, inp, M)
    dids = torch.from_numpy(ids.astype(np.int32)).cuda()
    w = np.tile(np.array([[0.6, 0.4]], dtype=np.float32), (M, 1))
    dw = torch.from_numpy(w).cuda()
    layer.align(M, ids=dids)
    layer.forward(to_dev(inp["h"]), M, ids=dids, w=dw)
    torch.cuda.synchronize()
    assert mb.moe_read_device_error(layer.ctx) == 0
    ref = O.vqlr_forward(inp["h"], ids, w.astype(np.float64), inp, inp["w_down"])
    check_close(layer.y[:M].cpu().numpy(), ref)
    layer.close()


def _step_outputs(layer, M):
    n = int(layer.counts[1]) if M else 0
    return {"ids": layer.ids[:M].clone(), "w": layer.w[:M].clone(), "logits": layer.logits[:M].clone(),
            "rows": layer.sorted_routes[:n].clone(), "blocks": layer.block_expert[: n // layer.cfg.block_b].clone(),
            "counts": layer.counts.clone(), "y": layer.y[:M].clone()}


@pytest.mark.parametrize("case", [
    "tiny",          # H=256: one router slice, E=16 (16-expert column groups)
    "full",          # the batch-1 Qwen3-30B-A3B-shaped layer, two tokens
    "ragged",        # H=1000 (hidden tail), I=72, E=24, k=3, block size 4
    "e512_bias",     # E=512 (one rank part per thread), additive router bias on 4 experts
    "h4096_e256",    # 16 router slices, 16-load register tile, E=256 (two rank parts)
    "k_eq_e",        # k = E = 16: every expert selected
    "ties",          # zero router weights + tied bias: the order is decided by the expert ids
    "m3_fallback",   # three tokens: the separate launches
    "i256_one_chunk",     # I=256, top-8: one 8-channel chunk per fused workgroup (256 workgroups)
    "i280_three_chunks",  # I=280: three chunks per workgroup, the last range 16 channels
])
def test_decode_step_matches_separate_calls(mb, case):
    """moe_decode_step gives bit for bit the outputs of moe_route_align +
    moe_expert_forward (ids, affinities, logits, plan, y), and both match the
    oracle."""
    import torch
    specs = {
        "tiny": dict(wl=synth.WORKLOADS["tiny_h256_i128_e16_k2"]),
        "full": dict(wl=synth.WORKLOADS["dense_h2048_i768_e128_k8_m1"], steps=2),
        "ragged": dict(wl=synth.small_workload("ds_ragged", H=1000, I=72, E=24, k=3, M=1, seed=41, block_b=4)),
        "e512_bias": dict(wl=synth.small_workload("ds_e512", H=512, I=40, E=512, k=8, M=1, seed=42, hot_experts=4)),
        "h4096_e256": dict(wl=synth.small_workload("ds_h4096", H=4096, I=24, E=256, k=5, M=1, seed=43)),
        "k_eq_e": dict(wl=synth.small_workload("ds_keqe", H=256, I=16, E=16, k=16, M=1, seed=44)),
        "ties": dict(wl=synth.small_workload("ds_ties", H=256, I=16, E=16, k=4, M=1, seed=45)),
        "m3_fallback": dict(wl=synth.small_workload("ds_m3", H=256, I=24, E=32, k=4, M=3, seed=46)),
        # the edge of the narrow-expert tiling: k * ceil(I / 8) = 256 takes one
        # 8-channel chunk per workgroup, 280 channels three (ragged last range)
        "i256_one_chunk": dict(wl=synth.small_workload("ds_i256", H=2048, I=256, E=128, k=8, M=1, seed=47)),
        "i280_three_chunks": dict(wl=synth.small_workload("ds_i280", H=2048, I=280, E=128, k=8, M=1, seed=48)),
    }[case]
    wl = specs["wl"]
    say("decode step vs separate calls:", case, dict(H=wl.H, I=wl.I, E=wl.E, k=wl.k, M=wl.M, b=wl.block_b))
    inp = synth.layer_inputs(wl, 0)
    if case == "ties":
        inp["router_w"] = np.zeros_like(inp["router_w"])
        inp["router_bias"] = np.array([0.5, 1.0, 1.0, 0.25, 1.0, 0.5] + [0.25] * 10, np.float32)
    layer = make_layer(mb, wl, inp, wl.M)
    for step in range(specs.get("steps", 1)):
        h_np = synth.hidden(wl, 0, step, M=wl.M)
        h = to_dev(h_np)
        layer.route_align(h, wl.M, logits=True)
        layer.forward(h, wl.M)
        torch.cuda.synchronize()
        a = _step_outputs(layer, wl.M)
        for t in (layer.ids, layer.w, layer.logits, layer.sorted_routes, layer.block_expert, layer.counts, layer.y):
            t.fill_(-3)
        layer.decode_step(h, wl.M, logits=True)
        torch.cuda.synchronize()
        b = _step_outputs(layer, wl.M)
        for what in a:
            assert torch.equal(a[what].view(torch.int32), b[what].view(torch.int32)), what
        assert mb.moe_read_device_error(layer.ctx) == 0
        g = {"ids": b["ids"].cpu().numpy().astype(np.int64), "w": b["w"].cpu().numpy(),
             "logits": b["logits"].cpu().numpy(), "num_blocks": int(b["counts"][0]),
             "num_padded": int(b["counts"][1]), "sorted_routes": b["rows"].cpu().numpy().astype(np.int64),
             "block_expert": b["blocks"].cpu().numpy().astype(np.int64)}
        stage_inp = dict(inp, h=h_np)
        check_router(g, stage_inp, wl.k, wl.H)
        if case == "ties":
            np.testing.assert_array_equal(g["ids"], [[1, 2, 4, 0]])
        check_plan(g, wl.E, wl.block_b)
        ref = O.dense_forward(h_np, g["ids"], g["w"].astype(np.float64), inp["w_gate"], inp["w_up"], inp["w_down"])
        say("  step", step, check_close(b["y"].cpu().numpy(), ref))
    layer.close()


@pytest.mark.parametrize("case", [
    "m4",         # the 4-token VQ + low-rank step (d 8, K 256, r 64): 32 routes, one-wave alignment
    "m16",        # 16 tokens: 128 routes, the workgroup alignment; four router token groups
    "r0_d2",      # the VQ-only point (no z tiles, no coefficient stream)
    "ragged",     # H 544, I 37, d 4, K 100, r 8, E 40, k 3, block size 4, 5 tokens, router bias
    "k_eq_e",     # k = E = 16 with three tokens: every expert routed by every token
    "e264",       # E > 256: the routing launch + separate launches
])
def test_vq_decode_step_matches_separate_calls(mb, case):
    """The VQ decode step, whose gate/up workgroups route their tokens from
    the router's slice partials and whose down launch (up to 64 routes) or
    finish launch (more) aligns the routes,
    gives bit for bit the ids, affinities, logits, plan and y of
    moe_route_align + moe_expert_forward; y matches the oracle."""
    import torch
    sw = synth.small_workload
    wl = {
        "m4": synth.WORKLOADS["vqlr_h2048_i768_e128_k8_m4_d8_K256_r64"],
        "m16": synth.WORKLOADS["vqlr_h2048_i768_e128_k8_m16_d8_K256_r64"],
        "r0_d2": synth.WORKLOADS["vqlr_h2048_i768_e128_k8_m4_d2_K256_r0"],
        "ragged": sw("vqds_ragged", H=544, I=37, E=40, k=3, M=5, seed=61, block_b=4, vq=True, vq_d=4, vq_K=100,
                     lr_r=8, hot_experts=3),
        "k_eq_e": sw("vqds_keqe", H=256, I=24, E=16, k=16, M=3, seed=62, vq=True, vq_d=8, vq_K=64, lr_r=16),
        "e264": sw("vqds_e264", H=512, I=40, E=264, k=4, M=2, seed=63, vq=True, vq_d=8, vq_K=256, lr_r=8),
    }[case]
    say("VQ decode step vs separate calls:", case, dict(H=wl.H, I=wl.I, E=wl.E, k=wl.k, M=wl.M, d=wl.vq_d,
                                                       r=wl.lr_r, b=wl.block_b))
    inp = synth.layer_inputs(wl, 0)
    layer = make_layer(mb, wl, inp, wl.M)
    h_np = inp["h"]
    h = to_dev(h_np)
    layer.route_align(h, wl.M, logits=True)
    layer.forward(h, wl.M)
    torch.cuda.synchronize()
    a = _step_outputs(layer, wl.M)
    for t in (layer.ids, layer.w, layer.logits, layer.sorted_routes, layer.block_expert, layer.counts, layer.y):
        t.fill_(-3)
    layer.decode_step(h, wl.M, logits=True)
    torch.cuda.synchronize()
    b = _step_outputs(layer, wl.M)
    for what in a:
        assert torch.equal(a[what].view(torch.int32), b[what].view(torch.int32)), what
    assert mb.moe_read_device_error(layer.ctx) == 0
    g = {"ids": b["ids"].cpu().numpy().astype(np.int64), "w": b["w"].cpu().numpy(),
         "logits": b["logits"].cpu().numpy(), "num_blocks": int(b["counts"][0]),
         "num_padded": int(b["counts"][1]), "sorted_routes": b["rows"].cpu().numpy().astype(np.int64),
         "block_expert": b["blocks"].cpu().numpy().astype(np.int64)}
    check_router(g, inp, wl.k, wl.H)
    check_plan(g, wl.E, wl.block_b)
    ref = O.vqlr_forward(h_np, g["ids"], g["w"].astype(np.float64), inp, inp["w_down"])
    say("  decode step", check_close(b["y"].cpu().numpy(), ref))
    layer.close()


@pytest.mark.parametrize("E,k,M", [
    (256, 32, 4),   # k' = 32 lane groups: most tokens have more than 64 keys above the threshold (all-keys count)
    (256, 2, 4),    # four keys per lane, few candidates
    (64, 16, 3),    # one key per lane
    (8, 8, 2),      # k = E: every key selected, lanes past E hold no expert
    (1024, 4, 1),   # E > 256: the count of every key
])
def test_router_threshold_and_count_paths(mb, E, k, M):
    """The router's top-k (one wave per token from the keys above a
    threshold, or every key counted) and the one-wave alignment: ids exact
    for the kernel's own fp32 logits, affinities and plan as the oracle's."""
    import torch
    wl = synth.small_workload("router_%d_%d_%d" % (E, k, M), H=512, I=1, E=E, k=k, M=M, seed=E + k + M)
    say("router paths", dict(E=E, k=k, M=M))
    inp = synth.layer_inputs(wl, 0, experts=[])
    inp["h"] = synth.hidden(wl, 0, 0, M=M)
    inp["w_gate"] = inp["w_up"] = inp["w_down"] = np.zeros((E, 1, wl.H), np.uint16)
    layer = mb.Layer(mb.make_config(wl.H, 1, E, k, wl.block_b, M), upload_layer(inp))
    h = to_dev(inp["h"])
    for call in ("route", "route_align"):
        for t in (layer.ids, layer.w, layer.logits, layer.sorted_routes, layer.block_expert, layer.counts):
            t.fill_(-3)
        if call == "route":
            layer.route(h, M, logits=True)
            layer.align(M)
        else:
            layer.route_align(h, M, logits=True)
        torch.cuda.synchronize()
        cnt = layer.counts.cpu().numpy()
        g = {"ids": layer.ids[:M].cpu().numpy().astype(np.int64), "w": layer.w[:M].cpu().numpy(),
             "logits": layer.logits[:M].cpu().numpy(), "num_blocks": int(cnt[0]), "num_padded": int(cnt[1]),
             "sorted_routes": layer.sorted_routes[: cnt[1]].cpu().numpy().astype(np.int64),
             "block_expert": layer.block_expert[: cnt[0]].cpu().numpy().astype(np.int64)}
        check_router(g, inp, k, wl.H)
        check_plan(g, E, wl.block_b)
    assert mb.moe_read_device_error(layer.ctx) == 0
    layer.close()


@pytest.mark.parametrize("case", [
    "full",      # the batch-1 channel-sparse workload: top 799 of 8 x 768 candidates
    "m3",        # three tokens (one selection workgroup each, partials of a 4-token router group)
    "e512",      # E > 256: the top-k counts every key
])
def test_decode_step_channel_sparse(mb, case):
    """moe_decode_step with keep > 0 (router partials, then a selection whose
    workgroups route their tokens) gives bit for bit the ids, affinities,
    logits, kept list and y of moe_route_topk + moe_expert_forward, and the
    oracle's selection and output."""
    import torch
    if case == "full":
        wl = synth.WORKLOADS["chansparse_h2048_i768_e128_k8_m1_keep799"]
        keep = wl.keep
    elif case == "m3":
        wl = synth.small_workload("cs_m3", H=512, I=40, E=64, k=4, M=3, seed=51)
        keep = 50
    else:
        wl = synth.small_workload("cs_e512", H=256, I=24, E=512, k=6, M=2, seed=52, hot_experts=4)
        keep = 31
    M = wl.M
    say("channel-sparse decode step vs separate calls:", case, dict(H=wl.H, I=wl.I, E=wl.E, k=wl.k, M=M, keep=keep))
    inp = synth.layer_inputs(wl, 0)
    dev = upload_layer(inp)
    cfg = mb.make_config(wl.H, wl.I, wl.E, wl.k, wl.block_b, M, max_keep=keep)
    norms = channel_tables(mb, cfg, dev)
    layer = mb.Layer(cfg, dev)
    h_np = synth.hidden(wl, 0, 1, M=M)
    h = to_dev(h_np)
    outs = []
    for one_call in (False, True):
        for t in (layer.ids, layer.w, layer.logits, layer.kept, layer.y):
            t.fill_(-3)
        if one_call:
            layer.decode_step(h, M, keep=keep, logits=True)
        else:
            layer.route(h, M, logits=True)
            layer.forward(h, M, keep=keep)
        torch.cuda.synchronize()
        outs.append([layer.ids[:M].clone(), layer.w[:M].clone(), layer.logits[:M].clone(),
                     layer.kept.view(-1)[: M * keep].clone(), layer.y[:M].clone()])
    for a, b, what in zip(outs[0], outs[1], ("ids", "w", "logits", "kept", "y")):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), what
    assert mb.moe_read_device_error(layer.ctx) == 0
    g = {"ids": outs[1][0].cpu().numpy().astype(np.int64), "w": outs[1][1].cpu().numpy(),
         "logits": outs[1][2].cpu().numpy()}
    check_router(g, dict(inp, h=h_np), wl.k, wl.H)
    kept = outs[1][3].view(M, keep).cpu().numpy().astype(np.int64)
    kept_ref = O.channel_select(g["w"], g["ids"], norms.cpu().numpy(), keep)
    np.testing.assert_array_equal(kept, kept_ref)
    ref = O.channel_sparse_forward(h_np, g["ids"], g["w"].astype(np.float64), inp["w_gate"], inp["w_up"],
                                   inp["w_down"], kept_ref)
    say("  ", check_close(outs[1][4].cpu().numpy(), ref))
    layer.close()
