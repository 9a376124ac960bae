"""One GPU's share of the batch-1 dense layer under channel sharding.

With G GPUs, GPU g would own channels 96 g .. 96 g + 95 of every expert
(its gate and up rows and the matching down rows), replicate the router and
the routing, and write a partial y; one exchange would add the G partials in
GPU order.  Only one GPU is used here: the G shards run one after another on
it, each as its own layer with I = 768 / G, through moe_decode_step (the
benchmarked call).  Checked: every shard routes exactly as the full layer
(same router, same bits), every shard's y is the oracle's for its channels,
and the shards' partials added in shard order give the full layer's y
(page "Channel Selection for Mixture-of-Experts Decoding Needs No
Calibration Data", "Background: Channels and Retention Rules": an expert's
output is a sum over its channels, so the routed output splits over any
partition of the channels).
"""
import numpy as np
import pytest

import oracle as O
import synth
from helpers import check_close, to_dev, upload_layer

pytestmark = pytest.mark.gpu

G = 8


@pytest.fixture(scope="module")
def mb():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_bound_routed_amd as m
    return m


def say(*a):
    print(*a, flush=True)


def _decode(mb, wl_like, inp, h):
    """One moe_decode_step on a dense layer; y, ids, weights and the error word."""
    import torch
    H, I = inp["w_gate"].shape[2], inp["w_gate"].shape[1]
    cfg = mb.make_config(H, I, wl_like.E, wl_like.k, wl_like.block_b, 1)
    layer = mb.Layer(cfg, upload_layer(inp))
    y = layer.decode_step(to_dev(h), 1).cpu().numpy().copy()
    torch.cuda.synchronize()
    out = {"y": y, "ids": layer.ids[:1].cpu().numpy().astype(np.int64), "w": layer.w[:1].cpu().numpy(),
           "err": mb.moe_read_device_error(layer.ctx)}
    layer.close()
    return out


def test_shard_workload_layer0(mb):
    """The bench's shard workload (layer 0) against the oracle."""
    wl = synth.WORKLOADS["shard8_h2048_i96_e128_k8_m1"]
    full = synth.WORKLOADS["dense_h2048_i768_e128_k8_m1"]
    say("shard8_h2048_i96_e128_k8_m1 layer 0")
    inp = synth.layer_inputs(wl, 0)
    np.testing.assert_array_equal(inp["router_w"], synth.router_weight(full, 0))  # the full layer's router
    g = _decode(mb, wl, inp, inp["h"])
    assert g["err"] == 0
    ref = O.dense_forward(inp["h"], g["ids"], g["w"].astype(np.float64), inp["w_gate"], inp["w_up"], inp["w_down"])
    say("  stage-isolated", check_close(g["y"], ref))


def test_channel_shards_add_up_to_the_full_layer(mb):
    """The full batch-1 layer and its G channel shards, all on one GPU."""
    wl = synth.WORKLOADS["dense_h2048_i768_e128_k8_m1"]
    assert wl.I % G == 0
    n = wl.I // G
    say("dense_h2048_i768_e128_k8_m1 layer 0: full layer and %d channel shards of %d" % (G, n))
    for step in range(2):
        h = synth.hidden(wl, 0, step)
        # only the routed experts' weights are drawn
        ids0 = O.topk_select(O.router_logits(h, synth.router_weight(wl, 0), None), wl.k)
        inp = synth.layer_inputs(wl, 0, experts=ids0.ravel())
        inp["h"] = h
        f = _decode(mb, wl, inp, h)
        assert f["err"] == 0
        parts = []
        for g in range(G):
            sh = dict(inp)
            for key in ("w_gate", "w_up", "w_down"):
                sh[key] = np.ascontiguousarray(inp[key][:, g * n:(g + 1) * n, :])
            s = _decode(mb, wl, sh, h)
            assert s["err"] == 0
            # the routing is replicated: the same bits on every shard
            np.testing.assert_array_equal(s["ids"], f["ids"])
            np.testing.assert_array_equal(s["w"].view(np.int32), f["w"].view(np.int32))
            ref = O.dense_forward(h, s["ids"], s["w"].astype(np.float64), sh["w_gate"], sh["w_up"], sh["w_down"])
            check_close(s["y"], ref, "shard %d y" % g)
            parts.append(s["y"].astype(np.float64))
        total = parts[0]
        for g in range(1, G):  # the exchange's fixed order
            total = total + parts[g]
        ref = O.dense_forward(h, f["ids"], f["w"].astype(np.float64), inp["w_gate"], inp["w_up"], inp["w_down"])
        say("  step", step, "sum of shards vs oracle", check_close(total, ref),
            "full layer vs oracle", check_close(f["y"], ref))
