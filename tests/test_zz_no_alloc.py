"""moe_decode_step_noalloc (no context, no allocation; its workspace is an
array inside the library) against moe_decode_step on a context, through the
C ABI: the same kernels run on another workspace, so every output must be
bitwise the same.  Two calls in a row on one layer, the second with fewer
tokens, so the second call runs on what the first left in the shared array."""
import numpy as np
import pytest

import synth
from helpers import to_dev, upload_layer


@pytest.fixture(scope="module")
def mb():
    import memory_bound_routed_amd as m
    return m


def say(*a):
    print(*a, flush=True)


def _cfg(mb, wl, max_tokens, keep):
    if wl.vq:
        return mb.make_config(wl.H, wl.I, wl.E, wl.k, wl.block_b, max_tokens, mb.MOE_WFORMAT_VQLR, wl.vq_d, wl.vq_K,
                              wl.lr_r)
    return mb.make_config(wl.H, wl.I, wl.E, wl.k, wl.block_b, max_tokens, max_keep=keep)


def _outputs(buf, M, keep):
    import torch
    out = {"y": buf["y"][:M].view(torch.int32), "ids": buf["ids"][:M], "w": buf["w"][:M].view(torch.int32)}
    if keep:
        out["kept"] = buf["kept"].view(-1)[: M * keep]
    else:
        out["counts"] = buf["counts"]
        n = int(buf["counts"][1].item())
        out["sorted_routes"] = buf["sorted_routes"][:n]
        out["block_expert"] = buf["block_expert"][: int(buf["counts"][0].item())]
    return {k: v.clone() for k, v in out.items()}


def _buffers(mb, cfg, M, keep):
    import torch
    cap = mb.moe_align_capacity(M, cfg.top_k, cfg.E, cfg.block_b)
    i32 = torch.int32
    return {"ids": torch.full((M, cfg.top_k), -3, dtype=i32, device="cuda"),
            "w": torch.full((M, cfg.top_k), -1.0, device="cuda"),
            "logits": torch.full((M, cfg.E), -1.0, device="cuda"),
            "sorted_routes": torch.full((max(cap, 1),), -7, dtype=i32, device="cuda"),
            "block_expert": torch.full((max(cap // cfg.block_b, 1),), -7, dtype=i32, device="cuda"),
            "counts": torch.full((2,), -1, dtype=i32, device="cuda"),
            "y": torch.full((M, cfg.H), -1.0, device="cuda"),
            "kept": torch.full((M, max(keep, 1)), -5, dtype=i32, device="cuda")}


def _call(fn, first, b, h, M, keep):
    args = (h, M, b["ids"], b["w"], b["logits"], b["sorted_routes"], b["block_expert"], b["counts"], keep,
            b["kept"] if keep else None, b["y"])
    fn(*first, *args)


# (workload, max_tokens, first M, second M, channel top-K)
CASES = [("dense_h2048_i768_e128_k8_m1", 8, 8, 1, 0),
         ("aligned_h2048_i768_e128_k8_m21", 21, 21, 5, 0),
         ("chansparse_h2048_i768_e128_k8_m1_keep799", 4, 3, 1, 799),
         ("vqlr_h2048_i768_e128_k8_m4_d8_K256_r64", 4, 4, 2, 0),
         ("tiny_h256_i128_e16_k2", 4, 4, 1, 0)]


@pytest.mark.gpu
@pytest.mark.parametrize("name,max_tokens,M1,M2,keep", CASES)
def test_noalloc_decode_step_equals_context_call(mb, name, max_tokens, M1, M2, keep):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = synth.WORKLOADS[name]
    say("no-alloc decode step vs context call:", name, "M =", M1, "then", M2)
    inp = synth.layer_inputs(wl, 0)
    dev = upload_layer(inp)
    cfg = _cfg(mb, wl, max_tokens, keep)
    if keep:
        dev["chan_norm"] = torch.empty((wl.E, wl.I), dtype=torch.float32, device="cuda")
        mb.moe_channel_norms(cfg, dev["w_gate"], dev["w_up"], dev["w_down"], dev["chan_norm"])
    layer = mb.Layer(cfg, dev)
    hs = to_dev(np.concatenate([synth.hidden(wl, 0, step=s, M=1) for s in range(M1)]))
    for M in (M1, M2):
        ref = _buffers(mb, cfg, M, keep)
        got = _buffers(mb, cfg, M, keep)
        h = hs[:M].contiguous()
        _call(mb.moe_decode_step, (layer.ctx,), ref, h, M, keep)
        _call(mb.moe_decode_step_noalloc, (cfg, layer.weights), got, h, M, keep)
        torch.cuda.synchronize()
        a, b = _outputs(ref, M, keep), _outputs(got, M, keep)
        for k in a:
            assert torch.equal(a[k], b[k]), "%s differs at M = %d" % (k, M)
        say("  M = %d: outputs bitwise equal (%s)" % (M, ", ".join(sorted(a))))
    assert mb.moe_read_device_error(layer.ctx) == 0
    layer.close()


@pytest.mark.gpu
def test_noalloc_calls_of_growing_and_shrinking_size(mb):
    """Calls of 4, 200 and 3 tokens in a row on the tiny layer (max_tokens
    256): the router's tickets of the 200-token call lie past those of the
    4-token call, where a size-dependent layout would have put the first
    call's router partials; each call equals the context call bit for bit."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = synth.WORKLOADS["tiny_h256_i128_e16_k2"]
    inp = synth.layer_inputs(wl, 0)
    dev = upload_layer(inp)
    cfg = _cfg(mb, wl, 256, 0)
    layer = mb.Layer(cfg, dev)
    hs = to_dev(np.concatenate([synth.hidden(wl, 0, step=s, M=1) for s in range(200)]))
    for M in (4, 200, 3):
        say("no-alloc tiny layer, M =", M)
        ref = _buffers(mb, cfg, M, 0)
        got = _buffers(mb, cfg, M, 0)
        h = hs[:M].contiguous()
        _call(mb.moe_decode_step, (layer.ctx,), ref, h, M, 0)
        _call(mb.moe_decode_step_noalloc, (cfg, layer.weights), got, h, M, 0)
        torch.cuda.synchronize()
        a, b = _outputs(ref, M, 0), _outputs(got, M, 0)
        for k in a:
            assert torch.equal(a[k], b[k]), "%s differs at M = %d" % (k, M)
    assert mb.moe_read_device_error(layer.ctx) == 0
    layer.close()


def test_noalloc_rejects_oversized_workspace_before_any_launch(mb):
    """Host checks only (no GPU needed): a layer whose workspace for this M
    exceeds the 16 MiB array, an M above max_tokens and invalid arguments are
    refused before the device is touched."""
    cfg = mb.make_config(8192, 16384, 64, 8, 8, 64)
    fake = 1 << 20  # aligned non-null stand-ins: nothing is dereferenced on these paths
    w = mb.make_weights(fake, fake, w_gate=fake, w_up=fake)
    need = mb.moe_workspace_bytes(cfg, 64)
    assert need > 16 * 2 ** 20
    st = mb.moe_decode_step_noalloc_status(cfg, w, fake, 64, fake, fake, None, fake, fake, fake, 0, None, fake)
    assert st == mb.MOE_ERR_CAPACITY
    st = mb.moe_decode_step_noalloc_status(cfg, w, fake, 65, fake, fake, None, fake, fake, fake, 0, None, fake)
    assert st == mb.MOE_ERR_CAPACITY
    st = mb.moe_decode_step_noalloc_status(cfg, w, fake, -1, fake, fake, None, fake, fake, fake, 0, None, fake)
    assert st == mb.MOE_ERR_INVALID_ARG
    bad = mb.make_config(2048, 768, 128, 8, 8, 1)
    bad.H = 2050
    st = mb.moe_decode_step_noalloc_status(bad, w, fake, 1, fake, fake, None, fake, fake, fake, 0, None, fake)
    assert st == mb.MOE_ERR_UNSUPPORTED
    nw = mb.make_weights(fake, None, w_gate=fake, w_up=fake)
    st = mb.moe_decode_step_noalloc_status(mb.make_config(2048, 768, 128, 8, 8, 1), nw, fake, 1, fake, fake, None,
                                           fake, fake, fake, 0, None, fake)
    assert st == mb.MOE_ERR_INVALID_ARG
