"""CPU tests of the C ABI: the library loads and exports every declared symbol,
host-side checks fail closed before touching the GPU, and the host plan
validator rejects each class of broken plan (in the spirit of the mutation
rejections of "Route-Block Membership Selects Packed-AWQ Arithmetic", Sec. 4.2)."""
import ctypes
import os
import re
import shutil
import subprocess
import sys

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def mb():
    import memory_bound_routed_amd as m
    return m


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_header_declares_the_five_calls_and_helpers():
    names = declared_functions()
    for n in ("moe_create", "moe_route_topk", "moe_align_blocks", "moe_expert_forward", "moe_destroy"):
        assert n in names


def test_library_exports_every_declared_symbol(mb):
    lib = ctypes.CDLL(mb.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert sorted(mb.EXPORTS) == declared_functions()
    nm = subprocess.run(["nm", "-D", "--defined-only", mb.LIB_PATH], capture_output=True, text=True).stdout
    for name in declared_functions():
        assert re.search(r"\bT %s\b" % name, nm), name


def test_status_strings_and_capacity(mb):
    for s in range(6):
        assert mb.moe_status_string(s)
    assert mb.moe_status_string(99) == "unknown status"
    assert mb.moe_align_capacity(21, 8, 128, 8) == 168 + 128 * 7 == O.align_capacity(21, 8, 128, 8)
    assert mb.moe_align_capacity(1, 8, 128, 8) == 8 + 8 * 7
    assert mb.moe_align_capacity(0, 8, 128, 8) == 0
    assert mb.moe_align_capacity(-1, 8, 128, 8) == -1
    assert mb.moe_kernel_name(3) == "gateup" and mb.moe_kernel_name(99) is None


def base_cfg(mb, **kw):
    d = dict(H=2048, I=768, E=128, top_k=8, block_b=8, max_tokens=1)
    d.update(kw)
    return mb.make_config(**d)


FAKE = 0x10000  # 16-byte aligned fake address: never dereferenced by host checks


@pytest.mark.parametrize("kw,status", [
    (dict(H=0), 1), (dict(I=-1), 1), (dict(top_k=0), 1), (dict(max_tokens=0), 1), (dict(max_keep=-1), 1),
    (dict(H=2044), 2), (dict(H=8200), 2), (dict(E=20), 2), (dict(E=2048), 2), (dict(top_k=33, E=64), 2),
    (dict(top_k=9, E=8), 2), (dict(block_b=65), 2), (dict(max_tokens=4097), 2), (dict(max_tokens=600), 2),
    (dict(wformat=7), 2), (dict(wformat=1, vq_d=16, vq_K=256, lr_r=64), 2),
    (dict(wformat=1, vq_d=3, vq_K=256, lr_r=64), 2), (dict(wformat=1, H=4096, vq_d=2, vq_K=256, lr_r=64), 2),
    (dict(wformat=1, vq_d=8, vq_K=257, lr_r=64), 2), (dict(wformat=1, vq_d=8, vq_K=256, lr_r=60), 2),
    (dict(max_keep=8 * 768 + 1), 2), (dict(wformat=1, vq_d=8, vq_K=256, lr_r=64, max_keep=10), 2),
    (dict(reader=2, max_keep=10), 1), (dict(rec_rank=-8, reader=1, max_keep=10), 1),
    (dict(reader=1), 2), (dict(reader=1, max_keep=10, H=2040), 2), (dict(rec_rank=32, max_keep=10), 2),
    (dict(reader=1, max_keep=10, rec_rank=12), 2), (dict(reader=1, max_keep=10, rec_rank=40), 2),
])
def test_create_rejects_bad_configs_before_any_gpu_call(mb, kw, status):
    cfg = base_cfg(mb, **kw)
    w = mb.make_weights(FAKE, FAKE, w_gate=FAKE, w_up=FAKE)
    st, ctx = mb.moe_create_status(cfg, w)
    assert st == status and ctx is None


def test_create_rejects_missing_or_misaligned_weights(mb):
    cfg = base_cfg(mb)
    assert mb.moe_create_status(cfg, mb.make_weights(FAKE, FAKE))[0] == mb.MOE_ERR_INVALID_ARG  # no gate/up
    assert mb.moe_create_status(cfg, mb.make_weights(None, FAKE, w_gate=FAKE, w_up=FAKE))[0] == 1
    assert mb.moe_create_status(cfg, mb.make_weights(FAKE, FAKE, w_gate=FAKE + 2, w_up=FAKE))[0] == 1
    vq = base_cfg(mb, wformat=1, vq_d=8, vq_K=256, lr_r=64)
    ok = dict(lr_basis=(FAKE, FAKE), lr_coef=(FAKE, FAKE), vq_book=(FAKE, FAKE), vq_idx=(FAKE, FAKE))
    bad = dict(ok, vq_idx=(FAKE, None))
    assert mb.moe_create_status(vq, mb.make_weights(FAKE, FAKE, **bad))[0] == 1
    bad = dict(ok, vq_idx=(FAKE, FAKE + 1))
    assert mb.moe_create_status(vq, mb.make_weights(FAKE, FAKE, **bad))[0] == 1
    keep = base_cfg(mb, max_keep=799)
    assert mb.moe_create_status(keep, mb.make_weights(FAKE, FAKE, w_gate=FAKE, w_up=FAKE))[0] == 1  # no norms
    assert mb.moe_create_status(keep, mb.make_weights(FAKE, FAKE, w_gate=FAKE, w_up=FAKE,
                                                      chan_norm=FAKE + 4))[0] == 1  # norms read 16 bytes at a time
    rd = base_cfg(mb, max_keep=756, reader=1, rec_rank=32)
    full = dict(w_gate=FAKE, w_up=FAKE, rot_signs=FAKE, sketch=FAKE, sketch_scale=FAKE, down_norm=FAKE,
                rec_basis=FAKE, rec_coef=FAKE)
    for name, val in (("rot_signs", None), ("sketch", None), ("sketch", FAKE + 8), ("sketch_scale", None),
                      ("down_norm", None), ("down_norm", FAKE + 4), ("rec_basis", None), ("rec_coef", None),
                      ("rec_coef", FAKE + 2)):
        assert mb.moe_create_status(rd, mb.make_weights(FAKE, FAKE, **dict(full, **{name: val})))[0] == 1, name
    assert mb.moe_create_status(None, mb.make_weights(FAKE, FAKE))[0] == 1


def test_calls_on_null_context_fail_closed(mb):
    lib = mb._lib
    assert lib.moe_route_topk(None, FAKE, 1, FAKE, FAKE, None, None) == 1
    assert lib.moe_align_blocks(None, FAKE, 1, FAKE, FAKE, FAKE, None) == 1
    assert lib.moe_expert_forward(None, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None, FAKE, None) == 1
    assert lib.moe_profile_enable(None, 1) == 1
    flags = ctypes.c_int32(0)
    assert lib.moe_read_device_error(None, ctypes.byref(flags), 0) == 1
    lib.moe_destroy(None)  # no-op
    cfg = base_cfg(mb)
    assert lib.moe_channel_norms(ctypes.byref(cfg), None, FAKE, FAKE, FAKE, None) == 1
    bad = base_cfg(mb, H=2044)
    assert lib.moe_channel_norms(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, None) == 2


# ---------------------------------------------------------------- plan validator

def plan_of(ids, E, b):
    al = O.align_blocks(ids, E, b)
    return (al["sorted_routes"].astype(np.int32), al["block_expert"].astype(np.int32),
            np.array([al["num_blocks"], al["num_padded"]], np.int32))


def routing(seed, M=21, k=8, E=128, hot=True):
    rng = np.random.default_rng(seed)
    p = np.ones(E)
    if hot:
        p[:4] = 30.0
    return np.stack([rng.choice(E, k, replace=False, p=p / p.sum()) for _ in range(M)]).astype(np.int32)


def test_validator_accepts_canonical_and_noncanonical_valid_plans(mb):
    for seed in range(30):
        ids = routing(seed)
        rows, blocks, counts = plan_of(ids, 128, 8)
        assert mb.moe_validate_plan(ids, 21, 8, 128, 8, rows, blocks, counts) == (0, 0)
        R = ids.size
        # within-block permutation
        perm = rows.copy()
        seg = perm[:8]
        v = seg[seg != R]
        seg[: v.size] = v[::-1]
        assert mb.moe_validate_plan(ids, 21, 8, 128, 8, perm, blocks, counts) == (0, 0)
        # cross-boundary exchange between two blocks of one expert
        multi = [e for e in set(blocks.tolist()) if (blocks == e).sum() >= 2]
        if multi:
            b0 = int(np.nonzero(blocks == multi[0])[0][0])
            sw = rows.copy()
            sw[b0 * 8], sw[b0 * 8 + 8] = rows[b0 * 8 + 8], rows[b0 * 8]
            assert mb.moe_validate_plan(ids, 21, 8, 128, 8, sw, blocks, counts) == (0, 0)


def test_validator_rejects_each_mutation_class(mb):
    ids = routing(7)
    R = ids.size
    rows, blocks, counts = plan_of(ids, 128, 8)
    V = lambda r=rows, b=blocks, c=counts, i=ids: mb.moe_validate_plan(i, 21, 8, 128, 8, r, b, c)
    assert V() == (0, 0)
    # 1: counts out of range / inconsistent
    assert V(c=np.array([counts[0], counts[1] + 1], np.int32))[1] == 1
    assert V(c=np.array([-1, -8], np.int32))[1] == 1
    # 2: a route dropped (replaced by a pad at a block tail that keeps another route)
    blk = next(i for i in range(counts[0]) if (rows[i * 8:i * 8 + 8] != R).sum() >= 2)
    last = blk * 8 + int((rows[blk * 8:blk * 8 + 8] != R).sum()) - 1
    m = rows.copy(); m[last] = R
    assert V(r=m)[1] == 2
    # 3: a route duplicated
    m = rows.copy(); m[last] = rows[blk * 8]
    assert V(r=m)[1] == 3
    # 4: a row placed in another expert's block
    other = next(i for i in range(counts[0]) if blocks[i] != blocks[blk])
    m = rows.copy(); m[blk * 8], m[other * 8] = rows[other * 8], rows[blk * 8]
    assert V(r=m)[1] == 4
    # 5: a pad before a route inside a block
    m = rows.copy(); m[blk * 8], m[last] = R, rows[blk * 8]
    assert V(r=m)[1] == 5
    # 6: blocks out of expert order
    b = blocks.copy(); b[0], b[-1] = blocks[-1], blocks[0]
    assert V(b=b)[1] in (4, 6)
    b = blocks.copy(); b[0] = 128
    assert V(b=b)[1] == 6
    # 7: an invalid route id present in the plan
    bad = ids.copy(); bad.flat[rows[0]] = -1
    assert V(i=bad)[1] in (4, 7)
    # 8: a row value outside [0, R]
    m = rows.copy(); m[0] = R + 5
    assert V(r=m)[1] == 8


def test_product_package_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "memory_bound_routed_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, re.M), f
                assert "moe_oracle" not in text, f


def test_binding_fails_loudly_without_the_library(tmp_path):
    dst = tmp_path / "memory_bound_routed_amd"
    dst.mkdir()
    shutil.copy(os.path.join(ROOT, "memory_bound_routed_amd", "__init__.py"), dst / "__init__.py")
    r = subprocess.run([sys.executable, "-c", "import memory_bound_routed_amd"], cwd=tmp_path,
                       capture_output=True, text=True)
    assert r.returncode != 0 and "libmoe.so is not built" in r.stderr


def test_multiply_high_division_identity():
    """The kernels divide by launch-time constants (E, k, block size) with
    multiply-high (Granlund & Montgomery 1994): s = ceil(log2 d),
    m = floor(2^32 (2^s - d) / d) + 1, x / d = (umulhi(x, m) + x) >> s for
    0 <= x < 2^31.  Checked against integer division over the divisors the
    library can see and x at the range edges and in between."""
    import numpy as np
    rng = np.random.default_rng(5)
    xs = np.unique(np.concatenate([np.arange(0, 70000, dtype=np.int64),
                                   (2 ** 31 - 1) - np.arange(0, 5000, dtype=np.int64),
                                   rng.integers(0, 2 ** 31, 20000, dtype=np.int64)]))
    for d in list(range(1, 2049)) + [4095, 4096, 4097, 6144, 8191, 8192, 65537, 2 ** 30 + 3]:
        s = 0
        while (1 << s) < d:
            s += 1
        m = ((1 << 32) * ((1 << s) - d)) // d + 1
        assert m < (1 << 32)
        q = (((xs * m) >> 32) + xs) >> s
        assert np.array_equal(q, xs // d), d


def test_workspace_bytes_at_the_accepted_limits():
    """The context workspace holds, per route, I floats of SiLU(gate)*up and one
    H-float down partial (the split schedule), plus the fused schedule's
    chunked partials of a single token's top_k routes; it never scales with
    max_tokens * top_k * (fused chunks).  Checked where check_config's limits
    bind (4096 routes, H = 4096, I = 16384) and on the 21-token workload."""
    import memory_bound_routed_amd as mb
    for (H, I, E, k, MT) in [(4096, 16384, 96, 8, 512), (8192, 16384, 32, 32, 128), (2048, 768, 128, 8, 21),
                             (2048, 768, 128, 8, 1)]:
        cfg = mb.make_config(H, I, E, k, 8, MT)
        ws = mb.moe_workspace_bytes(cfg, MT)
        R = MT * k
        fused_chunks = -(-I // 24) if H <= 2048 else -(-I // 8)
        fused = k * fused_chunks * H * 4 if H <= 4096 else 0
        main = R * I * 4 + max(R * H * 4, fused)
        assert main <= ws <= main + 8 * 2 ** 20, (H, I, E, k, MT, ws, main)
    # rejected configurations report -1
    assert mb.moe_workspace_bytes(mb.make_config(4096, 16384, 1024, 8, 8, 512), 512) == -1
    assert mb.moe_workspace_bytes(mb.make_config(2048, 768, 128, 8, 8, 1), 0) == -1


def test_reader_load_time_entry_points_check_arguments(mb):
    """Host-side checks of the reader's load-time calls (no GPU needed)."""
    lib = mb._lib
    assert mb.moe_sketch_row_bytes(768) == 160  # ceil(768 / 5) = 154 bytes, padded to 16
    assert mb.moe_sketch_row_bytes(5) == 16 and mb.moe_sketch_row_bytes(0) == -1
    cfg = base_cfg(mb)
    assert lib.moe_reader_sketch(ctypes.byref(cfg), FAKE, FAKE, None, FAKE, FAKE, None) == 1
    assert lib.moe_reader_sketch(ctypes.byref(base_cfg(mb, H=2056)), FAKE, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert lib.moe_reader_sketch(None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.moe_down_norms(ctypes.byref(cfg), FAKE + 8, FAKE, None) == 1
    assert lib.moe_recovery_basis(ctypes.byref(cfg), FAKE, 0, 10, FAKE, None) == 1
    assert lib.moe_recovery_basis(ctypes.byref(cfg), FAKE, 33, 10, FAKE, None) == 1
    assert lib.moe_recovery_basis(ctypes.byref(cfg), FAKE, 32, 0, FAKE, None) == 1
    assert lib.moe_recovery_basis(ctypes.byref(base_cfg(mb, H=2056)), FAKE, 32, 10, FAKE, None) == 2
    assert lib.moe_recovery_coefs(ctypes.byref(cfg), FAKE, 12, FAKE, FAKE, None) == 1
    assert lib.moe_recovery_coefs(ctypes.byref(cfg), FAKE, 32, FAKE, FAKE + 2, None) == 1
    assert lib.moe_reader_inspect(None, FAKE, 1, FAKE, FAKE, 10, None, None, None, None, None, None) == 1
