"""Seeded synthetic inputs for the MoE decode-step workloads.

This module only draws inputs (weights, hidden states, index maps, router
bias); it holds none of the MoE method's arithmetic.  The fp64 oracle and the
GPU library both take their inputs from here and from nowhere else.

Every tensor is a pure function of (seed, tag, index) -- see ``gen.c`` for the
exact stream definition -- so a single expert of a single layer can be drawn
on its own.  Per-expert tensors use one tag per expert, which lets the oracle
draw only the experts a token is routed to.

Workloads (shapes from the pages: hidden 2048, 768 channels per expert, 128
experts with top-8 routing and 8-row alignment blocks; synthetic values):

  tiny_h256_i128_e16_k2           one token, H=256, I=128, E=16, top-2
  dense_h2048_i768_e128_k8_m1     one token, 48 independent layers
  aligned_h2048_i768_e128_k8_m21  21 tokens, 4 hot experts biased to ~20% of routes
  chansparse_h2048_i768_e128_k8_m1_keep799   channel top-K, K = 799 of 6144
  vqlr_h2048_i768_e128_k8_m4_d8_K256_r64     VQ + low-rank gate/up, 4 tokens
  vqlr_..._d4_K256_r256, _d8_K256_r384, _d2_K256_r8, _d2_K256_r0   the same at
                                             the 4-bit storage rate, block lengths 4, 8, 2
                                             (r = 0: VQ only)
  dense_..._m8, _m16; vqlr_..._m8_..., _m16_...   batch 8 and 16 decode

Distributions: every weight ~ N(0, 0.02) rounded to bf16; hidden states
~ N(0, 1) in fp32; VQ index maps uniform over [0, 256).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Dict, Iterable, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the generator with gcc (OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.synth_normal_bf16.argtypes = [u64, u64, i64, dbl, vp]
        lib.synth_normal_f32.argtypes = [u64, u64, i64, dbl, vp]
        lib.synth_uniform_u8.argtypes = [u64, u64, i64, vp]
        lib.synth_words.argtypes = [u64, u64, i64, vp]
        for f in (lib.synth_normal_bf16, lib.synth_normal_f32, lib.synth_uniform_u8, lib.synth_words):
            f.restype = None
        _lib = lib
    return _lib


def tag_of(name: str) -> int:
    """64-bit FNV-1a hash of a tensor name."""
    h = 0xCBF29CE484222325
    for b in name.encode():
        h ^= b
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def normal_bf16(seed: int, name: str, shape, sigma: float, out: Optional[np.ndarray] = None) -> np.ndarray:
    n = int(np.prod(shape))
    if out is None:
        out = np.empty(shape, np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size == n
    _load().synth_normal_bf16(seed, tag_of(name), n, float(sigma), out.ctypes.data)
    return out


def normal_f32(seed: int, name: str, shape, sigma: float = 1.0) -> np.ndarray:
    out = np.empty(shape, np.float32)
    _load().synth_normal_f32(seed, tag_of(name), out.size, float(sigma), out.ctypes.data)
    return out


def uniform_u8(seed: int, name: str, shape, out: Optional[np.ndarray] = None) -> np.ndarray:
    if out is None:
        out = np.empty(shape, np.uint8)
    _load().synth_uniform_u8(seed, tag_of(name), out.size, out.ctypes.data)
    return out


def words(seed: int, name: str, n: int) -> np.ndarray:
    out = np.empty(n, np.uint64)
    _load().synth_words(seed, tag_of(name), n, out.ctypes.data)
    return out


def distinct_ints(seed: int, name: str, count: int, upper: int) -> np.ndarray:
    """`count` distinct integers in [0, upper), drawn in stream order (rejection of repeats)."""
    got = []
    n = 0
    while len(got) < count:
        for w in words(seed, name + "/%d" % n, 64):
            v = int(w % np.uint64(upper))
            if v not in got:
                got.append(v)
                if len(got) == count:
                    break
        n += 1
    return np.array(got, np.int64)


SIGMA_W = 0.02
# Additive router bias for the four hot experts of the 21-token workload.  A
# Monte Carlo over N(0, (0.02^2)*2048) logits puts 1.25 at a ~20% expected
# share of the 168 routes on the four hot experts; the realised share of each
# seed is reported by the tests rather than tuned.
HOT_BIAS = 1.25


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    H: int
    I: int
    E: int
    k: int
    M: int
    seed: int
    layers: int = 1
    block_b: int = 8
    hot_experts: int = 0          # experts given the additive router bias
    keep: int = 0                 # channel top-K (0 = dense)
    vq: bool = False
    vq_d: int = 8
    vq_K: int = 256
    lr_r: int = 64
    reader: bool = False          # channel scores from the ternary-sketch reader
    rec_rank: int = 0             # rank of the reader's recovery map (0 = none)

    def layer_seed(self, layer: int) -> int:
        return self.seed * 1000 + layer

    @property
    def routed_bytes_per_expert(self) -> int:
        if self.vq:
            return 2 * (self.I * (self.H // self.vq_d) + self.I * self.lr_r * 2) + self.I * self.H * 2
        return 3 * self.I * self.H * 2


WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    Workload("tiny_h256_i128_e16_k2", H=256, I=128, E=16, k=2, M=1, seed=1001),
    Workload("dense_h2048_i768_e128_k8_m1", H=2048, I=768, E=128, k=8, M=1, seed=1002, layers=48),
    Workload("aligned_h2048_i768_e128_k8_m21", H=2048, I=768, E=128, k=8, M=21, seed=1003, hot_experts=4),
    Workload("chansparse_h2048_i768_e128_k8_m1_keep799", H=2048, I=768, E=128, k=8, M=1, seed=1004,
             keep=(13 * 8 * 768 + 50) // 100),
    # the sketch reader at the page's exact-channel budget: 12.3% of the
    # 8 * 768 candidates computed exactly, without and with the rank-32 map
    Workload("reader_h2048_i768_e128_k8_m1_keep756", H=2048, I=768, E=128, k=8, M=1, seed=1008, keep=756,
             reader=True),
    Workload("reader_h2048_i768_e128_k8_m1_keep756_r32", H=2048, I=768, E=128, k=8, M=1, seed=1008, keep=756,
             reader=True, rec_rank=32),
    Workload("vqlr_h2048_i768_e128_k8_m4_d8_K256_r64", H=2048, I=768, E=128, k=8, M=4, seed=1005, vq=True),
    # block-length sweep at the 4-bit storage rate, same router, hidden states
    # and routing as the workload above (same seed)
    Workload("vqlr_h2048_i768_e128_k8_m4_d4_K256_r256", H=2048, I=768, E=128, k=8, M=4, seed=1005, vq=True,
             vq_d=4, lr_r=256),
    Workload("vqlr_h2048_i768_e128_k8_m4_d8_K256_r384", H=2048, I=768, E=128, k=8, M=4, seed=1005, vq=True,
             vq_d=8, lr_r=384),
    Workload("vqlr_h2048_i768_e128_k8_m4_d2_K256_r8", H=2048, I=768, E=128, k=8, M=4, seed=1005, vq=True,
             vq_d=2, lr_r=8),
    # the page's VQ-only point (d, r) = (2, 0): no low-rank term
    Workload("vqlr_h2048_i768_e128_k8_m4_d2_K256_r0", H=2048, I=768, E=128, k=8, M=4, seed=1005, vq=True,
             vq_d=2, lr_r=0),
    # dense bf16 at the VQ workloads' batch of 4: same seed, so the same router,
    # hidden states and routing as the VQ + low-rank workloads above
    Workload("dense_h2048_i768_e128_k8_m4", H=2048, I=768, E=128, k=8, M=4, seed=1005),
    # batch 8 and 16 decode (no hot experts): dense bf16 and VQ + low rank
    Workload("dense_h2048_i768_e128_k8_m8", H=2048, I=768, E=128, k=8, M=8, seed=1006),
    Workload("dense_h2048_i768_e128_k8_m16", H=2048, I=768, E=128, k=8, M=16, seed=1007),
    Workload("vqlr_h2048_i768_e128_k8_m8_d8_K256_r64", H=2048, I=768, E=128, k=8, M=8, seed=1006, vq=True),
    Workload("vqlr_h2048_i768_e128_k8_m16_d8_K256_r64", H=2048, I=768, E=128, k=8, M=16, seed=1007, vq=True),
    # one GPU's share of the batch-1 dense layer under 8-way channel sharding:
    # 96 of every expert's 768 channels (same seed: the same router, hidden
    # states and routing as dense_h2048_i768_e128_k8_m1)
    Workload("shard8_h2048_i96_e128_k8_m1", H=2048, I=96, E=128, k=8, M=1, seed=1002, layers=48),
]}


def small_workload(name: str, H: int, I: int, E: int, k: int, M: int, seed: int, **kw) -> Workload:
    """An ad-hoc workload for tests (ragged and tiny shapes)."""
    return Workload(name, H=H, I=I, E=E, k=k, M=M, seed=seed, **kw)


def hidden(wl: Workload, layer: int, step: int = 0, M: Optional[int] = None) -> np.ndarray:
    """h ~ N(0,1) fp32, [M][H]; `step` selects an independent draw."""
    M = wl.M if M is None else M
    return normal_f32(wl.layer_seed(layer), "h/step%d" % step, (M, wl.H), 1.0)


def router_weight(wl: Workload, layer: int) -> np.ndarray:
    return normal_bf16(wl.layer_seed(layer), "router_w", (wl.H, wl.E), SIGMA_W)


def router_bias(wl: Workload, layer: int) -> Optional[np.ndarray]:
    if not wl.hot_experts:
        return None
    hot = distinct_ints(wl.layer_seed(layer), "hot_experts", wl.hot_experts, wl.E)
    b = np.zeros(wl.E, np.float32)
    b[hot] = np.float32(HOT_BIAS)
    return b


def rotation_signs(wl: Workload, layer: int, block: int = 128) -> np.ndarray:
    """Random signs +-1 (int8 [H / block][block]) of the channel-selection
    reader's randomized Hadamard rotation: bit 0 of one stream word each."""
    w = words(wl.layer_seed(layer), "rotation_signs", wl.H)
    return np.where((w & np.uint64(1)) != 0, 1, -1).astype(np.int8).reshape(wl.H // block, block)


def expert_matrix(wl: Workload, layer: int, which: str, experts: Optional[Iterable[int]] = None,
                  out: Optional[np.ndarray] = None) -> np.ndarray:
    """Dense bf16 expert weights [E][I][H] (row j = channel j) for which in
    {'gate','up','down'}.  With `experts`, only those experts are drawn and the
    rest stay zero (np.zeros pages are untouched, so this is cheap)."""
    if out is None:
        out = np.zeros((wl.E, wl.I, wl.H), np.uint16)
    ex = range(wl.E) if experts is None else sorted(set(int(e) for e in experts))
    s = wl.layer_seed(layer)
    for e in ex:
        normal_bf16(s, "%s/e%d" % (which, e), (wl.I, wl.H), SIGMA_W, out=out[e])
    return out


def vq_tensors(wl: Workload, layer: int, experts: Optional[Iterable[int]] = None) -> Dict[str, np.ndarray]:
    """VQ + low-rank gate/up inputs: per projection P in (gate, up)
    basis D_P bf16 [H][r], coefficients C_P bf16 [E][I][r],
    code book B_P bf16 [K][d], index map J_P uint8 [E][I][H/d] with entries < K."""
    s = wl.layer_seed(layer)
    ex = range(wl.E) if experts is None else sorted(set(int(e) for e in experts))
    out = {}
    for P in ("gate", "up"):
        out["lr_basis_" + P] = normal_bf16(s, "lr_basis/" + P, (wl.H, wl.lr_r), SIGMA_W)
        out["vq_book_" + P] = normal_bf16(s, "vq_book/" + P, (wl.vq_K, wl.vq_d), SIGMA_W)
        C = np.zeros((wl.E, wl.I, wl.lr_r), np.uint16)
        J = np.zeros((wl.E, wl.I, wl.H // wl.vq_d), np.uint8)
        for e in ex:
            normal_bf16(s, "lr_coef/%s/e%d" % (P, e), (wl.I, wl.lr_r), SIGMA_W, out=C[e])
            uniform_u8(s, "vq_idx/%s/e%d" % (P, e), (wl.I, wl.H // wl.vq_d), out=J[e])
            if wl.vq_K < 256:  # indices into a smaller code book (identity at K = 256)
                np.remainder(J[e], wl.vq_K, out=J[e])
        out["lr_coef_" + P] = C
        out["vq_idx_" + P] = J
    return out


def layer_inputs(wl: Workload, layer: int = 0, experts: Optional[Iterable[int]] = None,
                 with_down: bool = True) -> Dict[str, np.ndarray]:
    """All inputs of one layer: h, router weight/bias and the expert weights."""
    d = {"h": hidden(wl, layer), "router_w": router_weight(wl, layer), "router_bias": router_bias(wl, layer)}
    if wl.vq:
        d.update(vq_tensors(wl, layer, experts))
    else:
        d["w_gate"] = expert_matrix(wl, layer, "gate", experts)
        d["w_up"] = expert_matrix(wl, layer, "up", experts)
    if with_down:
        d["w_down"] = expert_matrix(wl, layer, "down", experts)
    return d
