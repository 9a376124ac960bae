"""ctypes binding of libmoe.so: argument marshalling only (loaded by the
package __init__ once the library is built)."""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence, Tuple

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

# torch first: it loads its own HIP runtime, which libmoe.so must then bind to
# (the same soname); loaded the other way round, the process would hold two
# HIP runtimes and torch's device memory would be foreign to the library's.
try:
    import torch  # noqa: F401
except ImportError:  # the library can still be loaded (host-side checks)
    pass
_lib = ctypes.CDLL(LIB_PATH)

# ---------------------------------------------------------------- C types

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_CAPACITY, MOE_ERR_HIP, MOE_ERR_DEVICE = range(6)
MOE_WFORMAT_DENSE, MOE_WFORMAT_VQLR = 0, 1
DEVERR_BAD_ROUTE_ID, DEVERR_BAD_PLAN, DEVERR_BAD_BLOCK_EXPERT, DEVERR_BAD_COUNTS = 1, 2, 4, 8
KERNELS = ["router", "vq_shared", "align", "gateup", "gateup_vqlr", "down", "combine",
           "chan_select", "chan_gather", "chan_combine", "expert_fused", "router_align", "router_gemv",
           "decode_fused", "vq_finish", "reader_rotate", "reader_screen", "reader_select", "reader_recover",
           "reader_combine"]
MOE_KERNEL_COUNT = len(KERNELS)

# Every symbol include/moe.h declares (checked by the CPU test suite).
EXPORTS = ["moe_create", "moe_destroy", "moe_route_topk", "moe_route_align", "moe_align_blocks", "moe_expert_forward",
           "moe_decode_step", "moe_decode_step_noalloc",
           "moe_align_capacity", "moe_workspace_bytes", "moe_status_string", "moe_read_device_error", "moe_channel_norms",
           "moe_validate_plan", "moe_profile_enable", "moe_profile_read", "moe_kernel_name", "moe_reader_inspect",
           "moe_sketch_row_bytes", "moe_reader_sketch", "moe_down_norms", "moe_recovery_basis", "moe_recovery_coefs"]


class moe_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("H", "I", "E", "top_k", "block_b", "max_tokens", "wformat", "vq_d", "vq_K", "lr_r", "max_keep",
                 "reader", "rec_rank")]


_vp = ctypes.c_void_p


class moe_weights(ctypes.Structure):
    _fields_ = [("router_w", _vp), ("router_bias", _vp), ("w_gate", _vp), ("w_up", _vp), ("w_down", _vp),
                ("chan_norm", _vp), ("lr_basis", _vp * 2), ("lr_coef", _vp * 2), ("vq_book", _vp * 2),
                ("vq_idx", _vp * 2), ("rot_signs", _vp), ("sketch", _vp), ("sketch_scale", _vp), ("down_norm", _vp),
                ("rec_basis", _vp), ("rec_coef", _vp)]


_i32, _pi32 = ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)
_sig = {
    "moe_create": (_i32, [ctypes.POINTER(moe_config), ctypes.POINTER(moe_weights), ctypes.POINTER(_vp)]),
    "moe_destroy": (None, [_vp]),
    "moe_route_topk": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _vp]),
    "moe_align_blocks": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _vp]),
    "moe_route_align": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_expert_forward": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp]),
    "moe_decode_step": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp]),
    "moe_decode_step_noalloc": (_i32, [ctypes.POINTER(moe_config), ctypes.POINTER(moe_weights), _vp, _i32, _vp, _vp,
                                       _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp]),
    "moe_align_capacity": (_i32, [_i32, _i32, _i32, _i32]),
    "moe_workspace_bytes": (ctypes.c_int64, [ctypes.POINTER(moe_config), _i32]),
    "moe_status_string": (ctypes.c_char_p, [_i32]),
    "moe_read_device_error": (_i32, [_vp, _pi32, _i32]),
    "moe_channel_norms": (_i32, [ctypes.POINTER(moe_config), _vp, _vp, _vp, _vp, _vp]),
    "moe_validate_plan": (_i32, [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _pi32]),
    "moe_profile_enable": (_i32, [_vp, _i32]),
    "moe_profile_read": (_i32, [_vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
    "moe_kernel_name": (ctypes.c_char_p, [_i32]),
    "moe_reader_inspect": (_i32, [_vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_sketch_row_bytes": (_i32, [_i32]),
    "moe_reader_sketch": (_i32, [ctypes.POINTER(moe_config), _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_down_norms": (_i32, [ctypes.POINTER(moe_config), _vp, _vp, _vp]),
    "moe_recovery_basis": (_i32, [ctypes.POINTER(moe_config), _vp, _i32, _i32, _vp, _vp]),
    "moe_recovery_coefs": (_i32, [ctypes.POINTER(moe_config), _vp, _i32, _vp, _vp, _vp]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, moe_status_string(status), status))


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)


def _ptr(t) -> Optional[int]:
    """Device or host address of a tensor / array (None stays NULL)."""
    if t is None:
        return None
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    if hasattr(t, "ctypes"):
        return t.ctypes.data
    return int(t)


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


# ---------------------------------------------------------------- entry points

def moe_status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


def moe_kernel_name(kernel: int) -> Optional[str]:
    s = _lib.moe_kernel_name(kernel)
    return s.decode() if s else None


def moe_align_capacity(M: int, k: int, E: int, b: int) -> int:
    return _lib.moe_align_capacity(M, k, E, b)


def moe_workspace_bytes(cfg: "moe_config", max_tokens: int) -> int:
    return _lib.moe_workspace_bytes(ctypes.byref(cfg), max_tokens)


def make_config(H, I, E, top_k, block_b=8, max_tokens=1, wformat=MOE_WFORMAT_DENSE, vq_d=0, vq_K=0, lr_r=0,
                max_keep=0, reader=0, rec_rank=0) -> moe_config:
    return moe_config(H, I, E, top_k, block_b, max_tokens, wformat, vq_d, vq_K, lr_r, max_keep, reader, rec_rank)


def make_weights(router_w, w_down, router_bias=None, w_gate=None, w_up=None, chan_norm=None,
                 lr_basis=(None, None), lr_coef=(None, None), vq_book=(None, None),
                 vq_idx=(None, None), rot_signs=None, sketch=None, sketch_scale=None, down_norm=None,
                 rec_basis=None, rec_coef=None) -> moe_weights:
    w = moe_weights()
    w.router_w, w.router_bias, w.w_gate, w.w_up, w.w_down, w.chan_norm = (
        _ptr(router_w), _ptr(router_bias), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(chan_norm))
    for P in range(2):
        w.lr_basis[P], w.lr_coef[P] = _ptr(lr_basis[P]), _ptr(lr_coef[P])
        w.vq_book[P], w.vq_idx[P] = _ptr(vq_book[P]), _ptr(vq_idx[P])
    w.rot_signs, w.sketch, w.sketch_scale, w.down_norm = _ptr(rot_signs), _ptr(sketch), _ptr(sketch_scale), \
        _ptr(down_norm)
    w.rec_basis, w.rec_coef = _ptr(rec_basis), _ptr(rec_coef)
    return w


def moe_create(cfg: moe_config, weights: moe_weights) -> int:
    out = _vp()
    _check(_lib.moe_create(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(out)), "moe_create")
    return out.value


def moe_create_status(cfg: Optional[moe_config], weights: Optional[moe_weights]) -> Tuple[int, Optional[int]]:
    """Raw status variant (for tests of the failure paths)."""
    out = _vp()
    st = _lib.moe_create(ctypes.byref(cfg) if cfg is not None else None,
                         ctypes.byref(weights) if weights is not None else None, ctypes.byref(out))
    return st, out.value


def moe_destroy(ctx: Optional[int]) -> None:
    _lib.moe_destroy(ctx)


def moe_route_topk(ctx, h, M, topk_ids, topk_w, logits_out=None, stream=None) -> None:
    _check(_lib.moe_route_topk(ctx, _ptr(h), M, _ptr(topk_ids), _ptr(topk_w), _ptr(logits_out), _stream(stream)),
           "moe_route_topk")


def moe_route_align(ctx, h, M, topk_ids, topk_w, logits_out, sorted_routes, block_expert, counts, stream=None) -> None:
    _check(_lib.moe_route_align(ctx, _ptr(h), M, _ptr(topk_ids), _ptr(topk_w), _ptr(logits_out), _ptr(sorted_routes),
                                _ptr(block_expert), _ptr(counts), _stream(stream)), "moe_route_align")


def moe_align_blocks(ctx, topk_ids, M, sorted_routes, block_expert, counts, stream=None) -> None:
    _check(_lib.moe_align_blocks(ctx, _ptr(topk_ids), M, _ptr(sorted_routes), _ptr(block_expert), _ptr(counts),
                                 _stream(stream)), "moe_align_blocks")


def moe_expert_forward(ctx, h, M, topk_ids, topk_w, sorted_routes, block_expert, counts, keep_channels, kept_out, y,
                       stream=None) -> None:
    _check(_lib.moe_expert_forward(ctx, _ptr(h), M, _ptr(topk_ids), _ptr(topk_w), _ptr(sorted_routes),
                                   _ptr(block_expert), _ptr(counts), keep_channels, _ptr(kept_out), _ptr(y),
                                   _stream(stream)), "moe_expert_forward")


def moe_decode_step(ctx, h, M, topk_ids, topk_w, logits_out, sorted_routes, block_expert, counts, keep_channels,
                    kept_out, y, stream=None) -> None:
    _check(_lib.moe_decode_step(ctx, _ptr(h), M, _ptr(topk_ids), _ptr(topk_w), _ptr(logits_out), _ptr(sorted_routes),
                                _ptr(block_expert), _ptr(counts), keep_channels, _ptr(kept_out), _ptr(y),
                                _stream(stream)), "moe_decode_step")


def moe_decode_step_noalloc(cfg, weights, h, M, topk_ids, topk_w, logits_out, sorted_routes, block_expert, counts,
                            keep_channels, kept_out, y, stream=None) -> None:
    _check(_lib.moe_decode_step_noalloc(ctypes.byref(cfg), ctypes.byref(weights), _ptr(h), M, _ptr(topk_ids),
                                        _ptr(topk_w), _ptr(logits_out), _ptr(sorted_routes), _ptr(block_expert),
                                        _ptr(counts), keep_channels, _ptr(kept_out), _ptr(y), _stream(stream)),
           "moe_decode_step_noalloc")


def moe_decode_step_noalloc_status(cfg, weights, h, M, topk_ids, topk_w, logits_out, sorted_routes, block_expert,
                                   counts, keep_channels, kept_out, y, stream=0) -> int:
    """Raw status variant (for tests of the failure paths; the default stream
    is passed as NULL so that no device is touched before the checks)."""
    return _lib.moe_decode_step_noalloc(ctypes.byref(cfg), ctypes.byref(weights), _ptr(h), M, _ptr(topk_ids),
                                        _ptr(topk_w), _ptr(logits_out), _ptr(sorted_routes), _ptr(block_expert),
                                        _ptr(counts), keep_channels, _ptr(kept_out), _ptr(y), stream)


def moe_read_device_error(ctx, clear: bool = True) -> int:
    flags = _i32(0)
    st = _lib.moe_read_device_error(ctx, ctypes.byref(flags), 1 if clear else 0)
    if st not in (MOE_OK, MOE_ERR_DEVICE):
        raise MoeError(st, "moe_read_device_error")
    return flags.value


def moe_channel_norms(cfg: moe_config, w_gate, w_up, w_down, norms, stream=None) -> None:
    _check(_lib.moe_channel_norms(ctypes.byref(cfg), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(norms),
                                  _stream(stream)), "moe_channel_norms")


def moe_reader_inspect(ctx, h, M, topk_ids, topk_w, K, xsel=None, xval=None, est=None, score=None, kept=None,
                       stream=None) -> None:
    _check(_lib.moe_reader_inspect(ctx, _ptr(h), M, _ptr(topk_ids), _ptr(topk_w), K, _ptr(xsel), _ptr(xval),
                                   _ptr(est), _ptr(score), _ptr(kept), _stream(stream)), "moe_reader_inspect")


def moe_sketch_row_bytes(I: int) -> int:
    return _lib.moe_sketch_row_bytes(I)


def moe_reader_sketch(cfg: moe_config, w_gate, w_up, rot_signs, sketch, sketch_scale, stream=None) -> None:
    _check(_lib.moe_reader_sketch(ctypes.byref(cfg), _ptr(w_gate), _ptr(w_up), _ptr(rot_signs), _ptr(sketch),
                                  _ptr(sketch_scale), _stream(stream)), "moe_reader_sketch")


def moe_down_norms(cfg: moe_config, w_down, down_norm, stream=None) -> None:
    _check(_lib.moe_down_norms(ctypes.byref(cfg), _ptr(w_down), _ptr(down_norm), _stream(stream)), "moe_down_norms")


def moe_recovery_basis(cfg: moe_config, w_down, rank, iters, basis, stream=None) -> None:
    _check(_lib.moe_recovery_basis(ctypes.byref(cfg), _ptr(w_down), rank, iters, _ptr(basis), _stream(stream)),
           "moe_recovery_basis")


def moe_recovery_coefs(cfg: moe_config, basis, rank, w_down, coef, stream=None) -> None:
    _check(_lib.moe_recovery_coefs(ctypes.byref(cfg), _ptr(basis), rank, _ptr(w_down), _ptr(coef), _stream(stream)),
           "moe_recovery_coefs")


def moe_validate_plan(topk_ids, M, k, E, b, sorted_routes, block_expert, counts) -> Tuple[int, int]:
    """Host check of a plan (numpy int32 arrays).  Returns (status, reason)."""
    import numpy as np
    arrs = [np.ascontiguousarray(a, dtype=np.int32) if a is not None else None
            for a in (topk_ids, sorted_routes, block_expert, counts)]
    reason = _i32(0)
    st = _lib.moe_validate_plan(_ptr(arrs[0]), M, k, E, b, _ptr(arrs[1]), _ptr(arrs[2]), _ptr(arrs[3]),
                                ctypes.byref(reason))
    return st, reason.value


def moe_profile_enable(ctx, enable: bool = True) -> None:
    _check(_lib.moe_profile_enable(ctx, 1 if enable else 0), "moe_profile_enable")


def moe_profile_read(ctx) -> Dict[str, Tuple[float, int]]:
    """{kernel name: (total ms, launches)} of the recorded launches (synchronises)."""
    ms = (ctypes.c_double * MOE_KERNEL_COUNT)()
    n = (ctypes.c_int64 * MOE_KERNEL_COUNT)()
    _check(_lib.moe_profile_read(ctx, ms, n), "moe_profile_read")
    return {KERNELS[i]: (ms[i], n[i]) for i in range(MOE_KERNEL_COUNT) if n[i]}


# ---------------------------------------------------------------- convenience

class Layer:
    """One MoE layer bound to device tensors: owns a context and the per-call
    buffers, and runs the three calls of a step on the current stream."""

    def __init__(self, cfg: moe_config, tensors: Dict[str, object]):
        import torch
        self.cfg = cfg
        self.tensors = tensors  # keeps the borrowed weights alive
        t = tensors
        self.weights = make_weights(
            t["router_w"], t["w_down"], router_bias=t.get("router_bias"), w_gate=t.get("w_gate"),
            w_up=t.get("w_up"), chan_norm=t.get("chan_norm"),
            lr_basis=(t.get("lr_basis_gate"), t.get("lr_basis_up")),
            lr_coef=(t.get("lr_coef_gate"), t.get("lr_coef_up")),
            vq_book=(t.get("vq_book_gate"), t.get("vq_book_up")),
            vq_idx=(t.get("vq_idx_gate"), t.get("vq_idx_up")), rot_signs=t.get("rot_signs"),
            sketch=t.get("sketch"), sketch_scale=t.get("sketch_scale"), down_norm=t.get("down_norm"),
            rec_basis=t.get("rec_basis"), rec_coef=t.get("rec_coef"))
        self.ctx = moe_create(cfg, self.weights)
        dev = t["router_w"].device
        M, k = cfg.max_tokens, cfg.top_k
        cap = moe_align_capacity(M, k, cfg.E, cfg.block_b)
        i32 = torch.int32
        self.ids = torch.empty((M, k), dtype=i32, device=dev)
        self.w = torch.empty((M, k), dtype=torch.float32, device=dev)
        self.logits = torch.empty((M, cfg.E), dtype=torch.float32, device=dev)
        self.sorted_routes = torch.full((max(cap, 1),), -7, dtype=i32, device=dev)
        self.block_expert = torch.full((max(cap // cfg.block_b, 1),), -7, dtype=i32, device=dev)
        self.counts = torch.zeros(2, dtype=i32, device=dev)
        self.y = torch.empty((M, cfg.H), dtype=torch.float32, device=dev)
        self.kept = torch.empty((M, max(cfg.max_keep, 1)), dtype=i32, device=dev)

    def route(self, h, M, logits=False, stream=None):
        moe_route_topk(self.ctx, h, M, self.ids, self.w, self.logits if logits else None, stream)

    def align(self, M, ids=None, stream=None):
        moe_align_blocks(self.ctx, self.ids if ids is None else ids, M, self.sorted_routes, self.block_expert,
                         self.counts, stream)

    def forward(self, h, M, keep=0, ids=None, w=None, plan=None, stream=None, y=None):
        sr, be, ct = plan if plan is not None else (self.sorted_routes, self.block_expert, self.counts)
        moe_expert_forward(self.ctx, h, M, self.ids if ids is None else ids, self.w if w is None else w,
                           sr, be, ct, keep, self.kept if keep else None, self.y if y is None else y, stream)

    def route_align(self, h, M, logits=False, stream=None):
        moe_route_align(self.ctx, h, M, self.ids, self.w, self.logits if logits else None, self.sorted_routes,
                        self.block_expert, self.counts, stream)

    def decode_step(self, h, M, keep=0, logits=False, stream=None):
        """One decode step in one call (moe_decode_step)."""
        moe_decode_step(self.ctx, h, M, self.ids, self.w, self.logits if logits else None, self.sorted_routes,
                        self.block_expert, self.counts, keep, self.kept if keep else None, self.y, stream)
        return self.y[:M]

    def step(self, h, M, keep=0, stream=None, fused_route_align=True):
        """One decode step: routing, alignment (not needed by the channel-sparse
        mode) and the experts, as separate calls."""
        if keep:
            self.route(h, M, stream=stream)
        elif fused_route_align:
            self.route_align(h, M, stream=stream)
        else:
            self.route(h, M, stream=stream)
            self.align(M, stream=stream)
        self.forward(h, M, keep=keep, stream=stream)
        return self.y[:M]

    def close(self):
        if self.ctx:
            moe_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
