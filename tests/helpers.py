"""Shared helpers of the test suite: device upload, tolerance and the
certified-margin rule for comparing top-k decisions made in different
precisions."""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

import oracle as O

REL_L2_TOL = 1e-3        # ||y - y_ref|| / ||y_ref||
MAX_ABS_FRAC = 5e-3      # max|y - y_ref| <= MAX_ABS_FRAC * max|y_ref|
U32 = 2.0 ** -24         # unit roundoff of fp32


def router_depth(H: int, E: int) -> int:
    """Upper bound on the summation depth of a router logit, as documented in
    moe.h: 4 rows per thread, rpt/8 row groups in order per lane, a 3-level
    butterfly over 8 lanes, the row slices in order, one bias add."""
    c = 32 if E >= 32 else (16 if E >= 16 else 8)
    rpt = 2048 // c
    return 4 + rpt // 8 + 3 + math.ceil(H / (4 * rpt)) + 1


def logit_error_bound(h: np.ndarray, router_w: np.ndarray, H: int, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Rigorous bound on |fp32 logit - exact logit|: gamma_n * sum of |terms|
    (the products h_i w_ie and the bias)."""
    n = router_depth(H, router_w.shape[1])
    gamma = n * U32 / (1 - n * U32)
    s = np.abs(np.asarray(h, np.float64)) @ np.abs(O.bf16_to_f64(router_w))
    if bias is not None:
        s = s + np.abs(np.asarray(bias, np.float64))[None, :]
    return gamma * s + 1e-30


def certified_tokens(ref_logits: np.ndarray, bound: np.ndarray, k: int) -> np.ndarray:
    """Tokens whose ordered top-k is decided by more than twice the error bound
    (every gap among the k+1 largest exceeds 2 * max bound of the token)."""
    M, E = ref_logits.shape
    ok = np.ones(M, bool)
    for t in range(M):
        srt = np.sort(ref_logits[t])[::-1][: min(k + 1, E)]
        gaps = -np.diff(srt)
        ok[t] = bool(np.all(gaps > 2 * bound[t].max()))
    return ok


def check_close(y: np.ndarray, ref: np.ndarray, what: str = "y") -> Dict[str, float]:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.all(np.isfinite(y)), "%s has non-finite values" % what
    den = np.linalg.norm(ref)
    rel = float(np.linalg.norm(y - ref) / den) if den > 0 else float(np.linalg.norm(y))
    mx = float(np.abs(y - ref).max()) if y.size else 0.0
    lim = MAX_ABS_FRAC * float(np.abs(ref).max()) if ref.size else 0.0
    assert rel <= REL_L2_TOL, "%s rel-L2 %.3e > %.1e" % (what, rel, REL_L2_TOL)
    if den > 0:
        assert mx <= lim, "%s max-abs %.3e > %.3e" % (what, mx, lim)
    else:
        assert mx == 0.0
    return {"rel_l2": rel, "max_abs": mx}


def to_dev(a: Optional[np.ndarray], device="cuda"):
    """numpy -> torch device tensor with the same bytes (bf16 bits as int16)."""
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def upload_layer(inp: Dict[str, np.ndarray], device="cuda") -> Dict[str, object]:
    return {k: to_dev(v, device) for k, v in inp.items() if v is not None and k != "h"}
