"""fp64 CPU oracle for the routed MoE decode step.

TEST INFRASTRUCTURE ONLY.  Nothing but the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or call this module; the product path
(the HIP library and its Python binding) never does, and this module imports
nothing from it.  It is deliberately plain and slow: every quantity is widened
exactly to fp64 (bf16 and fp32 inputs are exactly representable there) and
computed straight from its definition, with numpy's matmul as the only library
primitive.  There is no blocking, fusion or reordering beyond what each
definition states.

Sources (page titles; sections as numbered on each page):
  [CARDAN]  "A Multi-Engine Dataflow for MoE Decoding on Scratchpad-Based Tensor
            Accelerators" -- MoE block (background, Fig. 2), blockwise VQ (Sec. 2.3),
            hybrid VQ + low-rank weights (Sec. 3.1, Eq. 1), shared projections and
            joint accumulation (Sec. 4.2), down projection and accumulated
            summation (Sec. 4.3).
  [CHANSEL] "Channel Selection for Mixture-of-Experts Decoding Needs No Calibration
            Data" -- "Background: Channels and Retention Rules", "Stage 2: Compute
            the Top k Exactly with Output-Level Scores".
  [ROUTEBLK] "Route-Block Membership Selects Packed-AWQ Arithmetic" -- MoE alignment
            and padded blocks (Sec. 2.1), route-block membership (Sec. 3.1, Eq. 1),
            stable canonical construction (Sec. 5.3, Sec. 6).

Readings where the pages leave a step open (each is listed with its reason in
the design notes):
  * the routing affinity is the softmax over the k selected logits
    (renormalised top-k softmax); selection uses logits, ties go to the lower
    expert id, and slot order is descending logit;
  * the expert activation phi is SiLU, applied to the gate output and
    multiplied elementwise by the up output;
  * the combine adds slot outputs in slot order s = 0..k-1;
  * alignment pads each expert with the sentinel M*k, gives no block to an
    expert with no route, and skips route ids outside [0, E);
  * the channel-sparse score is the exact product of the fp32 affinity and a
    static fp32 channel norm ||g_j||*||v_j||*||d_j||, top-K across all routed
    experts, ties broken by (expert id, channel, slot) ascending;
  * VQ blocks run along the hidden dimension inside each channel's column of
    W_e (length d), and gate and up each have their own basis and code book.

Parity status: every function here is pinned by CPU tests (brute force on tiny
inputs, closed forms, special cases that reduce to library routines, and the
pages' printed sizes); none is "parity unpinned".
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns: a bf16 value is the fp32 value whose upper 16
    bits are the pattern and whose lower 16 bits are zero (exact in fp64)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(F64)


def silu(x: np.ndarray) -> np.ndarray:
    """phi(x) = x * sigmoid(x) = x / (1 + exp(-x))."""
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


# ----------------------------------------------------------------------------
# Router: logits, top-k, affinities  ([CARDAN] MoE block; [ROUTEBLK] Sec. 2.1)
# ----------------------------------------------------------------------------

def router_logits(h: np.ndarray, router_w: np.ndarray, router_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """l[t][e] = sum_i h[t][i] * Wr[i][e] (+ bias[e]).  h fp32 [M][H], Wr bf16 [H][E]."""
    l = np.asarray(h, F64) @ bf16_to_f64(router_w)
    if router_bias is not None:
        l = l + np.asarray(router_bias, F64)[None, :]
    return l


def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    """The router's M x k expert-id array: per token, repeatedly take the
    largest remaining logit (ties to the lower expert id); slot s holds the
    s-th pick, so slots are in descending logit order."""
    M, E = logits.shape
    ids = np.empty((M, k), np.int64)
    for t in range(M):
        taken = np.zeros(E, bool)
        for s in range(k):
            best = -1
            for e in range(E):
                if taken[e]:
                    continue
                if best < 0 or logits[t, e] > logits[t, best]:
                    best = e
            ids[t, s] = best
            taken[best] = True
    return ids


def affinities(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """a[t][s] = exp(l_s - l_0) / sum_{s'} exp(l_{s'} - l_0) over the selected
    logits (the softmax over all E renormalised to the top-k; the shift by the
    largest selected logit l_0 does not change the value)."""
    sel = np.take_along_axis(logits, ids, axis=1)
    ex = np.exp(sel - sel[:, :1])
    return ex / ex.sum(axis=1, keepdims=True)


def route_topk(h, router_w, k, router_bias=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    l = router_logits(h, router_w, router_bias)
    ids = topk_select(l, k)
    return ids, affinities(l, ids), l


# ----------------------------------------------------------------------------
# Alignment into padded expert blocks  ([ROUTEBLK] Sec. 2.1, Sec. 3.1, Sec. 5.3)
# ----------------------------------------------------------------------------

def align_capacity(M: int, k: int, E: int, b: int = 8) -> int:
    """Largest possible number of aligned rows: every route plus at most b-1
    pads for each expert that receives a route."""
    return M * k + min(E, M * k) * (b - 1)


def align_blocks(ids: np.ndarray, E: int, b: int = 8) -> Dict[str, np.ndarray]:
    """Canonical alignment.  Routes are the row-major flattening r = t*k + s of
    the M x k id array.  Valid routes (0 <= id < E) are grouped by expert in
    (expert id, route id) order; each expert's group is padded with the
    sentinel M*k up to a multiple of b; experts follow each other in ascending
    id; a parallel vector gives the expert of every b-row block."""
    flat = np.asarray(ids).reshape(-1)
    R = flat.size
    sentinel = R
    sorted_routes: List[int] = []
    block_expert: List[int] = []
    invalid = 0
    for r in range(R):
        if not (0 <= flat[r] < E):
            invalid += 1
    for e in range(E):
        group = [r for r in range(R) if flat[r] == e]
        if not group:
            continue
        padded = -(-len(group) // b) * b
        sorted_routes.extend(group + [sentinel] * (padded - len(group)))
        block_expert.extend([e] * (padded // b))
    return {
        "sorted_routes": np.array(sorted_routes, np.int64),
        "block_expert": np.array(block_expert, np.int64),
        "num_blocks": len(block_expert),
        "num_padded": len(sorted_routes),
        "invalid_routes": invalid,
    }


def block_membership(sorted_routes: np.ndarray, block_expert: np.ndarray, sentinel: int, b: int = 8):
    """Route-block membership ([ROUTEBLK] Sec. 3.1, Eq. 1): the ordered sequence of
    (expert e, expert-local block j, sorted valid routes in that block), pads
    excluded and order inside a block ignored."""
    out = []
    local = {}
    for blk, e in enumerate(block_expert):
        e = int(e)
        j = local.get(e, 0)
        local[e] = j + 1
        rows = [int(r) for r in sorted_routes[blk * b:(blk + 1) * b] if int(r) != sentinel]
        out.append((e, j, tuple(sorted(rows))))
    return out


# ----------------------------------------------------------------------------
# Dense experts and the combine  ([CARDAN] MoE block, Sec. 4.3; [CHANSEL] Background)
# Weight layout: gate, up and down are [E][I][H]; row j of gate/up is channel j's
# gate/up row and row j of down is channel j's down column (transposed at load).
# ----------------------------------------------------------------------------

def expert_intermediate(h_t: np.ndarray, w_gate_e: np.ndarray, w_up_e: np.ndarray) -> np.ndarray:
    """p = phi(G h) * (V h) for one expert and one token (fp64 [I])."""
    x = np.asarray(h_t, F64)
    g = bf16_to_f64(w_gate_e) @ x
    u = bf16_to_f64(w_up_e) @ x
    return silu(g) * u


def expert_down(p: np.ndarray, w_down_rows: np.ndarray) -> np.ndarray:
    """y_e = W_down^T p: the sum over channels j of p_j times channel j's down column."""
    return bf16_to_f64(w_down_rows).T @ p


def dense_forward(h, ids, aff, w_gate, w_up, w_down) -> np.ndarray:
    """y[t] = sum_{s=0..k-1} a[t][s] * W_down,e(phi(W_gate,e h_t) * W_up,e h_t), e = ids[t][s]."""
    M, k = ids.shape
    H = w_down.shape[2]
    y_route = np.zeros((M, k, H), F64)
    for e in sorted(set(int(v) for v in ids.reshape(-1))):
        if not (0 <= e < w_gate.shape[0]):
            continue
        for t, s in zip(*np.nonzero(ids == e)):
            p = expert_intermediate(h[t], w_gate[e], w_up[e])
            y_route[t, s] = expert_down(p, w_down[e])
    return combine(y_route, np.asarray(aff, F64), ids, w_gate.shape[0])


def combine(y_route: np.ndarray, aff: np.ndarray, ids: np.ndarray, E: int) -> np.ndarray:
    """Accumulated summation in slot order; routes with an id outside [0, E) add nothing."""
    M, k, H = y_route.shape
    y = np.zeros((M, H), F64)
    for t in range(M):
        for s in range(k):
            if 0 <= ids[t, s] < E:
                y[t] += aff[t, s] * y_route[t, s]
    return y


# ----------------------------------------------------------------------------
# Channel-sparse reads  ([CHANSEL] Background; Stage 2)
# ----------------------------------------------------------------------------

def channel_norms(w_gate, w_up, w_down, experts: Optional[Sequence[int]] = None) -> np.ndarray:
    """Static per-channel weight norm n[e][j] = ||g_j|| * ||v_j|| * ||d_j||, computed
    in fp64 and rounded once to fp32 (a load-time quantity).  Experts not listed stay 0."""
    E, I, _ = w_gate.shape
    n = np.zeros((E, I), np.float32)
    ex = range(E) if experts is None else experts
    for e in ex:
        ng = np.sqrt((bf16_to_f64(w_gate[e]) ** 2).sum(axis=1))
        nv = np.sqrt((bf16_to_f64(w_up[e]) ** 2).sum(axis=1))
        nd = np.sqrt((bf16_to_f64(w_down[e]) ** 2).sum(axis=1))
        n[e] = (ng * nv * nd).astype(np.float32)
    return n


def channel_select(aff_f32: np.ndarray, ids: np.ndarray, norms: np.ndarray, K: int) -> np.ndarray:
    """Top-K channels across all routed experts of each token.

    Candidates are (slot s, channel j).  score = a_s * n[e_s][j], the exact fp64
    product of two fp32 numbers.  Candidates are ranked by score (descending),
    then expert id, then channel (ascending); the first K are kept.  The kept
    set is returned per token as s*I + j in ascending order ([M][K] int64)."""
    M, k = ids.shape
    I = norms.shape[1]
    out = np.empty((M, K), np.int64)
    for t in range(M):
        cands = []
        for s in range(k):
            e = int(ids[t, s])
            a = F64(np.float32(aff_f32[t, s]))
            for j in range(I):
                cands.append((-(a * F64(norms[e, j])), e, j, s))
        cands.sort()
        kept = sorted(s * I + j for (_, _, j, s) in cands[:K])
        out[t] = kept
    return out


def channel_sparse_forward(h, ids, aff, w_gate, w_up, w_down, kept: np.ndarray) -> np.ndarray:
    """y[t] = sum_s a[t][s] * sum_{j kept for (t, s)} p_j * d_j: kept channels read
    exactly, dropped channels contribute nothing (no recovery term)."""
    M, k = ids.shape
    I = w_gate.shape[1]
    H = w_down.shape[2]
    y_route = np.zeros((M, k, H), F64)
    for t in range(M):
        for s in range(k):
            e = int(ids[t, s])
            js = np.array([q % I for q in kept[t] if q // I == s], np.int64)
            if js.size == 0:
                continue
            x = np.asarray(h[t], F64)
            g = bf16_to_f64(w_gate[e][js]) @ x
            u = bf16_to_f64(w_up[e][js]) @ x
            p = silu(g) * u
            y_route[t, s] = expert_down(p, w_down[e][js])
    return combine(y_route, np.asarray(aff, F64), ids, w_gate.shape[0])


# ----------------------------------------------------------------------------
# VQ + low-rank gate/up weights  ([CARDAN] Sec. 2.3, Sec. 3.1 Eq. 1, Sec. 4.2)
# W_e (H x I) ~= D C_e + Q_B(J_e); stored channel-major here, so the
# reconstruction of channel j is What[j][i] = sum_rho D[i][rho] C_e[j][rho]
# + B[J_e[j][i // d]][i % d].
# ----------------------------------------------------------------------------

def vq_reconstruct(D: np.ndarray, C_e: np.ndarray, B: np.ndarray, J_e: np.ndarray) -> np.ndarray:
    """Materialise one expert's gate or up weights, channel-major [I][H] fp64."""
    Dd = bf16_to_f64(D)                  # [H][r]
    Cd = bf16_to_f64(C_e)                # [I][r]
    Bd = bf16_to_f64(B)                  # [K][d]
    I = C_e.shape[0]
    H = D.shape[0]
    d = B.shape[1]
    low_rank = Cd @ Dd.T                 # [I][H]
    vq = Bd[np.asarray(J_e, np.int64)]   # [I][H/d][d]: code word of every length-d block
    return low_rank + vq.reshape(I, H)


def vqlr_project(h_t: np.ndarray, D, C_e, B, J_e) -> np.ndarray:
    """o[j] = sum_i What[j][i] h[i], from the materialised reconstruction."""
    return vq_reconstruct(D, C_e, B, J_e) @ np.asarray(h_t, F64)


def shared_projections(h_t: np.ndarray, D: np.ndarray, B: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Routing-independent work done once per token: z = D^T h (rank r) and the
    projection code book T[b][c] = h_b . B_c for every length-d block h_b of h."""
    x = np.asarray(h_t, F64)
    d = B.shape[1]
    z = bf16_to_f64(D).T @ x
    T = x.reshape(-1, d) @ bf16_to_f64(B).T      # [H/d][K]
    return z, T


def vqlr_project_shared(h_t, D, C_e, B, J_e) -> np.ndarray:
    """o[j] = sum_rho C_e[j][rho] z[rho] + sum_b T[b][J_e[j][b]] (selection from T
    instead of the weight code book; same value as vqlr_project)."""
    z, T = shared_projections(h_t, D, B)
    J = np.asarray(J_e, np.int64)
    nb = J.shape[1]
    vq = T[np.arange(nb)[None, :], J].sum(axis=1)
    return bf16_to_f64(C_e) @ z + vq


def vqlr_forward(h, ids, aff, vq: Dict[str, np.ndarray], w_down) -> np.ndarray:
    """Gate/up from the VQ + low-rank format, down projection dense bf16."""
    M, k = ids.shape
    E = w_down.shape[0]
    H = w_down.shape[2]
    y_route = np.zeros((M, k, H), F64)
    for e in sorted(set(int(v) for v in ids.reshape(-1))):
        if not (0 <= e < E):
            continue
        Wg = vq_reconstruct(vq["lr_basis_gate"], vq["lr_coef_gate"][e], vq["vq_book_gate"], vq["vq_idx_gate"][e])
        Wu = vq_reconstruct(vq["lr_basis_up"], vq["lr_coef_up"][e], vq["vq_book_up"], vq["vq_idx_up"][e])
        for t, s in zip(*np.nonzero(ids == e)):
            x = np.asarray(h[t], F64)
            p = silu(Wg @ x) * (Wu @ x)
            y_route[t, s] = expert_down(p, w_down[e])
    return combine(y_route, np.asarray(aff, F64), ids, E)


# ----------------------------------------------------------------------------
# One whole step
# ----------------------------------------------------------------------------

def vq_storage_bits_per_weight(d: int, r: int, K: int, H: int, I: int, E: int) -> float:
    """Bits stored per original gate or up weight by the VQ + low-rank format
    ([CARDAN] Sec. 5.4; the formula is lost in the page's text, so this is the
    count of the format's own parts): an 8-bit code index per block of d
    weights, an expert-private bf16 coefficient matrix C_e of I x r entries
    over the I x H weights of one expert, and the layer-shared bf16 basis D
    (H x r) and code book B (K x d) amortised over the E experts."""
    return 8.0 / d + 16.0 * r / H + (16.0 * H * r + 16.0 * K * d) / (E * H * I)


def vq_private_bytes_per_projection(d: int, r: int, H: int, I: int) -> int:
    """Expert-private bytes of one projection: the uint8 index map J_e
    (I x H/d) and the bf16 coefficients C_e (I x r)."""
    return I * (H // d) + I * r * 2


def moe_step(inp: Dict[str, np.ndarray], k: int, keep: int = 0, b: int = 8,
             aff_f32_for_selection: Optional[np.ndarray] = None,
             norms: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Router -> top-k -> alignment -> experts -> combine for one layer.

    For the channel-sparse path `norms` (fp32 [E][I]) must be given, and the
    selection uses `aff_f32_for_selection` when given (else the fp64 affinities
    rounded to fp32)."""
    ids, aff, logits = route_topk(inp["h"], inp["router_w"], k, inp.get("router_bias"))
    E = inp["router_w"].shape[1]
    al = align_blocks(ids, E, b)
    out = {"ids": ids, "aff": aff, "logits": logits, **al}
    if "vq_idx_gate" in inp:
        out["y"] = vqlr_forward(inp["h"], ids, aff, inp, inp["w_down"])
    elif keep:
        a32 = aff.astype(np.float32) if aff_f32_for_selection is None else aff_f32_for_selection
        kept = channel_select(a32, ids, norms, keep)
        out["kept"] = kept
        out["y"] = channel_sparse_forward(inp["h"], ids, aff, inp["w_gate"], inp["w_up"], inp["w_down"], kept)
    else:
        out["y"] = dense_forward(inp["h"], ids, aff, inp["w_gate"], inp["w_up"], inp["w_down"])
    return out
