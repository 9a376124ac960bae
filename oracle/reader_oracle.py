"""fp64 CPU oracle of the channel-selection reader: ternary-sketch screening,
output-level scores, exact top-K compute and the rank-32 recovery map.

TEST INFRASTRUCTURE ONLY.  Nothing but the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or call this module; the product path
never does.  Plain and slow on purpose: every quantity comes straight from its
definition in fp64, with numpy's matmul and symmetric eigensolver as the only
library primitives.

Source: [CHANSEL] "Channel Selection for Mixture-of-Experts Decoding Needs No
Calibration Data" (a blog summary of the paper): "A Reader Built from Weights
Alone" (Fig. 6: 17.8% reads = 4.9% sketch + 12.3% exact channels + 0.6%
recovery map), "Stage 1: Screen with a Ternary Sketch", "Stage 2: Compute the
Top k Exactly with Output-Level Scores", "Stage 3: Recover Discarded Channels
with a rank-32 Map".  The page's displayed formulas -- the sketch's storage
format, Eq. 1 (the score) and Eq. 2 (the recovered output) -- are lost in the
extracted text.  Readings taken here (each restated where it is used):

  * rotation: every 128-coordinate block of a gate row, an up row and of the
    token x is multiplied by R = H_128 diag(sigma) / sqrt(128), H_128 the
    Sylvester Hadamard matrix and sigma random signs per block position, the
    same for every row and for x, so g . x = (R g) . (R x).  Computed here
    unnormalised, u = H_128 diag(sigma) g, by the fast transform's butterflies
    in fp64 (exact for bf16 rows and fp32 x of ordinary range), and the 1/128
    of (R g) . (R x) = (u . x'') / 128 folded into the stored scale;
  * ternary code of a rotated block u: the threshold rule of Ternary Weight
    Networks (Li and Liu, 2016): Delta = 0.7 * mean |u_i|, c_i = sign(u_i) if
    |u_i| > Delta else 0, scale = mean of |u_i| over the nonzero codes (0 if
    none), both sums taken by pairwise halving; stored as
    fp32(scale / 128);
  * storage: codes in base 3, five channels per byte (digit c + 1, channel
    5 g + m weighted by 3^m), coordinate-major -- for every (expert,
    projection, block, coordinate) one row of ceil(I / 5) bytes over the
    channels, padded with zero bytes to a multiple of 16 -- so that reading
    only some coordinates reads only their rows; at I = 768 that is 26.7 code
    bytes plus a 4-byte scale per 128-coordinate block of a channel, the
    page's "about 30 bytes" (about 7% of the bf16 weights);
  * partial scan: per block the 80 coordinates with the largest |x''_i|
    (ties to the lower coordinate); x'' exact as above, so the decision is
    the same in any implementation that computes it exactly;
  * estimate: g_hat_j = sum over blocks of scale_j,blk * sum over the
    scanned i of c_j,i x''_i (so g_hat_j = g_j . x when the sketch is exact
    and the scan full);
  * score (Eq. 1): w_s * ||d_j|| * |SiLU(g_hat_j) * v_hat_j|, w_s the route's
    affinity (fp32) and ||d_j|| the down column's norm (fp32); the K best of
    all (slot, channel) candidates of the token are kept, ties broken by
    (expert id, channel, slot) ascending;
  * recovered output (Eq. 2): y = sum over kept of w_s a_j d_j
    + U sum over dropped of w_s p_hat_j b_j, with p_hat_j = SiLU(g_hat_j)
    v_hat_j, U the top-32 left singular vectors of the layer's stacked down
    columns (eigenvectors of sum_j d_j d_j^T for its 32 largest eigenvalues,
    each column's largest-magnitude entry made positive) and b_j = U^T d_j
    stored in bf16.

Parity status: pinned by CPU tests (the fast transform against the dense
Sylvester matrix, orthogonality, hand-derived codes, scales and bytes, the
exact-sketch / full-scan limit equal to the exact activations, all-kept equal
to dense, brute-force selection, rank = H recovery exact, the basis against an
independent singular value decomposition, the page's byte figures).
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np

from .moe_oracle import F64, bf16_to_f64, channel_sparse_forward, silu

BLOCK = 128            # rotation block (coordinates)
SCAN = 80              # coordinates scanned per block
TWN_RATIO = 0.7        # ternary threshold, as a fraction of the mean magnitude
TRITS_PER_BYTE = 5     # 3^5 = 243 <= 256
RECOVERY_RANK = 32


# ----------------------------------------------------------------------------
# Rotation (Stage 1)
# ----------------------------------------------------------------------------

def hadamard(n: int) -> np.ndarray:
    """Sylvester's Hadamard matrix: H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    h = np.ones((1, 1), F64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    assert h.shape[0] == n, "n must be a power of two"
    return h


def fwht(v: np.ndarray) -> np.ndarray:
    """H_n v along the last axis by the fast transform: strides 1, 2, 4, ...,
    each pair (a, b) at distance `stride` inside a group of 2 * stride becomes
    (a + b, a - b).  fp64."""
    a = np.array(v, F64, copy=True)
    n = a.shape[-1]
    h = 1
    while h < n:
        b = a.reshape(a.shape[:-1] + (n // (2 * h), 2, h))
        x, y = b[..., 0, :].copy(), b[..., 1, :].copy()
        b[..., 0, :] = x + y
        b[..., 1, :] = x - y
        a = b.reshape(a.shape)
        h *= 2
    return a


def rotate(v: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """Unnormalised rotation of the blocks of v [..., H]: per block,
    u = H_128 diag(sigma_blk) v_blk.  Returns [..., H / 128, 128] fp64."""
    v = np.asarray(v, F64)
    nb = v.shape[-1] // BLOCK
    blocks = v.reshape(v.shape[:-1] + (nb, BLOCK)) * np.asarray(signs, F64).reshape(nb, BLOCK)
    return fwht(blocks)


# ----------------------------------------------------------------------------
# Ternary sketch (Stage 1; storage format lost -- reading in the header)
# ----------------------------------------------------------------------------

def pair_sum(a: np.ndarray) -> np.ndarray:
    """Sum along the last axis (a power of two) by pairwise halving: adjacent
    elements first, then adjacent pairs, and so on (a fixed order, so the
    ternary threshold below is the same in any implementation of it)."""
    a = np.asarray(a, F64)
    while a.shape[-1] > 1:
        a = a[..., 0::2] + a[..., 1::2]
    return a[..., 0]


def ternary_code(u: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Ternary Weight Networks code of each rotated block (last axis, 128):
    Delta = 0.7 * (sum |u_i|) / 128, c_i = sign(u_i) for |u_i| > Delta else
    0, scale = (sum of |u_i| over the nonzero codes) / (their count), 0 if
    none; sums by pairwise halving.  Returns codes int8 and the stored scale
    fp32(scale / 128)."""
    a = np.abs(np.asarray(u, F64))
    total = pair_sum(a)
    delta = TWN_RATIO * (total / BLOCK)
    nz = a > delta[..., None]
    codes = np.where(nz, np.sign(u), 0).astype(np.int8)
    cnt = nz.sum(axis=-1)
    snz = pair_sum(np.where(nz, a, 0.0))
    scale = np.where(cnt > 0, snz / np.maximum(cnt, 1), 0.0)
    return codes, (scale / BLOCK).astype(np.float32)


def sketch_expert(w_rows: np.ndarray, signs: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Sketch of one expert's gate or up rows (bf16 [I][H]): codes int8
    [H/128][128][I] (block, coordinate, channel) and stored scales fp32
    [H/128][I]."""
    u = rotate(bf16_to_f64(w_rows), signs)           # [I][nb][128]
    codes, scale = ternary_code(u)                   # [I][nb][128], [I][nb]
    return np.ascontiguousarray(codes.transpose(1, 2, 0)), np.ascontiguousarray(scale.T)


def sketch_row_bytes(I: int) -> int:
    """Bytes of one coordinate row: ceil(I / 5), padded to a multiple of 16."""
    g = -(-I // TRITS_PER_BYTE)
    return -(-g // 16) * 16


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Base-3 rows of codes [..., I] (values -1, 0, 1): byte g holds channels
    5g .. 5g + 4 as sum_m (c + 1) 3^m (channels past I count as code 0);
    zero padding to sketch_row_bytes(I)."""
    I = codes.shape[-1]
    ng = -(-I // TRITS_PER_BYTE)
    dig = np.ones(codes.shape[:-1] + (ng * TRITS_PER_BYTE,), np.int64)
    dig[..., :I] = np.asarray(codes, np.int64) + 1
    dig = dig.reshape(codes.shape[:-1] + (ng, TRITS_PER_BYTE))
    val = (dig * (3 ** np.arange(TRITS_PER_BYTE))).sum(axis=-1)
    out = np.zeros(codes.shape[:-1] + (sketch_row_bytes(I),), np.uint8)
    out[..., :ng] = val
    return out


def unpack_codes(rows: np.ndarray, I: int) -> np.ndarray:
    """Inverse of pack_codes (used to check the packing)."""
    ng = -(-I // TRITS_PER_BYTE)
    v = np.asarray(rows[..., :ng], np.int64)
    dig = np.stack([(v // 3 ** m) % 3 for m in range(TRITS_PER_BYTE)], axis=-1)
    return (dig.reshape(rows.shape[:-1] + (ng * TRITS_PER_BYTE,))[..., :I] - 1).astype(np.int8)


# ----------------------------------------------------------------------------
# Partial scan and estimates (Stage 1)
# ----------------------------------------------------------------------------

def scan_mask(xr: np.ndarray, keep: int = SCAN) -> np.ndarray:
    """Per block (last axis), the `keep` coordinates of largest |x''|, ties to
    the lower coordinate.  bool [nb][128]."""
    nb, n = xr.shape
    mask = np.zeros((nb, n), bool)
    for b in range(nb):
        order = sorted(range(n), key=lambda i: (-abs(xr[b, i]), i))
        mask[b, order[:keep]] = True
    return mask


def sketch_estimate(codes: np.ndarray, scale: np.ndarray, xr: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """g_hat_j = sum over blocks of scale[blk][j] * sum over scanned i of
    codes[blk][i][j] * x''[blk][i].  fp64 [I]."""
    part = np.einsum("bij,bi->bj", np.asarray(codes, F64), np.where(mask, xr, 0.0))
    return (np.asarray(scale, F64) * part).sum(axis=0)


def down_norms(w_down_e: np.ndarray) -> np.ndarray:
    """||d_j|| of one expert's down columns (bf16 [I][H]), fp64 rounded once to fp32."""
    return np.sqrt((bf16_to_f64(w_down_e) ** 2).sum(axis=1)).astype(np.float32)


# ----------------------------------------------------------------------------
# Output-level scores and the exact top K (Stage 2)
# ----------------------------------------------------------------------------

def reader_scores(aff_f32: np.ndarray, g_hat: np.ndarray, v_hat: np.ndarray, dnorm: np.ndarray) -> np.ndarray:
    """Score of candidate (slot s, channel j): w_s * ||d_j|| * |SiLU(g_hat) v_hat|
    (fp64; aff_f32 [k], g_hat/v_hat [k][I], dnorm [k][I] of the routed experts)."""
    a = np.asarray(aff_f32, np.float32).astype(F64)[:, None]
    return a * np.asarray(dnorm, np.float32).astype(F64) * np.abs(silu(g_hat) * v_hat)


def select_top(scores: np.ndarray, ids: np.ndarray, K: int) -> np.ndarray:
    """The K best candidates (s, j) of one token by score, ties to (expert id,
    channel, slot) ascending; returned as s * I + j, ascending."""
    k, I = scores.shape
    cands = sorted(((-scores[s, j], int(ids[s]), j, s) for s in range(k) for j in range(I)))
    return np.array(sorted(s * I + j for (_, _, j, s) in cands[:K]), np.int64)


# ----------------------------------------------------------------------------
# Rank-32 recovery map (Stage 3)
# ----------------------------------------------------------------------------

def recovery_basis(w_down: np.ndarray, rank: int = RECOVERY_RANK) -> np.ndarray:
    """U [H][rank]: eigenvectors of G = sum over all channels of all experts of
    d_j d_j^T (the left singular vectors of the stacked down columns) for the
    `rank` largest eigenvalues, in decreasing order, each column's entry of
    largest magnitude made positive.  w_down bf16 [E][I][H]."""
    E, I, H = w_down.shape
    G = np.zeros((H, H), F64)
    for e in range(E):
        d = bf16_to_f64(w_down[e])
        G += d.T @ d
    lam, vec = np.linalg.eigh(G)
    U = vec[:, ::-1][:, :rank].copy()
    for c in range(rank):
        i = int(np.argmax(np.abs(U[:, c])))
        if U[i, c] < 0:
            U[:, c] = -U[:, c]
    return U


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to fp32 (nearest even), then to bf16 (nearest even); bit patterns."""
    u = np.asarray(x, F64).astype(np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def recovery_coefs(U: np.ndarray, w_down_e: np.ndarray) -> np.ndarray:
    """b_j = U^T d_j for one expert's channels, stored bf16 [I][rank]."""
    return f64_to_bf16_bits(bf16_to_f64(w_down_e) @ np.asarray(U, F64))


def recovery_term(U: np.ndarray, b_bf16: np.ndarray, aff: np.ndarray, p_hat: np.ndarray,
                  dropped: np.ndarray) -> np.ndarray:
    """U sum over dropped (s, j) of w_s p_hat[s][j] b[s][j] (one token).
    b_bf16 [k][I][rank] (the routed experts' coefficients; bf16 patterns, or
    fp64 values for the unrounded map), dropped bool [k][I]."""
    coef = np.asarray(aff, F64)[:, None] * np.where(dropped, p_hat, 0.0)     # [k][I]
    b = bf16_to_f64(b_bf16) if np.asarray(b_bf16).dtype == np.uint16 else np.asarray(b_bf16, F64)
    r = np.einsum("sj,sjr->r", coef, b)
    return np.asarray(U, F64) @ r


# ----------------------------------------------------------------------------
# One token through the reader
# ----------------------------------------------------------------------------

def reader_step(h_t: np.ndarray, ids: np.ndarray, aff_f32: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
                w_down: np.ndarray, signs: np.ndarray, K: int, scan: int = SCAN,
                recovery: Optional[Tuple[np.ndarray, np.ndarray]] = None,
                sketches: Optional[Dict[int, tuple]] = None) -> Dict[str, np.ndarray]:
    """Screen -> score -> top K -> exact compute (-> recovery) for one token
    with routing (ids [k], fp32 affinities [k]).  `recovery` = (U, b bf16
    [E][I][rank]); `sketches` may hold precomputed (codes_g, scale_g, codes_u,
    scale_u, dnorm) per expert."""
    k = len(ids)
    I = w_gate.shape[1]
    xr = rotate(np.asarray(h_t, F64)[None, :], signs)[0]
    mask = scan_mask(xr, scan)
    g_hat = np.zeros((k, I))
    v_hat = np.zeros((k, I))
    dn = np.zeros((k, I), np.float32)
    for s in range(k):
        e = int(ids[s])
        if sketches is not None and e in sketches:
            cg, sg, cu, su, dne = sketches[e]
        else:
            cg, sg = sketch_expert(w_gate[e], signs)
            cu, su = sketch_expert(w_up[e], signs)
            dne = down_norms(w_down[e])
        g_hat[s] = sketch_estimate(cg, sg, xr, mask)
        v_hat[s] = sketch_estimate(cu, su, xr, mask)
        dn[s] = dne
    scores = reader_scores(aff_f32, g_hat, v_hat, dn)
    kept = select_top(scores, ids, K)
    aff = np.asarray(aff_f32, np.float32).astype(F64)
    y = channel_sparse_forward(np.asarray(h_t)[None, :], np.asarray(ids)[None, :], aff[None, :], w_gate, w_up,
                               w_down, kept[None, :])[0]
    out = {"x_rot": xr, "mask": mask, "g_hat": g_hat, "v_hat": v_hat, "scores": scores, "kept": kept}
    if recovery is not None:
        U, b = recovery
        dropped = np.ones((k, I), bool)
        dropped.reshape(-1)[kept] = False
        p_hat = silu(g_hat) * v_hat
        y = y + recovery_term(U, np.stack([b[int(e)] for e in ids]), aff, p_hat, dropped)
        out["p_hat"] = p_hat
    out["y"] = y
    return out
