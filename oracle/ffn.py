"""fp64 definitions of every step of the MoE / SwiGLU FFN hot path.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by the tests,
the smoke check and the benchmark's CPU-baseline leg, never by the GPU path.

Orientation. Weights follow the pages' notation: a linear layer is
``Y = X W`` with ``W`` of shape ``[d_in, d_out]`` ([P1] 张量并行和通信). The
router weight is ``W_r`` of shape ``[E, d]`` because the pages write
``z = x W_r^T`` ([P1] MoE Router 过程). Callers holding weights in another
storage order pass transposed views; a transpose is not arithmetic.

Readings of points the pages leave open are marked READING and are the same
ones the design document lists.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# exact decoding of stored bit patterns
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly.

    A bf16 value is the upper half of the float32 with the same sign, exponent
    and leading 7 mantissa bits, so shifting the 16 bits into the top of a
    32-bit word gives that float32 exactly; float32 -> float64 is exact.
    """
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3fn_decode_table() -> np.ndarray:
    """Value of every one of the 256 OCP FP8 E4M3FN codes, as float64.

    Layout: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits. Exponent
    field 0 encodes subnormals m/8 * 2^(1-7); the code S.1111.111 is NaN; there
    is no infinity, so exponent field 15 with m < 7 is an ordinary normal number
    (largest 448). Block fp8 weights are named by [P5] (量化支持, blockfp8); the
    E4M3FN format itself is READING R21.
    """
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            out[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_E4M3FN = e4m3fn_decode_table()


def fp8_bits_to_f64(bits) -> np.ndarray:
    """E4M3FN codes (uint8) -> float64 via the decode table."""
    return _E4M3FN[np.asarray(bits, dtype=np.uint8)]


def dequant_block_fp8(q_bits, scales, block: int = 128) -> np.ndarray:
    """Block-scaled fp8 weight -> float64: ``w[i, j] = q[i, j] * scale[i//128, j//128]``.

    READING R21: one float32 scale per 128x128 block of the weight's index
    space; the dequantised weight is the exact product code value x scale.
    """
    q = fp8_bits_to_f64(q_bits)
    s = np.asarray(scales, dtype=np.float64)
    rows, cols = q.shape
    assert rows % block == 0 and cols % block == 0
    assert s.shape == (rows // block, cols // block)
    # element (i, j) sits in block (i // block, j // block): view q as
    # [row block, row in block, column block, column in block] and multiply
    # each element by its block's scale
    qb = q.reshape(rows // block, block, cols // block, block)
    return (qb * s[:, None, :, None]).reshape(rows, cols)


# ---------------------------------------------------------------------------
# RMSNorm  ([P1] Norm&Residual: V = RMSNorm_ffn(R); RMSNorm equation)
# ---------------------------------------------------------------------------


def rmsnorm(x, gamma, eps: float = 1e-5) -> np.ndarray:
    """``y[t, j] = gamma_j * x[t, j] / sqrt(mean_k x[t, k]^2 + eps)``.

    [P1] Norm&Residual, RMSNorm equation: the mean square runs over the whole
    hidden vector (the page's 1/4096 sum over k = 0..4095 for d = 4096; READING
    R1 generalises to 1/d) and eps = 1e-5 sits inside the square root, added to
    the mean square (R2). gamma multiplies after normalising (R3).
    """
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return g * x / np.sqrt(ms + eps)


# ---------------------------------------------------------------------------
# gated MLP  ([P1] 实际 MLP 计算策略)
# ---------------------------------------------------------------------------


def sigmoid(z) -> np.ndarray:
    """Logistic function 1 / (1 + e^-z) (READING R5: the textbook definition)."""
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def silu(a) -> np.ndarray:
    """SiLU(a) = a * sigmoid(a) (READING R5)."""
    a = np.asarray(a, dtype=np.float64)
    return a * sigmoid(a)


def swiglu(x, w_gate, w_up, w_down) -> np.ndarray:
    """``Y = (SiLU(X W_gate) ⊙ X W_up) W_down``.

    [P1] 实际 MLP 计算策略, gated MLP equation: SiLU acts on the gate branch
    only, the product with the up branch is elementwise, then the down
    projection. Shapes: x [m, d], w_gate and w_up [d, f], w_down [f, d].
    """
    x = np.asarray(x, dtype=np.float64)
    g = x @ np.asarray(w_gate, dtype=np.float64)
    u = x @ np.asarray(w_up, dtype=np.float64)
    h = silu(g) * u
    return h @ np.asarray(w_down, dtype=np.float64)


# ---------------------------------------------------------------------------
# tensor-parallel shards  ([P1] 列并行 / 行并行; [P3] Outer Dim / Inner Dim;
# [P2] §1.1 and §1.4; [P4] column/row-parallel MLP)
# ---------------------------------------------------------------------------


def _block(n: int, p: int, i: int) -> slice:
    """Block i of p contiguous, equal blocks of range(n) (READING R8)."""
    assert p >= 1 and 0 <= i < p and n % p == 0, (n, p, i)
    w = n // p
    return slice(i * w, (i + 1) * w)


def column_parallel(x, w, p: int, i: int) -> np.ndarray:
    """Column shard ``Y_i = X W_i`` where ``W = [W_0 ... W_{p-1}]`` split by columns.

    [P1] 列并行 equation; [P3] Outer Dim (each device k computes
    ``C_k = A x B_k``; the All-Gather concatenates the C_k along columns).
    """
    w = np.asarray(w, dtype=np.float64)
    return np.asarray(x, dtype=np.float64) @ w[:, _block(w.shape[1], p, i)]


def row_parallel_partial(x, w, p: int, i: int) -> np.ndarray:
    """Row shard partial ``X_i W_i`` with X split by columns and W by rows.

    [P1] 行并行 equations (each ``X_i W_i`` has the full output shape but is
    only part of the sum ``Y = Σ_i X_i W_i``); [P3] Inner Dim.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    blk = _block(w.shape[0], p, i)
    return x[:, blk] @ w[blk, :]


def tp_shard_mlp(x, w_gate, w_up, w_down, p: int, i: int) -> np.ndarray:
    """Partial output of TP shard i of p for the gated MLP.

    [P1] 实际 MLP 计算策略: W_gate and W_up are column-parallel, SiLU and the
    pointwise product need no communication, and the per-rank shard of the
    intermediate is exactly the X split that a row-parallel W_down needs; each
    rank's output is a full-shape partial sum. [P2] §1.4 (B column split + C
    row split); [P4] column-parallel first layer with
    ``W1[:, i*(f//N):(i+1)*(f//N)]`` and row-parallel second layer. Shard
    blocks are contiguous and equal (READING R8). The sum over i of the
    returned partials is swiglu(x, w_gate, w_up, w_down).
    """
    w_gate = np.asarray(w_gate, dtype=np.float64)
    w_up = np.asarray(w_up, dtype=np.float64)
    w_down = np.asarray(w_down, dtype=np.float64)
    f = w_gate.shape[1]
    blk = _block(f, p, i)
    return swiglu(x, w_gate[:, blk], w_up[:, blk], w_down[blk, :])


# ---------------------------------------------------------------------------
# MoE router  ([P1] 专家并行 / MoE Router 过程)
# ---------------------------------------------------------------------------


def route_weights(s, idx) -> np.ndarray:
    """``w_i = s_i / Σ_{j∈I} s_j`` for i in I, over UNBIASED scores.

    [P1] MoE Router 过程, router equation (the bias takes no part in the
    weights). READING R15: no extra scaling factor and no epsilon in the sum
    (s lies in (0, 1), so the sum of 8 scores is positive).
    """
    s = np.asarray(s, dtype=np.float64)
    idx = np.asarray(idx)
    sel = np.take_along_axis(s, idx, axis=-1)
    return sel / sel.sum(axis=-1, keepdims=True)


def route(x, w_r, bias, k: int = 8):
    """Sigmoid-with-bias top-k router.

    [P1] MoE Router 过程, router equation:
    ``z = x W_r^T``, ``s = sigmoid(z)``, ``I = Top8(s + b)``,
    ``w_i = s_i / Σ_{j∈I} s_j``.

    READINGS: the bias is added after the sigmoid (R12, as the equation
    writes ``s + b``); ties in ``s + b`` go to the lower expert index (R13);
    I is a set, so its ids are returned in ascending order with the weights
    aligned (R14).

    Returns ``(idx [T,k] int64 ascending, w [T,k] f64, s [T,E] f64,
    key [T,E] f64, gap [T] f64)`` where ``gap`` is key_(k) - key_(k+1) in the
    descending (key, then ascending id) order; +inf when E == k.
    """
    x = np.asarray(x, dtype=np.float64)
    w_r = np.asarray(w_r, dtype=np.float64)
    b = np.asarray(bias, dtype=np.float64)
    T = x.shape[0]
    E = w_r.shape[0]
    assert 1 <= k <= E
    z = x @ w_r.T
    s = sigmoid(z)
    key = s + b[None, :]
    ids = np.broadcast_to(np.arange(E), key.shape)
    # np.lexsort sorts by the LAST key first: primary -key (descending key),
    # secondary expert id (ascending) -> ties go to the lower index.
    order = np.lexsort((ids, -key), axis=-1)
    top = order[:, :k]
    idx = np.sort(top, axis=-1)
    w = route_weights(s, idx)
    rows = np.arange(T)
    if E > k:
        gap = key[rows, order[:, k - 1]] - key[rows, order[:, k]]
    else:
        gap = np.full(T, np.inf)
    return idx.astype(np.int64), w, s, key, gap


# ---------------------------------------------------------------------------
# token permutation  ([P5] token_permutation; tokens contiguous by expert id;
# [P1] EP 路径: grouped GEMM over the rank's local experts)
# ---------------------------------------------------------------------------


def permute(idx, e_begin: int, e_count: int, x=None):
    """Stable counting sort of the routing slots (t, j) by expert.

    Only experts in the local range ``[e_begin, e_begin + e_count)`` are kept
    ([P1] EP 路径: each rank runs its own experts; READING R17 for the range).
    Within an expert, slots keep token order (stable sort, READING R19), the
    layout is contiguous by expert id with no padding ([P5] experts: input
    tokens laid out contiguously by expert id).

    Returns ``(counts [e_count], offsets [e_count+1], src_token [S],
    inv_pos [T,k], x_perm [S,d] or None)``: ``src_token[r]`` is the token of
    row r of the permuted layout; ``inv_pos[t, j]`` is the row holding slot
    (t, j), or -1 when that slot's expert is not local.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    buckets = [[] for _ in range(e_count)]
    local_pos = np.full((T, k), -1, dtype=np.int64)
    local_exp = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j]) - e_begin
            if 0 <= e < e_count:
                local_pos[t, j] = len(buckets[e])
                local_exp[t, j] = e
                buckets[e].append(t)
    counts = np.array([len(bk) for bk in buckets], dtype=np.int64)
    offsets = np.zeros(e_count + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    src_token = np.array([t for bk in buckets for t in bk], dtype=np.int64)
    inv_pos = np.where(local_exp >= 0,
                       offsets[np.maximum(local_exp, 0)] + local_pos, -1)
    x_perm = None
    if x is not None:
        x_perm = np.asarray(x, dtype=np.float64)[src_token]
    return counts, offsets, src_token, inv_pos.astype(np.int64), x_perm


def dispatch_masked(idx, e_begin: int, e_count: int, cap: int):
    """Masked (fixed-capacity) layout of the routing slots ([P5] decode: masked
    expert GEMM; READING R34).

    Local expert e owns rows ``[e*cap, (e+1)*cap)``. Walking the slots in
    token order, slot (t, j) of a local expert e gets rank = the number of
    earlier tokens routed to e; it goes to row ``e*cap + rank`` if rank < cap,
    else it is dropped (-1). Returns ``(counts [e_count] = min(routed, cap),
    row_token [e_count*cap] (-1 where unused), pos [T,k])``.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    seen = [0] * e_count
    row_token = np.full(e_count * cap, -1, dtype=np.int64)
    pos = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j]) - e_begin
            if 0 <= e < e_count:
                r = seen[e]
                seen[e] += 1
                if r < cap:
                    pos[t, j] = e * cap + r
                    row_token[e * cap + r] = t
    counts = np.minimum(np.array(seen, dtype=np.int64), cap)
    return counts, row_token, pos


# ---------------------------------------------------------------------------
# experts  ([P1] EP 路径: grouped GEMM; [P5] BatchedExperts)
# ---------------------------------------------------------------------------


def experts(x_perm, offsets, weights) -> np.ndarray:
    """Run every local expert's gated MLP on its contiguous rows.

    ``y_perm[o_e:o_{e+1}] = swiglu(x_perm[o_e:o_{e+1}], Wg_e, Wu_e, Wd_e)``.
    [P1] EP 路径 (one rank runs many experts, grouped); [P1] 实际 MLP 计算策略
    for each expert's MLP. ``weights`` is a sequence of (Wg, Wu, Wd) float64
    triples in the pages' orientation, or a callable ``e -> triple`` so large
    weight sets can be produced one expert at a time.
    """
    x_perm = np.asarray(x_perm, dtype=np.float64)
    offsets = np.asarray(offsets)
    e_count = len(offsets) - 1
    get = weights if callable(weights) else (lambda e: weights[e])
    y = np.zeros((x_perm.shape[0], x_perm.shape[1]), dtype=np.float64)
    for e in range(e_count):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            wg, wu, wd = get(e)
            y[a:b] = swiglu(x_perm[a:b], wg, wu, wd)
    return y


# ---------------------------------------------------------------------------
# combine  ([P1] EP 路径: weighted sum back at the source; [P5] token_unpermutation)
# ---------------------------------------------------------------------------


def combine(y_perm, inv_pos, w, residual=None) -> np.ndarray:
    """``out[t] = Σ_{j : inv_pos[t,j] >= 0} w[t,j] · y_perm[inv_pos[t,j]]`` (+ ``residual[t]``).

    [P1] EP 路径: the expert outputs are summed with the router weights back
    at the token's source. READING R18: the global weights are used unchanged
    (no renormalisation over the local experts), so a token with no local
    expert gets 0 and the outputs of disjoint expert ranges add up to the
    all-local result. The sum runs over slots in order j = 0..k-1.

    ``residual`` (optional, [T, d]): [P1] Norm&Residual, the Pre-Norm block's
    output is the residual stream R plus the FFN of its normalised copy; the
    skip connection is added once, after the expert sum.
    """
    y_perm = np.asarray(y_perm, dtype=np.float64)
    inv_pos = np.asarray(inv_pos)
    w = np.asarray(w, dtype=np.float64)
    T, k = inv_pos.shape
    d = y_perm.shape[1] if y_perm.ndim == 2 else 0
    out = np.zeros((T, d), dtype=np.float64)
    for j in range(k):
        m = inv_pos[:, j] >= 0
        if m.any():
            out[m] += w[m, j][:, None] * y_perm[inv_pos[m, j]]
    if residual is not None:
        out = out + np.asarray(residual, dtype=np.float64)
    return out


# ---------------------------------------------------------------------------
# end to end  ([P1] Norm&Residual: FFN(V) with V = RMSNorm_ffn(R))
# ---------------------------------------------------------------------------


def moe_ffn(x, gamma, w_r, bias, weights, e_begin: int, e_count: int,
            k: int = 8, eps: float = 1e-5, norm: bool = True, idx=None, act_fp8: bool = False):
    """One rank's share of the MoE FFN sub-block, ``FFN(RMSNorm(x))``.

    Steps in the pages' order: RMSNorm ([P1] Norm&Residual) -> router ([P1]
    MoE Router 过程) -> permutation by expert ([P5] token_permutation) ->
    grouped expert MLPs ([P1] EP 路径) -> weighted combine ([P1] EP 路径).
    The residual add is not part of this sub-call (READING R20). With
    ``norm=False`` the router sees x directly (READING R11, the router-only
    workload). ``idx`` optionally fixes the routed sets (the weights are then
    recomputed from the unbiased scores), which the parity checker uses when a
    token's 8th/9th key gap is below the tie threshold. ``act_fp8`` runs the
    experts with fp8 activations (``quant.experts_a8``, the block-fp8 prefill
    variant, READINGS R32/R33) on the bf16-held V.

    Returns a dict with every intermediate: v, idx, w, s, key, gap, counts,
    offsets, src_token, inv_pos, x_perm, y_perm, out.
    """
    x = np.asarray(x, dtype=np.float64)
    v = rmsnorm(x, gamma, eps) if norm else x
    r_idx, r_w, s, key, gap = route(v, w_r, bias, k)
    if idx is not None:
        r_idx = np.asarray(idx, dtype=np.int64)
        r_w = route_weights(s, r_idx)
    counts, offsets, src_token, inv_pos, x_perm = permute(r_idx, e_begin, e_count, v)
    if act_fp8:
        from .quant import bf16_round, experts_a8
        # the GEMM input V is held in bf16 between RMSNorm and the quantiser
        y_perm, _ = experts_a8(bf16_round(x_perm), offsets, weights)
    else:
        y_perm = experts(x_perm, offsets, weights)
    out = combine(y_perm, inv_pos, r_w)
    return dict(v=v, idx=r_idx, w=r_w, s=s, key=key, gap=gap, counts=counts,
                offsets=offsets, src_token=src_token, inv_pos=inv_pos,
                x_perm=x_perm, y_perm=y_perm, out=out)
