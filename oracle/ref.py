"""Reference (oracle) implementation of the routed-expert MoE FFN path.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke entry point and the
bench's CPU-baseline leg may import this module.  It is deliberately plain:
explicit per-expert loops, dequantise-then-matmul, exact top-k, no blocking,
no fusion.  Floating point is fp64 unless a function says otherwise; the one
place where fp32 is prescribed is the routing decision (see
`logits_pinned_f32`), which both sides take in the same fp32 arithmetic.

Sources (the pages; cited by title and section):
  [S1] "Specter: Fast MoE Inference via Quantization-Enabled Multi-Step
       Speculative Offloading" (AI summary page): Key Contributions 1-4,
       Methodology in Plain English.
  [S2] "Specter previews expert routing with an INT4 copy of the model
       itself": What shipped.
  [S1] also, Main Findings and Future Directions: the draft's routing
       fidelity is compared across 2-, 4- and 8-bit precisions (the 2/8-bit
       draft FFN here).

Readings taken where the pages are silent are named R1..R12 in each
docstring; the design notes list all of them.

Parity status of each function (what pins it, in tests/test_oracle_*.py):
  logits_pinned_f32 / logits_f64 ... pinned (closed forms, Higham bound)
  route_topk ....................... pinned (brute force over subsets, ties)
  elb_update ....................... pinned (library bincount, sums)
  gather_maps ...................... pinned (permutation/inverse invariants,
                                     library stable argsort)
  dequant_gptq ..................... pinned (hand-packed closed forms, 2/4/8-bit
                                     codes)
  expert_ffn_f16 ................... pinned (one-hot closed form with known
                                     SiLU values, zero weights, textbook
                                     dense MLP at E=1, shared-expert
                                     concatenation identity)
  expert_ffn_int4 .................. pinned (hand-packed one-hot closed form;
                                     equals expert_ffn_f16 on weights placed
                                     exactly on the quantisation grid)
  expert_ffn_awq ................... pinned (unit factors give expert_ffn_int4
                                     exactly; hand-packed one-hot closed form
                                     with factors 2 and 4 on both inputs)
  grouped_ffn ...................... pinned (masked brute force; the grid
                                     identity above through the loop)
  moe_layer ........................ pinned (zero routed experts leave
                                     sigmoid(x . w_sg) * shared expert, in
                                     closed form; routed + gated shared
                                     closed form; residual added once)
  per_token_ffn .................... pinned (equals grouped_ffn, the pages'
                                     claim that grouping by expert
                                     leaves the values unchanged)
  combine .......................... pinned (k=1 identity, hand sums)
  rms_norm ......................... pinned (constant rows, scale invariance)
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

GROUP = 128
LANES = 64          # width of the pinned reduction (one wave of 64 lanes)
CHUNK = 8           # consecutive hidden elements owned together by a lane

__all__ = [
    "logits_pinned_f32", "logits_f64", "route_topk", "elb_update", "gather_maps",
    "unpack_gptq", "dequant_gptq", "silu", "swiglu_ffn", "expert_ffn_f16",
    "expert_ffn_int4", "expert_ffn_awq", "grouped_ffn", "per_token_ffn", "combine", "moe_layer",
    "to_f16", "rms_norm",
]


def to_f16(a: np.ndarray) -> np.ndarray:
    """Round to fp16, nearest-even, no flush (R11)."""
    return np.asarray(a).astype(np.float16)


# ---------------------------------------------------------------------------
# S1  routing
# ---------------------------------------------------------------------------

def logits_pinned_f32(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Router logits x . w_e in fp32, in one fixed summation order.

    [S1 Key Contributions 3] routing decisions come from the target router;
    [S2 What shipped] the draft reuses that same FP16 router tensor.  The
    pages fix no arithmetic for it.  Reading R1: because the top-k choice is
    an integer decided by floating point, the fp32 sum is taken in one pinned
    order that both sides follow:

      * the hidden axis is cut into chunks of 8 consecutive elements;
        chunk c belongs to lane c mod 64;
      * each lane starts from +0 and adds, chunk by chunk in increasing c and
        element by element inside a chunk, the product x_h * w_h (exact in
        fp32: both factors are fp16) with one fp32 rounding per addition;
      * the 64 lane sums are then combined by six pairwise rounds: in round
        with distance d in (32, 16, 8, 4, 2, 1) every lane p replaces its sum
        by fl(s_p + s_(p xor d));
      * the logit is lane 0's value (all lanes agree).

    x: fp16 [T, H]; w: fp16 [E, H] (or [H] for one vector).  Returns fp32
    [T, E] (or [T]).
    """
    x = np.asarray(x)
    w = np.asarray(w)
    one = w.ndim == 1
    if one:
        w = w[None, :]
    T, H = x.shape
    E = w.shape[0]
    assert H % CHUNK == 0
    nch = H // CHUNK
    xf = x.astype(np.float32).reshape(T, nch, CHUNK)
    wf = w.astype(np.float32).reshape(E, nch, CHUNK)
    s = np.zeros((T, E, LANES), dtype=np.float32)
    rounds = (nch + LANES - 1) // LANES
    for i in range(rounds):
        c0 = i * LANES
        c1 = min(nch, c0 + LANES)
        n = c1 - c0
        for j in range(CHUNK):
            prod = xf[:, None, c0:c1, j] * wf[None, :, c0:c1, j]   # exact
            s[:, :, :n] = s[:, :, :n] + prod                         # fp32 round
    lane = np.arange(LANES)
    for d in (32, 16, 8, 4, 2, 1):
        s = s + s[:, :, lane ^ d]
    out = s[:, :, 0].copy()
    return out[:, 0] if one else out


def logits_f64(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Router logits in fp64 (for the near-tie margin diagnostic)."""
    return np.asarray(x).astype(np.float64) @ np.asarray(w).astype(np.float64).T


def route_topk(x: np.ndarray, w_router: np.ndarray, k: int, renormalize: bool = False,
               w_shared_gate: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Top-k routing by the (shared) FP16 router.

    [S1 Key Contributions 3; S2 What shipped] The target router's decisions
    are authoritative and the draft uses the same router tensor.
    R1: logits in the pinned fp32 order (`logits_pinned_f32`).
    R2: experts are ranked by logit, larger first; equal logits put the lower
        expert index first (R3).  The k best, in that rank order, are the ids.
    R4: weights are the softmax over all E logits (fp64 here, from the fp32
        logits) taken at the chosen ids; with `renormalize` they are divided
        by their sum.  Selection on logits equals selection on softmax since
        softmax is monotone.
    R5: when a shared-expert gate vector is given, gate_t =
        sigmoid(x_t . w_sg), the dot taken in the same pinned order.

    Returns ids int32 [T,k], weights fp64 [T,k], gate fp64 [T] (or None),
    logits32 [T,E], logits64 [T,E] and margin64 [T] (fp64 gap between the
    k-th and (k+1)-th ranked logits, inf when k == E).
    """
    T, H = x.shape
    E = w_router.shape[0]
    assert 1 <= k <= E
    L32 = logits_pinned_f32(x, w_router)
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        # exact ranking by (-logit, index): lexsort's last key is primary
        order = np.lexsort((np.arange(E), -L32[t].astype(np.float64)))
        ids[t] = order[:k]
    Ld = L32.astype(np.float64)
    m = Ld.max(axis=1, keepdims=True)
    p = np.exp(Ld - m)
    p /= p.sum(axis=1, keepdims=True)
    wts = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renormalize:
        wts = wts / wts.sum(axis=1, keepdims=True)
    L64 = logits_f64(x, w_router)
    margin = np.full(T, np.inf)
    if k < E:
        for t in range(T):
            srt = np.sort(L64[t])[::-1]
            margin[t] = srt[k - 1] - srt[k]
    gate = None
    if w_shared_gate is not None:
        g32 = logits_pinned_f32(x, w_shared_gate).astype(np.float64)
        gate = 1.0 / (1.0 + np.exp(-g32))
    return dict(ids=ids, weights=wts, gate=gate, logits32=L32, logits64=L64, margin64=margin)


# ---------------------------------------------------------------------------
# S2  Expert Lookahead Buffer counters
# ---------------------------------------------------------------------------

def elb_update(counters: np.ndarray, ids: np.ndarray, layer: int) -> np.ndarray:
    """Add one to counters[layer, e] for every (token, slot) routed to e.

    [S1 Key Contributions 3; Methodology in Plain English] the Expert
    Lookahead Buffer keeps, per layer and expert, a count of draft routing
    choices in device memory; copies taken at chunk boundaries drive
    prefetch.  R6: one count per (token, selected expert), unweighted,
    accumulated across calls until the caller snapshots or clears it.
    Ids outside [0, E) are not counted.
    """
    out = np.array(counters, dtype=np.int32, copy=True)
    E = out.shape[1]
    for e in np.asarray(ids).reshape(-1):
        if 0 <= e < E:
            out[layer, e] += 1
    return out


# ---------------------------------------------------------------------------
# S3  gather by expert
# ---------------------------------------------------------------------------

def gather_maps(ids: np.ndarray, E: int) -> Dict[str, np.ndarray]:
    """Stable grouping of the T*k (token, slot) pairs by expert.

    [S1 Key Contributions 4; Methodology] draft and verification both
    process each expert's rows as one block.  R7: pair p = t*k + j; pairs are ordered by expert and, inside
    one expert, by increasing p (a stable counting sort).

    Returns offsets [E+1] (exclusive prefix sum of per-expert counts),
    sorted_pair [T*k] (pair at each sorted row), sorted_token [T*k]
    (= sorted_pair // k), pair_pos [T*k] (sorted row of each pair, the
    inverse of sorted_pair), active [E] (touched experts in increasing id,
    padded with -1) and n_active.  Ids outside [0, E) are dropped: their
    pair_pos is -1 and no row holds them.
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    flat = ids.reshape(-1)
    n = flat.size
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        if 0 <= e < E:
            counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:-1].copy()
    sorted_pair = np.full(n, -1, dtype=np.int64)
    pair_pos = np.full(n, -1, dtype=np.int64)
    for p in range(n):                      # increasing p: stability
        e = flat[p]
        if 0 <= e < E:
            r = cursor[e]
            cursor[e] += 1
            sorted_pair[r] = p
            pair_pos[p] = r
    rows = int(offsets[E])
    sorted_token = np.full(n, -1, dtype=np.int64)
    sorted_token[:rows] = sorted_pair[:rows] // k
    act = [e for e in range(E) if counts[e] > 0]
    active = np.full(E, -1, dtype=np.int64)
    active[:len(act)] = act
    i32 = lambda a: a.astype(np.int32)
    return dict(offsets=i32(offsets), sorted_pair=i32(sorted_pair), sorted_token=i32(sorted_token),
                pair_pos=i32(pair_pos), active=i32(active), n_active=np.int32(len(act)),
                counts=i32(counts))


# ---------------------------------------------------------------------------
# S4 / S6  expert FFNs
# ---------------------------------------------------------------------------

def unpack_gptq(qweight: np.ndarray, qzeros: np.ndarray, bits: int = 4):
    """Codes q [K, N] and zeros z [K/128, N] (uint8) from the GPTQ words.

    [S2 What shipped] the draft's routed experts are GPTQ INT4 with group
    size 128.  R8 (the usual GPTQ checkpoint layout): nibble i, bits 4i..4i+3,
    of qweight[r, n] is row 8r+i of column n; nibble i of qzeros[g, c] is the
    zero of column 8c+i in group g; zeros carry no offset; no act-order.
    R21: the 2- and 8-bit drafts ([S1] Main Findings) use the same layout
    with c = 32/bits codes per word: code i (bits bits*i ...) of qweight[r, n]
    is row c*r+i, code i of qzeros[g, w] the zero of column c*w+i.
    """
    assert bits in (2, 4, 8)
    per = 32 // bits
    mask = np.uint32((1 << bits) - 1)
    qw = np.asarray(qweight).view(np.uint32)
    R, N = qw.shape
    q = np.empty((R * per, N), dtype=np.uint8)
    for i in range(per):
        q[i::per, :] = (qw >> np.uint32(bits * i)) & mask
    qz = np.asarray(qzeros).view(np.uint32)
    G, C = qz.shape
    z = np.empty((G, C * per), dtype=np.uint8)
    for i in range(per):
        z[:, i::per] = (qz >> np.uint32(bits * i)) & mask
    return q, z


def dequant_gptq(qweight, scales, qzeros, dtype=np.float64, bits: int = 4) -> np.ndarray:
    """W[kk, n] = (q[kk, n] - z[kk // 128, n]) * s[kk // 128, n]  ([K, N]).

    [S2 What shipped] INT4 weight tiles are dequantised and the product is
    formed in higher precision.  In fp32 the result is exact: (q - z) lies in
    [-(2^bits - 1), 2^bits - 1] (at most 9 significant bits) and s has an
    11-bit significand.
    """
    q, z = unpack_gptq(qweight, qzeros, bits)
    s = np.asarray(scales).astype(dtype)
    g = np.arange(q.shape[0]) // GROUP
    return (q.astype(dtype) - z[g, :].astype(dtype)) * s[g, :]


def silu(a: np.ndarray) -> np.ndarray:
    """silu(a) = a / (1 + exp(-a)) (R9)."""
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def swiglu_ffn(xr: np.ndarray, w_gate_kn: np.ndarray, w_up_kn: np.ndarray,
               w_down_kn: np.ndarray) -> np.ndarray:
    """SwiGLU MLP on rows xr: (silu(xr Wg) * (xr Wu)) Wd, all [K, N] weights.

    R9: the pages do not name the expert MLP form; the workloads use SwiGLU
    without biases.
    """
    g = xr @ w_gate_kn
    u = xr @ w_up_kn
    return (silu(g) * u) @ w_down_kn


def expert_ffn_f16(xr: np.ndarray, w13: np.ndarray, w2: np.ndarray, dtype=np.float64):
    """FP16 target expert on rows xr.  w13 fp16 [2I, H] (gate rows, then up
    rows), w2 fp16 [H, I], nn.Linear layout (y = x W^T)."""
    I = w2.shape[1]
    a = np.asarray(xr).astype(dtype)
    w13f = w13.astype(dtype)
    return swiglu_ffn(a, w13f[:I].T, w13f[I:].T, w2.astype(dtype).T)


def expert_ffn_int4(xr: np.ndarray, q13, q2, dtype=np.float64, bits: int = 4):
    """INT4 (or, with bits, 2/8-bit) draft expert on rows xr; q13/q2 =
    (qweight, scales, qzeros) of w13^T [H, 2I] and w2^T [I, H] (GPTQ [K, N]
    layout)."""
    W13 = dequant_gptq(*q13, dtype=dtype, bits=bits)   # [H, 2I]
    W2 = dequant_gptq(*q2, dtype=dtype, bits=bits)     # [I, H]
    I = W2.shape[0]
    a = np.asarray(xr).astype(dtype)
    return swiglu_ffn(a, W13[:, :I], W13[:, I:], W2)


def expert_ffn_awq(xr: np.ndarray, q13, q2, a13, a2, dtype=np.float64):
    """AWQ-style INT4 draft expert on rows xr ([S1] Main Findings compare
    AWQ, GPTQ and GGUF 4-bit drafts).  Reading R22: an AWQ-style expert was
    quantised after input channel c of each projection had been multiplied
    by a positive factor a[c]; the product then takes the activation divided
    by that factor.  q13/q2 are GPTQ tensors of w13^T [H, 2I] and w2^T [I, H]
    as in expert_ffn_int4; a13 [H] and a2 [I] the factors of the gate/up and
    the down projection's inputs.
      h = silu((x / a13) Wg) * ((x / a13) Wu);   y = (h / a2) Wd
    """
    W13 = dequant_gptq(*q13, dtype=dtype)   # [H, 2I]
    W2 = dequant_gptq(*q2, dtype=dtype)     # [I, H]
    I = W2.shape[0]
    xa = np.asarray(xr).astype(dtype) / np.asarray(a13).astype(dtype)
    g = xa @ W13[:, :I]
    u = xa @ W13[:, I:]
    h = silu(g) * u
    return (h / np.asarray(a2).astype(dtype)) @ W2


_QBITS = {"int2": 2, "int4": 4, "int8": 8}


def grouped_ffn(x: np.ndarray, maps: Dict[str, np.ndarray], experts: Sequence, kind: str,
                dtype=np.float64, only: Optional[Sequence[int]] = None) -> np.ndarray:
    """Expert outputs for every sorted row, by an explicit loop over experts.

    [S1 Key Contributions 4; Methodology] tokens routed to one expert are
    packed and that expert is applied to all of them at once.  Row r of the
    result holds FFN_e(x[sorted_token[r]]) for the expert e owning row r.
    `kind` is "int4" (experts[e] = dict(w13=(qw,s,qz), w2=(...))), "int2" /
    "int8" (the same with 2/8-bit codes), "awq" (the int4 dict with the
    input-channel factors a13, a2 added) or "f16" (experts[e] = (w13, w2)).
    Rows of experts outside `only` stay NaN.
    """
    off = maps["offsets"]
    st = maps["sorted_token"]
    E = len(off) - 1
    rows = int(off[E])
    H = x.shape[1]
    y = np.full((rows, H), np.nan, dtype=dtype)
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0 or (only is not None and e not in only):
            continue
        xr = x[st[r0:r1]]
        if kind == "awq":
            ex = experts[e]
            y[r0:r1] = expert_ffn_awq(xr, ex["w13"], ex["w2"], ex["a13"], ex["a2"], dtype)
        elif kind in _QBITS:
            y[r0:r1] = expert_ffn_int4(xr, experts[e]["w13"], experts[e]["w2"], dtype,
                                       bits=_QBITS[kind])
        else:
            y[r0:r1] = expert_ffn_f16(xr, experts[e][0], experts[e][1], dtype)
    return y


def per_token_ffn(x: np.ndarray, ids: np.ndarray, experts: Sequence, kind: str,
                  dtype=np.float64) -> np.ndarray:
    """The unregrouped ordering: token by token, slot by slot, one
    vector-matrix product per (token, expert).  Returns [T, k, H].

    [S1 Methodology] grouping rows by expert changes the evaluation order
    only, not the values; the tests hold the two orderings to each other.
    """
    T, k = ids.shape
    H = x.shape[1]
    out = np.zeros((T, k, H), dtype=dtype)
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            xr = x[t:t + 1]
            if kind in _QBITS:
                out[t, j] = expert_ffn_int4(xr, experts[e]["w13"], experts[e]["w2"], dtype,
                                            bits=_QBITS[kind])[0]
            else:
                out[t, j] = expert_ffn_f16(xr, experts[e][0], experts[e][1], dtype)[0]
    return out


# ---------------------------------------------------------------------------
# S7  combine
# ---------------------------------------------------------------------------

def combine(y_sorted: np.ndarray, pair_pos: np.ndarray, weights: np.ndarray,
            shared_out: Optional[np.ndarray] = None, shared_scale: Optional[np.ndarray] = None,
            residual: Optional[np.ndarray] = None, dtype=np.float64) -> np.ndarray:
    """out[t] = sum_j w[t,j] * y[pair_pos[t*k+j]] + c_t * shared[t] (+ residual[t]).

    R10: the pages do not describe the combine; it is the usual routed-MoE
    weighted sum of the chosen experts' outputs plus the shared expert (c_t =
    its sigmoid gate, or 1 without one).  The optional residual input turns a
    layer into x + MoE(x) for layer chaining.  Returned unrounded (`dtype`);
    apply `to_f16` for the fp16 output.
    """
    T, k = weights.shape
    H = y_sorted.shape[1]
    out = np.zeros((T, H), dtype=dtype)
    for t in range(T):
        for j in range(k):
            r = int(pair_pos[t * k + j])
            if r >= 0:
                out[t] += np.float64(weights[t, j]) * y_sorted[r].astype(dtype)
        if shared_out is not None:
            c = 1.0 if shared_scale is None else float(shared_scale[t])
            out[t] += c * shared_out[t].astype(dtype)
        if residual is not None:
            out[t] += residual[t].astype(dtype)
    return out


def rms_norm(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) per row, fp64, unit weight.

    R17: the pages say draft and target share the non-expert parts, the
    normalisation included ([S1] Methodology), without defining them.  Layers
    of a multi-layer chunk are pre-norm residual blocks x <- x + MoE(rms(x)),
    the plainest reading that keeps a synthetic chain finite.
    """
    a = np.asarray(x).astype(np.float64)
    return a / np.sqrt(np.mean(a * a, axis=-1, keepdims=True) + eps)


# ---------------------------------------------------------------------------
# whole layer (the plain definition)
# ---------------------------------------------------------------------------

def moe_layer(x: np.ndarray, w_router: np.ndarray, k: int, experts: Sequence, kind: str,
              shared: Optional[Dict] = None, renormalize: bool = False,
              residual=None, dtype=np.float64) -> Dict[str, np.ndarray]:
    """One routed-expert MoE layer: route, group, per-expert FFN, combine.

    out_t = sum_j w_tj FFN_(ids_tj)(x_t) + c_t FFN_shared(x_t)  (+ r_t),
    with r the `residual` array (or x itself when `residual` is True).
    [S1 Key Contributions 2] routers and shared experts are FP16 in both the
    draft and the target; only routed experts are INT4 in the draft.
    """
    gate_vec = None if shared is None else shared.get("gate")
    r = route_topk(x, w_router, k, renormalize, gate_vec)
    E = w_router.shape[0]
    maps = gather_maps(r["ids"], E)
    y = grouped_ffn(x, maps, experts, kind, dtype)
    sh = None
    if shared is not None:
        sh = expert_ffn_f16(x, shared["w13"], shared["w2"], dtype)
    if residual is True:
        residual = x
    elif residual is False:
        residual = None
    out = combine(y, maps["pair_pos"], r["weights"], sh, r["gate"], residual, dtype)
    return dict(route=r, maps=maps, y_sorted=y, shared_out=sh, out=out)
