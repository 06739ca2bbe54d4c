"""Plain, slow CPU oracle of one MoE layer: route -> capacity dispatch -> expert FFN
-> combine, plus the counters-only ledger.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's
CPU-baseline leg, never by the GPU library.  It shares no code with the GPU path.

Pages cited (by title):
  [EP47] "47. MoE Expert Parallel | MoE 专家并行"  (llm-algo-leetcode, chapter 47)
  [EP46] "46. MoE Expert Parallel | MoE 专家并行"  (llm-algo-leetcode, chapter 46)
  [WIKI] "MoE 与专家并行"  (ai-infra-wiki, distributed training / expert parallel)
  [EPC]  "专家并行（Expert Parallelism）"  (tier6-model, LLM 并行通信)
  [DSV3] "MoE大模型专家并行与动态路由优化——从DeepSeek-V3到生产级推理架构"  (ybb.press)

Arithmetic: float64 throughout, from the exact stored input values; each result
is rounded once to the storage type of the matching GPU buffer (fp32 logits,
gates, expert outputs Y and layer output; bf16 hidden activations H on bf16
workloads).  Library primitives (matmul, lexsort, exp, tanh) serve as steps.

Readings taken where the pages are silent or disagree (each is restated at the
function that uses it):
  R1  softmax is taken over the K selected logits only ([DSV3] 3.1).
  R2  top-k order: descending logit; equal logits -> lower expert id first;
      -0.0 equals +0.0; logits are finite.
  R3  capacity = ceil((A/E)*cf) in IEEE double, 0 when A == 0 ([EP47] Step 3,
      [EP46] TODO 1).  The floor (int()) of [DSV3] 3.3 is not used.
  R4  drops: routes are taken in (token, k-slot) order and the first `capacity`
      routes of each expert are accepted ([DSV3] 3.3 capacity loop).
  R5  accepted rows are packed per expert in acceptance order, experts in id
      order: row = offset[e] + rank, offset = exclusive prefix of accepted counts.
  R6  a dropped route contributes zero; gates are not renormalised; a token
      with no accepted route outputs zero ([EP46] combine: zeros + index_add).
  R7  expert FFN = W2 * GELU_tanh(W1 x + b1) + b2 ([DSV3] section 一), GELU in
      its tanh form; W1 stored [E, F, h], W2 stored [E, h, F].
  R8  byte counters count all A routes (pre-capacity), as the pages' ledgers
      do; accepted-route counterparts are reported beside them.
  R9  locality is counted over all routes ([EP46] contract) and, separately,
      over accepted routes (the prose of [EP46] Step 2).
  R10 L_aux: the formula of [DSV3] 3.2 (alpha * sum f_i P_i) is `l_aux`; its
      code's normalisation (alpha * E * sum f_i P_i / K) is `l_aux_norm`.
  R11 aux-loss-free balancing ([DSV3] section 八): the bias update counts each
      token once, at the argmax of its adjusted logits (the top-1 expert, as
      the page's bincount of argmax does), and applies
      bias += alpha * (mean_count - count) with alpha = 0.1 in fp32, one
      rounding per operation.  The dropless variant is the same dispatch with
      a capacity of at least T (no expert can receive more than T routes).
  R12 FP8 dispatch payload ([DSV3] 4.3): one scale for the whole [T, h]
      activation tensor, scale = bf16(max|x| / 448); codes = E4M3(bf16(x /
      scale)) with ties to even; the receiver's bf16(decode * scale) feeds the
      experts.  All-zero activations (scale 0) give zero codes.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "round_bf16", "round_f32", "router_logits", "add_logit_bias", "topk_softmax",
    "expert_loads", "capacity", "overflow", "slot_routes", "dispatch",
    "gelu_tanh", "expert_ffn_segment", "expert_ffn", "expert_ffn_rows", "combine", "combine_index_add",
    "summarize_routes", "dispatch_locality", "aux_loss_terms",
    "uniform_expert_placement", "load_monitor", "ledger", "moe_layer",
    "moe_layer_per_token", "routes_from_idx", "top1_counts", "expert_bias_update",
    "E4M3_MAX", "e4m3_encode", "e4m3_decode", "fp8_scale", "fp8_quantize", "fp8_dequantize",
    "PLAN_THRESHOLDS", "recommend_plan",
    "expert_rank_affinity", "local_routes_under", "locality_placement", "rank_loads",
]


# ----------------------------------------------------------------------------
# rounding to storage types
# ----------------------------------------------------------------------------
def round_f32(a) -> np.ndarray:
    """Round float64 values to the nearest fp32 (IEEE round-half-even), as f64."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(a) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (round-half-even), as f64.

    bfloat16 keeps 8 significant bits (7 stored + the implicit one) over the
    fp32 exponent range, so the quantum of a value in [2^(e-1), 2^e) is
    2^(e-8), and never finer than 2^-133 (the bf16 subnormal step).
    """
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.rint(a / q) * q


# ----------------------------------------------------------------------------
# a1-a2: router  ([DSV3] section 一: g = Softmax(TopK(W_g x)); 3.1 TopKGate)
# ----------------------------------------------------------------------------
def router_logits(x: np.ndarray, w_gate: np.ndarray) -> np.ndarray:
    """logits[t, e] = sum_j x[t, j] * W_g[e, j] in float64, rounded once to fp32.

    [DSV3] 3.1: the gate is a bias-free linear map model_dim -> num_experts.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_gate, dtype=np.float64)
    return (x @ w.T).astype(np.float32)


def add_logit_bias(logits32: np.ndarray, bias32: Optional[np.ndarray]) -> np.ndarray:
    """Per-expert additive logit bias, one IEEE fp32 add per element.

    [DSV3] section 八 (the DeepSeek-V3 gate adds a per-expert bias to the
    logits and routes on the adjusted logits); used by the hot-expert workload.
    """
    l32 = np.asarray(logits32, dtype=np.float32)
    if bias32 is None:
        return l32
    return (l32 + np.asarray(bias32, dtype=np.float32)[None, :]).astype(np.float32)


def topk_softmax(logits32: np.ndarray, K: int, bias32: Optional[np.ndarray] = None):
    """Per token: the K largest logits and the softmax over those K.

    [DSV3] 3.1 (topk, then softmax of the selected logits), readings R1, R2.
    Returns (idx int32 [T, K], gate float32 [T, K]); slot 0 holds the largest.
    """
    l32 = add_logit_bias(logits32, bias32)
    T, E = l32.shape
    if not 1 <= K <= E:
        raise ValueError("need 1 <= K <= E")
    if T == 0:
        return np.zeros((0, K), np.int32), np.zeros((0, K), np.float32)
    ids = np.broadcast_to(np.arange(E), (T, E))
    neg = -l32.astype(np.float64)
    # primary key: -logit ascending (largest first); secondary: expert id
    order = np.lexsort((ids, neg), axis=-1)[:, :K]
    sel = np.take_along_axis(l32.astype(np.float64), order, axis=1)
    w = np.exp(sel - sel[:, :1])          # softmax, shifted by the largest logit
    g = w / w.sum(axis=1, keepdims=True)
    return order.astype(np.int32), g.astype(np.float32)


# ----------------------------------------------------------------------------
# a3-a4: loads, capacity, overflow, slotting
# ----------------------------------------------------------------------------
def routes_from_idx(idx: np.ndarray) -> list:
    """[T, K] expert ids -> the pages' `routes` form: one list of ids per token."""
    return [[int(e) for e in row] for row in np.asarray(idx)]


def expert_loads(idx, E: int) -> np.ndarray:
    """load[e] = number of routes (t, k) with idx[t, k] == e ([EP47] Step 3:
    expand the routes and count each expert's hits)."""
    if E <= 0:
        raise ValueError("num_experts must be positive")
    loads = np.zeros(E, np.int64)
    for e in np.asarray(idx).reshape(-1):
        e = int(e)
        if not 0 <= e < E:
            raise ValueError("expert id out of range")
        loads[e] += 1
    return loads


def capacity(A: int, E: int, cf: float) -> int:
    """ceil((A / E) * capacity_factor), 0 when there are no routes.

    [EP47] Step 3 and [EP46] TODO 1; reading R3.
    """
    if E <= 0:
        raise ValueError("num_experts must be positive")
    if not (cf > 0 and math.isfinite(cf)):
        raise ValueError("capacity_factor must be positive")
    if A == 0:
        return 0
    return int(math.ceil((A / E) * cf))


def overflow(loads, cap: int) -> int:
    """sum_e max(load_e - capacity, 0)  ([EP47] Step 3)."""
    return int(sum(max(int(l) - cap, 0) for l in loads))


def slot_routes(idx: np.ndarray, E: int, cap: int) -> dict:
    """Capacity-limited slotting in (token, k-slot) order.

    Follows the capacity loop of [DSV3] 3.3: walk tokens, then k-slots; a route
    is accepted while its expert has taken fewer than `cap` routes.  Besides the
    accept mask it records, per route, its rank = number of earlier routes to
    the same expert (accepted or not), and lays accepted routes out in the
    expert-grouped buffer (reading R5).

    Returns route_rank [T, K] (-1 never occurs for valid ids), route_row [T, K]
    (-1 = dropped), row_token [R], expert_offsets [E + 1], accepted [E].
    """
    idx = np.asarray(idx)
    T, K = idx.shape
    if cap < 0:
        raise ValueError("capacity must be >= 0")
    taken = [0] * E     # accepted so far per expert ([DSV3] 3.3 expert_count)
    seen = [0] * E      # routes so far per expert, accepted or not
    route_rank = np.full((T, K), -1, np.int32)
    slot = np.full((T, K), -1, np.int64)
    for t in range(T):
        for k in range(K):
            e = int(idx[t, k])
            if not 0 <= e < E:
                raise ValueError("expert id out of range")
            route_rank[t, k] = seen[e]
            seen[e] += 1
            if taken[e] < cap:
                slot[t, k] = taken[e]
                taken[e] += 1
    offsets = np.zeros(E + 1, np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + taken[e]
    R = int(offsets[E])
    route_row = np.full((T, K), -1, np.int32)
    row_token = np.full(R, -1, np.int32)
    for t in range(T):
        for k in range(K):
            if slot[t, k] >= 0:
                r = int(offsets[int(idx[t, k])] + slot[t, k])
                route_row[t, k] = r
                row_token[r] = t
    return {"route_rank": route_rank, "route_row": route_row,
            "row_token": row_token, "expert_offsets": offsets.astype(np.int32),
            "accepted": np.asarray(taken, np.int64), "R": R}


# ----------------------------------------------------------------------------
# a5: dispatch ([EPC] dispatch: send each routed token to its expert)
# ----------------------------------------------------------------------------
def dispatch(x: np.ndarray, row_token: np.ndarray) -> np.ndarray:
    """xd[row] = x[row_token[row]]: accepted token rows, grouped by expert."""
    x = np.asarray(x)
    xd = np.empty((len(row_token), x.shape[1]), dtype=x.dtype)
    for r, t in enumerate(row_token):
        xd[r] = x[t]
    return xd


# ----------------------------------------------------------------------------
# a6: expert FFN ([DSV3] section 一: FFN(x) = W2 sigma(W1 x + b1) + b2)
# ----------------------------------------------------------------------------
def gelu_tanh(u):
    """GELU in its tanh form (Hendrycks & Gimpel, 2016):
    0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)))."""
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * u * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (u + 0.044715 * u ** 3)))


def _round_h(H, h_round):
    if h_round is None:
        return H
    if h_round == "bf16":
        return round_bf16(H)
    if h_round == "f32":
        return round_f32(H)
    raise ValueError(h_round)


def expert_ffn_segment(rows_x, w1_e, b1_e, w2_e, b2_e, h_round: Optional[str] = None):
    """One expert's FFN ([DSV3] section 一) on a block of its rows:
    H = GELU_tanh(rows_x W1_e^T + b1_e), rounded to `h_round` ("bf16" on bf16
    workloads: H is the bf16 operand of the second product); Y = H W2_e^T +
    b2_e rounded to fp32.  W1_e is [F, h], W2_e is [h, F] (reading R7).
    Returns (H, Y) as float64 arrays."""
    xe = np.asarray(rows_x, dtype=np.float64)
    u = xe @ np.asarray(w1_e, np.float64).T + np.asarray(b1_e, np.float64)
    H = _round_h(gelu_tanh(u), h_round)
    Y = round_f32(H @ np.asarray(w2_e, np.float64).T + np.asarray(b2_e, np.float64))
    return H, Y


def expert_ffn(xd, offsets, w1, b1, w2, b2, h_round: Optional[str] = None):
    """Each expert's FFN over its own rows [offsets[e], offsets[e+1]), by
    `expert_ffn_segment`.  Reading R7.  Returns (H, Y) as float64 arrays.
    `w1`, `w2`, `b1`, `b2` are indexed by expert (arrays, or any sequence
    that yields one expert's weights at a time)."""
    xd = np.asarray(xd, dtype=np.float64)
    E = len(offsets) - 1
    R = int(offsets[E])
    F = np.asarray(w1[0]).shape[0]
    h = np.asarray(w2[0]).shape[0]
    H = np.zeros((R, F))
    Y = np.zeros((R, h))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        H[lo:hi], Y[lo:hi] = expert_ffn_segment(xd[lo:hi], w1[e], b1[e], w2[e], b2[e], h_round)
    return H, Y


def expert_ffn_rows(rows_x, rows_expert, w1, b1, w2, b2, h_round=None):
    """The same FFN for an arbitrary list of (row, expert) pairs, one by one
    (used to check sampled rows of full-size workloads)."""
    rows_x = np.asarray(rows_x, dtype=np.float64)
    n = rows_x.shape[0]
    F = np.asarray(w1[0]).shape[0]
    h = np.asarray(w2[0]).shape[0]
    H = np.zeros((n, F))
    Y = np.zeros((n, h))
    for i in range(n):
        e = int(rows_expert[i])
        u = np.asarray(w1[e], np.float64) @ rows_x[i] + np.asarray(b1[e], np.float64)
        H[i] = _round_h(gelu_tanh(u), h_round)
        Y[i] = round_f32(np.asarray(w2[e], np.float64) @ H[i] + np.asarray(b2[e], np.float64))
    return H, Y


# ----------------------------------------------------------------------------
# a7: combine ([EP46] combine_expert_outputs; [DSV3] section 一 MoE(x))
# ----------------------------------------------------------------------------
def combine(Y, route_row, gate) -> np.ndarray:
    """out[t] = sum over k (ascending) with route_row[t, k] >= 0 of
    gate[t, k] * Y[route_row[t, k]]; zero if every route of t was dropped.

    Weighted expert outputs written back in original token order (reading R6).
    Summed in float64, rounded to fp32.
    """
    Y = np.asarray(Y, dtype=np.float64)
    route_row = np.asarray(route_row)
    gate = np.asarray(gate, dtype=np.float64)
    T, K = route_row.shape
    out = np.zeros((T, Y.shape[1] if Y.ndim == 2 else 0))
    for k in range(K):
        m = route_row[:, k] >= 0
        if m.any():
            out[m] += gate[m, k][:, None] * Y[route_row[m, k]]
    return round_f32(out)


def combine_index_add(token_indices, expert_outputs, routing_weights, num_tokens):
    """The scatter form of [EP46] combine: start from zeros and add each
    weighted expert output row into its token's row."""
    token_indices = np.asarray(token_indices)
    expert_outputs = np.asarray(expert_outputs, dtype=np.float64)
    routing_weights = np.asarray(routing_weights, dtype=np.float64)
    if token_indices.ndim != 1 or routing_weights.ndim != 1:
        raise ValueError("token_indices and routing_weights must be 1-D")
    if (expert_outputs.ndim != 2 or len(token_indices) != len(expert_outputs)
            or len(token_indices) != len(routing_weights)):
        raise ValueError("length mismatch")
    out = np.zeros((num_tokens, expert_outputs.shape[1]))
    for i in range(len(token_indices)):
        out[int(token_indices[i])] += routing_weights[i] * expert_outputs[i]
    return out


# ----------------------------------------------------------------------------
# a8: ledger
# ----------------------------------------------------------------------------
def summarize_routes(routes: Sequence[Sequence[int]], num_experts: int, hidden_size: int,
                     bytes_per_elem: int = 2, capacity_factor: float = 1.0) -> dict:
    """Load / capacity / overflow / byte ledger of a list of per-token routes.

    [EP47] Step 3 (A = sum of route lengths, average load A/E, capacity,
    overflow, dispatch bytes A*h*bytes, all-to-all bytes = 2x dispatch,
    balance = max load / average load, 0 when the average is 0) and [EP46]
    TODO 1 (argument checks; the same bytes named logical_route_bytes).
    balance_ratio is returned unrounded.
    """
    if num_experts <= 0 or hidden_size <= 0 or bytes_per_elem <= 0 or capacity_factor <= 0:
        raise ValueError("num_experts, hidden_size, bytes_per_elem and capacity_factor must be positive")
    loads = [0] * num_experts
    total_routes = 0
    for token_routes in routes:
        for e in token_routes:
            if not 0 <= e < num_experts:
                raise ValueError("expert id out of range")
            loads[e] += 1
            total_routes += 1
    avg = total_routes / num_experts
    cap = capacity(total_routes, num_experts, capacity_factor)
    ovf = overflow(loads, cap)
    route_bytes = total_routes * hidden_size * bytes_per_elem
    return {
        "total_tokens": len(routes),
        "total_routes": total_routes,
        "expert_loads": loads,
        "capacity": cap,
        "overflow": ovf,
        "dispatch_bytes": route_bytes,
        "logical_route_bytes": route_bytes,
        "all_to_all_bytes": 2 * route_bytes,
        "balance_ratio": (max(loads) / avg) if avg > 0 else 0.0,
    }


def dispatch_locality(routes, token_source_ranks, expert_owner_ranks, hidden_size: int,
                      bytes_per_elem: int = 2) -> dict:
    """Local vs cross-rank routes under an expert -> rank placement.

    [EP46] TODO 2: a route is local iff the token's source rank equals the
    owner rank of its expert; cross-rank dispatch bytes = cross routes * h *
    bytes, round trip = 2x (dispatch + combine), hit ratio = local / total
    (0.0 for no routes).  `expert_owner_ranks` maps expert id -> rank.
    """
    if len(routes) != len(token_source_ranks):
        raise ValueError("every token needs a source rank")
    if hidden_size <= 0 or bytes_per_elem <= 0:
        raise ValueError("hidden_size and bytes_per_elem must be positive")
    local = cross = 0
    for t, token_routes in enumerate(routes):
        src = token_source_ranks[t]
        for e in token_routes:
            if e not in expert_owner_ranks:
                raise ValueError("routed expert has no owner rank")
            if expert_owner_ranks[e] == src:
                local += 1
            else:
                cross += 1
    total = local + cross
    cross_bytes = cross * hidden_size * bytes_per_elem
    return {"total_routes": total, "local_routes": local, "cross_rank_routes": cross,
            "cross_rank_dispatch_bytes": cross_bytes,
            "cross_rank_roundtrip_bytes": 2 * cross_bytes,
            "local_hit_ratio": (local / total) if total else 0.0}


def aux_loss_terms(idx, gate, num_experts: int, alpha: float = 0.01) -> dict:
    """Load-balance terms of [DSV3] 3.2.

    f_i = (1/T) * #tokens whose top-K contains i; P_i = (1/T) * sum_t g_{t,i}
    (g_{t,i} = the token's gate for i if selected, else 0); l_aux = alpha *
    sum_i f_i P_i (the formula); l_aux_norm = alpha * E * sum_i f_i P_i / K
    (the page's code, which divides P by T*K and multiplies by E).  Reading R10.
    All zero when T == 0.
    """
    idx = np.asarray(idx)
    gate = np.asarray(gate, dtype=np.float64)
    T, K = idx.shape
    f = np.zeros(num_experts)
    P = np.zeros(num_experts)
    for t in range(T):
        for k in range(K):
            e = int(idx[t, k])
            f[e] += 1.0
            P[e] += gate[t, k]
    if T == 0:
        return {"f": f, "P": P, "l_aux": 0.0, "l_aux_norm": 0.0}
    f /= T
    P /= T
    s = float(np.sum(f * P))
    return {"f": f, "P": P, "l_aux": alpha * s, "l_aux_norm": alpha * num_experts * s / K}


def uniform_expert_placement(num_experts: int, num_devices: int) -> dict:
    """Round-robin placement: expert e lives on device e % num_devices
    ([DSV3] 2.2).  Returns {device: [experts in id order]}."""
    placement: dict = {}
    for e in range(num_experts):
        placement.setdefault(e % num_devices, []).append(e)
    return placement


def load_monitor(loads) -> dict:
    """[DSV3] section 九 load monitor: variance/mean (unbiased variance, as
    torch's default .var()) and max/mean; [WIKI] / [DSV3] flag max/mean > 2."""
    loads = np.asarray(loads, dtype=np.float64)
    mean = loads.mean() if loads.size else 0.0
    if mean == 0.0:
        return {"var_over_mean": 0.0, "max_over_mean": 0.0, "imbalanced": False}
    var = loads.var(ddof=1) if loads.size > 1 else 0.0
    mx = loads.max() / mean
    return {"var_over_mean": var / mean, "max_over_mean": mx, "imbalanced": bool(mx > 2.0)}


def ledger(idx, gate, route_row, cap: int, src_rank, owner_rank, n_ep: int,
           hidden_size: int, bytes_per_elem: int, alpha: float = 0.01) -> dict:
    """Counters-only ledger of one routed batch.

    Loads, capacity, overflow, bytes and balance from `summarize_routes`
    ([EP47], [EP46]); locality over all routes and over accepted routes from
    `dispatch_locality` with owner = the given expert -> rank map ([EP46],
    [DSV3] 2.2); f, P and L_aux from `aux_loss_terms` ([DSV3] 3.2); the
    accepted-route traffic matrix pair_routes[src, dst] (routes a real
    expert-parallel dispatch would send from rank src to rank dst); and the
    uniform per-pair all-to-all size of [EPC] (route bytes / N_EP).
    """
    idx = np.asarray(idx)
    T, K = idx.shape
    E = len(owner_rank)
    route_row = np.asarray(route_row)
    for r in owner_rank:
        if not 0 <= int(r) < n_ep:
            raise ValueError("owner rank out of range")
    routes = routes_from_idx(idx)
    s = summarize_routes(routes, E, hidden_size, bytes_per_elem, 1.0)
    owners = {e: int(owner_rank[e]) for e in range(E)}
    src = [int(v) for v in np.asarray(src_rank)]
    loc = dispatch_locality(routes, src, owners, hidden_size, bytes_per_elem)
    acc_routes = [[int(idx[t, k]) for k in range(K) if route_row[t, k] >= 0] for t in range(T)]
    acc_loc = dispatch_locality(acc_routes, src, owners, hidden_size, bytes_per_elem)
    pair = np.zeros((n_ep, n_ep), np.int64)
    for t in range(T):
        for e in acc_routes[t]:
            pair[src[t], owners[e]] += 1
    aux = aux_loss_terms(idx, gate, E, alpha)
    loads = np.asarray(s["expert_loads"], np.int64)
    accepted = int(sum(len(r) for r in acc_routes))
    mon = load_monitor(loads)
    A = s["total_routes"]
    return {
        "total_tokens": T, "total_routes": A, "num_experts": E,
        "expert_loads": loads, "capacity": int(cap),
        "accepted_routes": accepted,
        "overflow": overflow(loads, cap),
        "max_load": int(loads.max()) if E else 0,
        "logical_route_bytes": s["logical_route_bytes"],
        "dispatch_bytes": s["dispatch_bytes"],
        "all_to_all_bytes": s["all_to_all_bytes"],
        "accepted_route_bytes": accepted * hidden_size * bytes_per_elem,
        "pair_bytes_uniform": s["logical_route_bytes"] / n_ep,
        "balance_ratio": s["balance_ratio"],
        "local_routes": loc["local_routes"], "cross_rank_routes": loc["cross_rank_routes"],
        "cross_rank_dispatch_bytes": loc["cross_rank_dispatch_bytes"],
        "cross_rank_roundtrip_bytes": loc["cross_rank_roundtrip_bytes"],
        "local_hit_ratio": loc["local_hit_ratio"],
        "accepted_local_routes": acc_loc["local_routes"],
        "accepted_cross_rank_routes": acc_loc["cross_rank_routes"],
        "accepted_cross_rank_dispatch_bytes": acc_loc["cross_rank_dispatch_bytes"],
        "accepted_cross_rank_roundtrip_bytes": acc_loc["cross_rank_roundtrip_bytes"],
        "accepted_local_hit_ratio": acc_loc["local_hit_ratio"],
        "pair_routes": pair,
        "f": aux["f"], "P": aux["P"], "l_aux": aux["l_aux"], "l_aux_norm": aux["l_aux_norm"],
        "load_var_over_mean": mon["var_over_mean"], "imbalanced": mon["imbalanced"],
    }


# ----------------------------------------------------------------------------
# the whole layer, two formulations
# ----------------------------------------------------------------------------
def moe_layer(x, w_gate, w1, b1, w2, b2, K: int, cf: float, logit_bias=None,
              h_round: Optional[str] = None, logits32=None) -> dict:
    """route -> capacity dispatch -> expert FFN -> combine, in the pages' order
    ([EPC] Router -> Dispatch -> Expert Compute -> Combine).

    `logits32` (optional) replaces the router product (shared-logits checks).
    """
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    E = np.asarray(w_gate).shape[0]
    if logits32 is None:
        logits32 = router_logits(x, w_gate)
    idx, gate = topk_softmax(logits32, K, logit_bias)
    cap = capacity(T * K, E, cf)
    sl = slot_routes(idx, E, cap)
    xd = dispatch(x, sl["row_token"])
    H, Y = expert_ffn(xd, sl["expert_offsets"], w1, b1, w2, b2, h_round)
    out = combine(Y, sl["route_row"], gate)
    return {"logits": logits32, "idx": idx, "gate": gate, "capacity": cap,
            "loads": expert_loads(idx, E), **sl, "xd": xd, "H": H, "Y": Y, "out": out}


def moe_layer_per_token(x, idx, gate, accepted_mask, w1, b1, w2, b2,
                        h_round: Optional[str] = None) -> np.ndarray:
    """Second formulation with no permutation ([DSV3] section 一):
    out[t] = sum over accepted k of g[t,k] * FFN_{idx[t,k]}(x[t]), computed
    token by token straight from x."""
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    h = np.asarray(w2).shape[1]
    out = np.zeros((T, h))
    for t in range(T):
        for k in range(idx.shape[1]):
            if not accepted_mask[t, k]:
                continue
            e = int(idx[t, k])
            u = np.asarray(w1[e], np.float64) @ x[t] + np.asarray(b1[e], np.float64)
            Hrow = _round_h(gelu_tanh(u), h_round)
            y = round_f32(np.asarray(w2[e], np.float64) @ Hrow + np.asarray(b2[e], np.float64))
            out[t] += float(gate[t, k]) * y
    return round_f32(out)


# ----------------------------------------------------------------------------
# aux-loss-free balancing: the expert-bias update
# ----------------------------------------------------------------------------
def top1_counts(adjusted_logits32: np.ndarray) -> np.ndarray:
    """count[e] = number of tokens whose largest adjusted logit is expert e
    ([DSV3] section 八, DeepSeekV3Gate: bincount of the argmax over experts of
    logits + expert_bias).  Equal logits: the lowest expert id, which is what
    an argmax that returns the first maximum gives (reading R2)."""
    a = np.asarray(adjusted_logits32, dtype=np.float64)
    T, E = a.shape
    counts = np.zeros(E, dtype=np.int64)
    for t in range(T):
        best = 0
        for e in range(1, E):
            if a[t, e] > a[t, best]:
                best = e
        counts[best] += 1
    return counts


def expert_bias_update(bias32, counts, alpha: float = 0.1) -> np.ndarray:
    """One step of [DSV3] section 八's bias rule,
        bias <- bias + alpha * (mean_count - count),
    with the page's fp32 tensors: mean_count = fp32(sum(count) / E), then per
    expert one fp32 subtraction, one fp32 product with fp32(alpha) and one
    fp32 addition, each rounded (no fused multiply-add).  Returns the new
    bias (fp32 values, as float64)."""
    b = np.asarray(bias32, dtype=np.float32)
    c = np.asarray(counts, dtype=np.float32)
    E = b.shape[0]
    mean = np.float32(np.float32(np.sum(np.asarray(counts, np.int64))) / np.float32(E))
    diff = (mean - c).astype(np.float32)
    step = (np.float32(alpha) * diff).astype(np.float32)
    return (b + step).astype(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# FP8 (OCP E4M3) dispatch payload
# ----------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_encode(v) -> np.ndarray:
    """Round each value to the nearest E4M3 (1 sign, 4 exponent bits with bias
    7, 3 mantissa bits; no infinities, code 0x7F/0xFF = NaN, largest finite
    448), ties to even, as the 'to(float8_e4m3fn)' conversion of [DSV3] 4.3
    does.  Magnitudes above 464 (past the midpoint to the next, missing,
    step) become NaN; below 2^-6 the spacing is 2^-9 (subnormals).
    Returns uint8 codes."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    a = np.abs(v)
    nan = np.isnan(a) | (a > 464.0)
    a = np.where(nan, 0.0, a)
    # a = f * 2^ex with f in [0.5, 1): the leading bit has weight 2^(ex-1)
    _, ex = np.frexp(a)
    lead = ex.astype(np.int64) - 1
    normal = a >= 2.0 ** -6
    # spacing: 2^(lead-3) for normals, 2^-9 below 2^-6; rint = ties to even
    step_exp = np.where(normal, lead - 3, -9)
    q = np.rint(np.ldexp(a, -step_exp)).astype(np.int64)
    # normals: q in [8, 16]; 16 carries into the next binade
    carry = normal & (q == 16)
    lead = np.where(carry, lead + 1, lead)
    q = np.where(carry, 8, q)
    code = np.where(normal, ((lead + 7) << 3) | (q - 8), q)  # subnormal q = 0..8
    code = np.where(nan, 0x7F, code)
    return (sign | code).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 code -> value (float64; NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


def fp8_scale(x_bf16) -> float:
    """Per-tensor scale of [DSV3] 4.3 on bf16 activations: amax = max |x|
    (a bf16 value), scale = bf16(amax / 448) (bf16 tensor arithmetic: the
    quotient is formed in fp32 and rounded to bf16)."""
    amax = float(np.max(np.abs(np.asarray(x_bf16, np.float64)))) if np.size(x_bf16) else 0.0
    return float(round_bf16(round_f32(amax / E4M3_MAX)))


def fp8_quantize(x_bf16, scale: float) -> np.ndarray:
    """codes = e4m3(bf16(x / scale)): the division in bf16 tensor arithmetic
    (fp32 quotient rounded to bf16), then the E4M3 rounding.  A zero scale
    (all-zero input) gives zero codes (reading: the page divides by it)."""
    x = np.asarray(x_bf16, np.float64)
    if scale == 0.0:
        return np.zeros(x.shape, np.uint8)
    return e4m3_encode(round_bf16(round_f32(x / scale)))


def fp8_dequantize(codes, scale: float) -> np.ndarray:
    """bf16(decode(code) * scale): the E4M3 value widened to bf16 (exact),
    times the bf16 scale, rounded to bf16 ([DSV3] 4.3 dequantisation)."""
    return round_bf16(round_f32(e4m3_decode(codes) * scale))


# ----------------------------------------------------------------------------
# the joint parallel-plan decision over the ledger
# ----------------------------------------------------------------------------
PLAN_THRESHOLDS = {"max_accept_balance": 1.2, "max_accept_cross_rank": 0.5,
                   "max_tune_overflow_ratio": 0.25, "max_tune_balance": 1.8,
                   "max_tune_cross_rank": 0.9}


def recommend_plan(summary: dict, locality: Optional[dict] = None, **thresholds) -> str:
    """[EP46] TODO 3 (joint decision): 'accept' when nothing overflows and
    both the load balance ratio and the cross-rank share of routes stay within
    the accept limits; 'tune' when the overflow share, the balance ratio and
    the cross-rank share all stay within the (looser) tune limits; 'reject'
    otherwise, and for an empty batch.  Without a locality summary the
    cross-rank share counts as 0.  Limits default to the page's values.

    The page's summary stores the balance ratio rounded to 3 decimals (its
    Step 4 reference summary), and the decision compares that stored value;
    `summarize_routes` returns it unrounded, so it is rounded here, with
    Python's round (ties to even on the exact binary value)."""
    th = dict(PLAN_THRESHOLDS, **thresholds)
    A = summary["total_routes"]
    if A == 0:
        return "reject"
    overflow_share = summary["overflow"] / A
    cross = 0.0
    if locality is not None and locality["total_routes"]:
        cross = locality["cross_rank_routes"] / locality["total_routes"]
    bal = round(summary["balance_ratio"], 3)
    if (summary["overflow"] == 0 and bal <= th["max_accept_balance"]
            and cross <= th["max_accept_cross_rank"]):
        return "accept"
    if (overflow_share <= th["max_tune_overflow_ratio"] and bal <= th["max_tune_balance"]
            and cross <= th["max_tune_cross_rank"]):
        return "tune"
    return "reject"


# ----------------------------------------------------------------------------
# locality-aware expert placement
# ----------------------------------------------------------------------------
def expert_rank_affinity(idx, src_rank, num_experts: int, n_ep: int, route_row=None):
    """affinity[e, r] = routes (t, k) with idx[t, k] == e whose token comes
    from rank r: the routes that stay local when expert e is placed on rank r
    ([EP46] TODO 2: a route is local iff the token's source rank owns its
    expert).  Over all routes, or over accepted routes (route_row >= 0) when
    `route_row` is given.  Integer counts."""
    idx = np.asarray(idx)
    T, K = idx.shape
    aff = np.zeros((num_experts, n_ep), np.int64)
    for t in range(T):
        r = int(src_rank[t])
        if not 0 <= r < n_ep:
            raise ValueError("source rank out of range")
        for k in range(K):
            if route_row is not None and route_row[t, k] < 0:
                continue
            e = int(idx[t, k])
            if not 0 <= e < num_experts:
                raise ValueError("expert id out of range")
            aff[e, r] += 1
    return aff


def local_routes_under(affinity, owner) -> int:
    """Local routes of a placement: sum_e affinity[e, owner[e]]."""
    aff = np.asarray(affinity)
    return int(sum(int(aff[e, int(owner[e])]) for e in range(aff.shape[0])))


def locality_placement(affinity, n_ep: int) -> np.ndarray:
    """Locality-aware expert -> rank map ([EP46] Step 3: a more local
    placement cuts cross-rank dispatch; [DSV3] 2.2: topology-aware placement
    matches experts to devices with the Hungarian algorithm on an affinity
    matrix).  Every rank hosts E / n_ep experts, as the uniform placement
    does, and the map maximises the local routes sum_e affinity[e, owner[e]].
    Solved as a linear assignment of experts to E slots (slot j belongs to
    rank j // (E / n_ep)) with a library assignment routine.  The optimum
    value is unique; when several maps reach it, any one is returned."""
    from scipy.optimize import linear_sum_assignment
    aff = np.asarray(affinity, dtype=np.int64)
    E = aff.shape[0]
    if n_ep <= 0 or E % n_ep != 0:
        raise ValueError("the experts must split evenly over the ranks")
    per = E // n_ep
    slot_rank = np.arange(E) // per
    gain = aff[:, slot_rank].astype(np.float64)          # [expert, slot]
    rows, cols = linear_sum_assignment(gain, maximize=True)
    owner = np.empty(E, np.int32)
    owner[rows] = slot_rank[cols]
    return owner


def rank_loads(idx, route_row, owner, n_ep: int) -> np.ndarray:
    """Accepted routes each rank's experts compute under a placement: the
    per-rank load whose longest member sets the slowest rank ([EP46] Step 3,
    routing skew row)."""
    idx = np.asarray(idx)
    route_row = np.asarray(route_row)
    loads = np.zeros(n_ep, np.int64)
    T, K = idx.shape
    for t in range(T):
        for k in range(K):
            if route_row[t, k] >= 0:
                loads[int(owner[int(idx[t, k])])] += 1
    return loads
